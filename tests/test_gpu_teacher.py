"""Teacher-forced parity at the workloads' full sizes.

Every layer the benchmark times is run on the GPU with a trace, and each of
its steps is checked against the oracle on the GPU's own inputs to that step
(tests/teacher.py): selections at the 1e-5 window, scores at the fp32 bar,
outputs at the bf16 bar by their maximum error on sampled rows, skipped rows
bit-identical.  The free-running comparisons (both sides from the same seeded
inputs only) are in test_gpu_layer.py.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layer as olayer, numerics, pap
from free_token_skipping_amd import capi, pipeline
from parity import np64, max_rel_err, window_violations, F32_REL
from teacher import check_layer, check_dense_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
WKEYS = ["wq", "wk", "wv", "wo", "wg", "wu", "wd", "u_t", "v_t"]


def _log(msg):
    print(msg, flush=True)


def _gpu_w(inp):
    return {k: inp[k].to(DEV) for k in WKEYS if k in inp}


def _cpu_w(inp):
    return {k: inp[k] for k in WKEYS if k in inp}


@pytest.mark.timeout(900)
def test_layer_32k_teacher_forced():
    """The 32K attention + FFN layer (PAP + LTP, keep 0.35 / 0.35, MaxNorm-Add
    0.5/0.5), every step at full size."""
    cfgd = W.CONFIGS["layer_32k"]
    sh = cfgd["shape"]
    _log("generate 32K layer")
    inp = W.make_layer(sh, seed=cfgd["seed"])
    cfg = pipeline.LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"],
                               keep_ffn=cfgd["keep_ffn"], w_fuse=cfgd["w_fuse"])
    x = inp["x"].to(DEV).clone()
    tr = {}
    _log("gpu 32K layer")
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), _gpu_w(inp), cfg, trace=tr)
    torch.cuda.synchronize()
    assert torch.equal(tr["x_in"].cpu(), inp["x"])
    _log("teacher-forced oracle steps, 32K layer")
    ocfg = dict(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"], keep_ffn=cfgd["keep_ffn"],
                w_fuse=cfgd["w_fuse"])
    check_layer(tr, _cpu_w(inp), ocfg, log=_log)


@pytest.mark.timeout(1200)
def test_msdp_stack_32k_teacher_forced():
    """The 8-layer pre-norm RoPE MSDP stack at 32768 tokens as the benchmark
    runs it (stages of two layers, budgets 0.6 / 0.45 / 0.35 / 0.25 of N):
    structure at any size (nesting, forcing, counts, rows never selected
    passing through bit-identically) and every layer teacher-forced."""
    cfgd = W.CONFIGS["msdp_stack_32k"]
    sh = cfgd["shape"]
    N, P, Hq = sh.n, sh.P, sh.Hq
    _log("generate 32K stack inputs")
    st = W.make_stack(sh, cfgd["layers"], seed=cfgd["seed"])
    budgets = [numerics.keep_count(r, N) for r in cfgd["budget_ratios"]]
    pts = pipeline.prune_points(0, cfgd["stage_ends"], budgets)
    assert pts == olayer.prune_points(0, cfgd["stage_ends"], budgets)
    cfg = pipeline.LayerConfig(Hq=Hq, Hkv=sh.Hkv, dh=sh.dh, P=P, keep_attn=cfgd["keep_attn"],
                               keep_ffn=cfgd["keep_ffn"], w_fuse=cfgd["w_fuse"], prenorm=True, eps=cfgd["eps"],
                               theta=cfgd["theta"])
    x0 = st["x"].to(DEV)
    traces = []
    _log("gpu 32K stack with traces")
    x, pos = pipeline.msdp_stack(x0, [_gpu_w(w) for w in st["layers"]], cfg, pts, traces=traces)
    torch.cuda.synchronize()
    assert torch.equal(x0.cpu(), st["x"])                 # the stack never writes its input

    # structure of every layer
    counts = olayer.candidate_counts(N, cfgd["layers"], pts)
    prev = np.arange(N)
    selected = set()
    for li, tr in enumerate(traces):
        cur = tr["pos"].cpu().numpy().astype(np.int64)
        assert len(cur) == counts[li] and np.all(np.diff(cur) > 0), li
        assert np.isin(cur, prev).all() and np.isin(np.arange(N - P, N), cur).all(), li
        for name in ("idx", "idx_f"):
            selected.update(cur[tr[name].cpu().numpy().astype(np.int64)].tolist())
        if li + 1 < len(traces):                          # the next layer starts from this one's output
            assert torch.equal(traces[li + 1]["x_in"], tr["x_out"])
        prev = cur
    final = pos.cpu().numpy().astype(np.int64)
    assert np.array_equal(final, prev)
    got = np64(x)
    untouched = ~np.isin(final, np.fromiter(selected, dtype=np.int64))
    _log(f"final candidates never selected by any layer: {int(untouched.sum())}")
    assert np.array_equal(got[untouched], W.as_f64(st["x"])[final[untouched]])

    ocfg = dict(Hq=Hq, Hkv=sh.Hkv, dh=sh.dh, P=P, keep_attn=cfgd["keep_attn"], keep_ffn=cfgd["keep_ffn"],
                w_fuse=cfgd["w_fuse"], prenorm=True, eps=cfgd["eps"], theta=cfgd["theta"])
    for li, tr in enumerate(traces):
        _log(f"teacher-forced oracle steps, stack layer {li} ({len(tr['pos'])} candidates)")
        budget = pts.get(li)
        check_layer(tr, _cpu_w(st["layers"][li]), ocfg, prune_to=budget, seed=li, log=_log)
        for k in list(tr):                                # free this layer's GPU copies
            tr[k] = None
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_long_layer_128k_teacher_forced():
    """The 128K layer at full length: clustered keys with 512 needles, 128
    probes, keep 0.25 / 0.25; every step teacher-forced, plus needle recall."""
    cfgd = W.CONFIGS["long_layer_128k"]
    sh = cfgd["shape"]
    _log("generate 128K layer")
    inp = W.make_layer(sh, seed=cfgd["seed"], needles=cfgd["needles"],
                       clustered_keys=(cfgd["centroids"], cfgd["sigma"]))
    cfg = pipeline.LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"],
                               keep_ffn=cfgd["keep_ffn"], w_fuse=cfgd["w_fuse"])
    x = inp["x"].to(DEV).clone()
    tr = {}
    _log("gpu 128K layer")
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), _gpu_w(inp), cfg,
                        k_given=inp["k"].to(DEV), trace=tr)
    torch.cuda.synchronize()
    idx = tr["idx"].cpu().numpy()
    assert np.isin(inp["needle_pos"].numpy(), idx).mean() >= 0.95      # sanity: needles are found
    _log("teacher-forced oracle steps, 128K layer")
    ocfg = dict(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"], keep_ffn=cfgd["keep_ffn"],
                w_fuse=cfgd["w_fuse"])
    check_layer(tr, _cpu_w(inp), ocfg, k_given=True, log=_log)


@pytest.mark.timeout(600)
def test_attention_layer_8k_teacher_forced():
    """The 8K attention-only layer with 64 needles, keep 0.5."""
    cfgd = W.CONFIGS["attn_layer_8k"]
    sh = cfgd["shape"]
    inp = W.make_layer(sh, seed=cfgd["seed"], with_ffn=False, needles=cfgd["needles"])
    cfg = pipeline.LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"], keep_ffn=None)
    x = inp["x"].to(DEV).clone()
    tr = {}
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), _gpu_w(inp), cfg, trace=tr)
    torch.cuda.synchronize()
    ocfg = dict(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"], keep_ffn=None)
    _log("teacher-forced oracle steps, 8K attention layer")
    check_layer(tr, _cpu_w(inp), ocfg, log=_log)


@pytest.mark.timeout(600)
def test_score_path_128k_teacher_forced():
    """Full-length 128K probe -> score -> top-k on the GPU's projected probe
    queries and the clustered keys: fp32 bar and the 1e-5 window."""
    cfgd = W.CONFIGS["long_layer_128k"]
    sh = cfgd["shape"]
    inp = W.make_layer(sh, seed=cfgd["seed"], with_ffn=False, needles=cfgd["needles"],
                       clustered_keys=(cfgd["centroids"], cfgd["sigma"]))
    Qp = capi.spts_linear(inp["x"][-sh.P:].to(DEV).contiguous(), inp["wq"].to(DEV))
    K = inp["k"].to(DEV)
    S = capi.spts_probe_attention(Qp.view(sh.P, sh.Hq, sh.dh), K)
    k = numerics.keep_count(cfgd["keep_attn"], sh.n)
    idx = capi.spts_score_topk(S, k, sh.P)
    torch.cuda.synchronize()
    _log("oracle score over 131072 keys")
    S_ref = pap.pap_scores(np64(Qp).reshape(sh.P, sh.Hq, sh.dh), W.as_f64(inp["k"]), sh.dh ** -0.5)
    err = max_rel_err(np64(S), S_ref)
    assert err <= F32_REL, err
    assert window_violations(S_ref, idx.cpu().numpy(), k, sh.P) == 0


@pytest.mark.timeout(600)
def test_prefill_schedule_teacher_forced():
    """A Table B style prefill schedule on a reduced shape: dense layers, then
    SPTS layers pruned at stage starts.  Each dense layer against the oracle's
    keep-all layer and each SPTS layer step by step, on the GPU's own layer
    inputs ([SPTS] Table B, Table 4)."""
    sh = W.LayerShape(n=2048, d=512, Hq=8, Hkv=2, dh=128, f=1024, r=256, P=64)
    st = W.make_stack(sh, 3, seed=4)
    cfg = pipeline.LayerConfig(Hq=8, Hkv=2, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, prenorm=True,
                               eps=1e-5, theta=500000.0)
    ws = [_gpu_w(w) for w in st["layers"]]
    pts = pipeline.prune_points(2, (3, 5), (1229, 700), final_budget=400)
    traces = []
    _log("schedule: 2 dense + 5 SPTS layers")
    x, pos = pipeline.prefill_schedule(st["x"].to(DEV), ws, cfg, n_layers=7, first_skip_layer=2, points=pts,
                                       traces=traces)
    torch.cuda.synchronize()
    assert x.shape[0] == 400 and np.all(np.diff(pos.cpu().numpy()) > 0)
    ocfg = dict(Hq=8, Hkv=2, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, prenorm=True, eps=1e-5, theta=500000.0)
    for li, tr in enumerate(traces):
        w = _cpu_w(st["layers"][li % 3])
        if tr.get("dense"):
            _log(f"dense layer {li}")
            check_dense_layer(tr, w, ocfg, seed=li, log=_log)
        else:
            _log(f"SPTS layer {li}, {len(tr['pos'])} candidates")
            budget = pts.get(li)
            check_layer(tr, w, ocfg, prune_to=budget, seed=li, log=_log)
        if li + 1 < len(traces):
            assert torch.equal(traces[li + 1]["x_in"], tr["x_out"])
