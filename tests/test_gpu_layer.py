"""Whole-layer and whole-stack runs of the HIP path against the oracle.

Both sides start from the same seeded inputs and run free: the GPU never
feeds the oracle.  Because the GPU's projections accumulate in fp32 in a
different order than the oracle's float64 products, about one bf16 rounding
in a thousand lands on the other side, which moves probe scores by ~1e-4
relative.  So at the chain level:
  * structure is checked exactly (sizes, forced probes, ascending order,
    nesting, skipped rows passing through bit-identically, score mass);
  * the index sets must satisfy the window rule with a 2e-3 window (the
    per-call tests hold the 1e-5 window on identical inputs);
  * outputs are compared, at the bf16 bar, on the rows where both sides took
    the same decisions.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layer as olayer, numerics, pap
from free_token_skipping_amd import capi, pipeline
from parity import np64, assert_close, window_violations, BF16_REL

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHAIN_WINDOW = 2e-3
WKEYS = ["wq", "wk", "wv", "wo", "wg", "wu", "wd", "u_t", "v_t"]


def _log(msg):
    print(msg, flush=True)


def _gpu_w(inp):
    return {k: inp[k].to(DEV) for k in WKEYS if k in inp}


def _f64_w(inp):
    return {k: W.as_f64(inp[k]) for k in WKEYS if k in inp}


def _mask(n, rows):
    m = np.zeros(n, bool)
    m[np.asarray(rows)] = True
    return m


def _check_selection(idx_gpu, k, P, n, s_oracle):
    idx = idx_gpu.cpu().numpy().astype(np.int64)
    assert len(idx) == k and np.all(np.diff(idx) > 0)
    assert np.isin(np.arange(n - P, n), idx).all()
    assert window_violations(s_oracle, idx, k, P, rel=CHAIN_WINDOW) == 0
    return idx


def test_attention_layer_8k_needles():
    """Attention-only layer, 8K tokens, 64 planted needles, keep 0.5."""
    cfgd = W.CONFIGS["attn_layer_8k"]
    sh = cfgd["shape"]
    _log("generate attention layer 8K")
    inp = W.make_layer(sh, seed=0, with_ffn=False, needles=cfgd["needles"])
    cfg = pipeline.LayerConfig(P=sh.P, keep_attn=cfgd["keep_attn"], keep_ffn=None)
    x0 = inp["x"].to(DEV)
    x = x0.clone()
    tr = {}
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), _gpu_w(inp), cfg, trace=tr)
    torch.cuda.synchronize()
    _log("oracle attention block 8K")
    ocfg = dict(Hq=32, Hkv=8, dh=128, P=sh.P, keep_attn=cfgd["keep_attn"])
    y_ref, st = olayer.attention_block(W.as_f64(inp["x"]), np.arange(sh.n), _f64_w(inp), ocfg)
    S = np64(tr["S"])
    assert abs(S.sum() - 32 * sh.P) < 1e-2 * 32 * sh.P
    assert_close(S, st["S"], 1e-2, "probe scores (chain)")
    k_a = numerics.keep_count(0.5, sh.n)
    idx = _check_selection(tr["idx"], k_a, sh.P, sh.n, st["S"])
    needles = inp["needle_pos"].numpy()
    assert np.isin(needles, idx).mean() >= 0.95           # sanity: needles are found
    got = np64(x)
    skipped = ~_mask(sh.n, idx)
    assert np.array_equal(got[skipped], W.as_f64(inp["x"])[skipped])
    same = _mask(sh.n, idx) & _mask(sh.n, st["idx"])
    assert_close(got[same], y_ref[same], BF16_REL, "attention layer rows")


def _layer_case(n, seed=0):
    sh = W.LayerShape(n=n, P=64)
    return sh, W.make_layer(sh, seed=seed)


@pytest.mark.parametrize("fused,fusion", [(True, "maxnorm_add"), (False, "maxnorm_add"), (True, "multiply")])
def test_layer_32k_recipe_at_4k(fused, fusion):
    """The 32K layer's recipe (attention + FFN, keep 0.35 / 0.35, MaxNorm-Add
    0.5/0.5 or Multiply fusion, rank-256 proxy) at 4096 tokens, where the
    oracle runs in seconds."""
    sh, inp = _layer_case(4096)
    cfg = pipeline.LayerConfig(P=64, keep_attn=0.35, keep_ffn=0.35, fusion=fusion)
    x = inp["x"].to(DEV).clone()
    tr = {}
    _log(f"gpu layer fused={fused} fusion={fusion}")
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), _gpu_w(inp), cfg, fused=fused,
                        trace=tr)
    torch.cuda.synchronize()
    _log("oracle layer 4K")
    ocfg = dict(Hq=32, Hkv=8, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, fusion=fusion)
    ref, st_a, st_f = olayer.spts_layer(W.as_f64(inp["x"]), np.arange(sh.n), _f64_w(inp), ocfg)
    k = numerics.keep_count(0.35, sh.n)
    idx = _check_selection(tr["idx"], k, 64, sh.n, st_a["S"])
    assert_close(np64(tr["L"]), st_f["L"], 1e-2, "LTP scores (chain)")
    idx_f = _check_selection(tr["idx_f"], k, 64, sh.n, st_f["fused"].astype(np.float64))
    got = np64(x)
    untouched = ~(_mask(sh.n, idx) | _mask(sh.n, idx_f))
    assert np.array_equal(got[untouched], W.as_f64(inp["x"])[untouched])
    same = (_mask(sh.n, idx) == _mask(sh.n, st_a["idx"])) & (_mask(sh.n, idx_f) == _mask(sh.n, st_f["idx_f"]))
    assert same.mean() > 0.98
    assert_close(got[same], ref[same], BF16_REL, "layer output rows")


def test_layer_4k_page_defaults():
    """The pages' default scoring: Multiply fusion and the structured proxy
    (512 channels, rank 256 per projection), on the 32K layer's recipe at
    4096 tokens."""
    sh, inp = _layer_case(4096)
    sp = W.structured_proxy(inp["wg"], inp["wu"], inp["wd"], 512, 256, seed=5)
    keys = ("a_g_t", "b_g_t", "a_u_t", "b_u_t", "c_t", "d_t")
    gw = _gpu_w(inp)
    gw["proxy_packed"] = capi.pack_structured_proxy(*[sp[k].to(DEV) for k in keys])
    cfg = pipeline.LayerConfig(P=64, keep_attn=0.35, keep_ffn=0.35, fusion="multiply", proxy="structured")
    x = inp["x"].to(DEV).clone()
    tr = {}
    _log("gpu layer, page defaults")
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), gw, cfg, trace=tr)
    torch.cuda.synchronize()
    ow = _f64_w(inp)
    ow.update({k: W.as_f64(sp[k]) for k in keys})
    ocfg = dict(Hq=32, Hkv=8, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, fusion="multiply", proxy="structured")
    _log("oracle layer 4K, page defaults")
    ref, st_a, st_f = olayer.spts_layer(W.as_f64(inp["x"]), np.arange(sh.n), ow, ocfg)
    k = numerics.keep_count(0.35, sh.n)
    idx = _check_selection(tr["idx"], k, 64, sh.n, st_a["S"])
    assert_close(np64(tr["L"]), st_f["L"], 1e-2, "structured LTP scores (chain)")
    idx_f = _check_selection(tr["idx_f"], k, 64, sh.n, st_f["fused"].astype(np.float64))
    got = np64(x)
    same = (_mask(sh.n, idx) == _mask(sh.n, st_a["idx"])) & (_mask(sh.n, idx_f) == _mask(sh.n, st_f["idx_f"]))
    assert same.mean() > 0.98
    assert_close(got[same], ref[same], BF16_REL, "layer output rows")


def test_layer_32k_full_size_structure_and_scores():
    """Full 32K layer on the GPU: exact structure, and the probe score and
    first selection against the oracle's own projections of the inputs."""
    sh, inp = _layer_case(32768)
    cfg = pipeline.LayerConfig(P=64, keep_attn=0.35, keep_ffn=0.35)
    x = inp["x"].to(DEV).clone()
    tr = {}
    _log("gpu layer 32K")
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), _gpu_w(inp), cfg, trace=tr)
    torch.cuda.synchronize()
    S = np64(tr["S"])
    assert abs(S.sum() - 32 * 64) < 0.5
    _log("oracle probe score 32K")
    x64 = W.as_f64(inp["x"])
    K = numerics.bf16(x64 @ W.as_f64(inp["wk"]).T).reshape(sh.n, 8, 128)
    Qp = numerics.bf16(x64[-64:] @ W.as_f64(inp["wq"]).T).reshape(64, 32, 128)
    S_ref = pap.pap_scores(Qp, K, 128 ** -0.5)
    assert_close(S, S_ref, 1e-2, "probe scores 32K (chain)")
    k = numerics.keep_count(0.35, sh.n)
    idx = _check_selection(tr["idx"], k, 64, sh.n, S_ref)
    idx_f = tr["idx_f"].cpu().numpy()
    assert len(idx_f) == k and np.all(np.diff(idx_f) > 0) and np.isin(np.arange(sh.n - 64, sh.n), idx_f).all()
    got = np64(x)
    assert np.isfinite(got).all()
    untouched = ~(_mask(sh.n, idx) | _mask(sh.n, idx_f))
    assert np.array_equal(got[untouched], x64[untouched])


def test_long_layer_prefix_16k():
    """The 128K workload's recipe (clustered keys + needles, P=128, keep 0.25)
    on a 16384-token prefix with its own last 128 probe rows."""
    sh = W.LayerShape(n=16384, P=128)
    _log("generate 16K prefix layer")
    inp = W.make_layer(sh, seed=0, needles=64, clustered_keys=(256, 0.3))
    cfg = pipeline.LayerConfig(P=128, keep_attn=0.25, keep_ffn=0.25)
    x = inp["x"].to(DEV).clone()
    tr = {}
    pipeline.spts_layer(x, torch.arange(sh.n, dtype=torch.int32, device=DEV), _gpu_w(inp), cfg,
                        k_given=inp["k"].to(DEV), trace=tr)
    torch.cuda.synchronize()
    _log("oracle 16K prefix layer")
    ocfg = dict(Hq=32, Hkv=8, dh=128, P=128, keep_attn=0.25, keep_ffn=0.25)
    ref, st_a, st_f = olayer.spts_layer(W.as_f64(inp["x"]), np.arange(sh.n), _f64_w(inp), ocfg,
                                        k_given=W.as_f64(inp["k"]))
    k = numerics.keep_count(0.25, sh.n)
    idx = _check_selection(tr["idx"], k, 128, sh.n, st_a["S"])
    idx_f = _check_selection(tr["idx_f"], k, 128, sh.n, st_f["fused"].astype(np.float64))
    assert np.isin(inp["needle_pos"].numpy(), idx).mean() >= 0.95
    got = np64(x)
    same = (_mask(sh.n, idx) == _mask(sh.n, st_a["idx"])) & (_mask(sh.n, idx_f) == _mask(sh.n, st_f["idx_f"]))
    assert same.mean() > 0.98
    assert_close(got[same], ref[same], BF16_REL, "16K prefix layer rows")


def test_long_layer_full_128k_score_path():
    """Full-length 128K probe -> score -> top-k from the projected probe
    queries and the clustered keys with 512 needles."""
    sh = W.LayerShape(n=131072, P=128)
    _log("generate 128K inputs")
    inp = W.make_layer(sh, seed=0, with_ffn=False, needles=512, clustered_keys=(256, 0.3))
    xp = inp["x"][-128:].to(DEV).contiguous()
    Qp = capi.spts_linear(xp, inp["wq"].to(DEV))
    S = capi.spts_probe_attention(Qp.view(128, 32, 128), inp["k"].to(DEV))
    k = numerics.keep_count(0.25, sh.n)
    idx = capi.spts_score_topk(S, k, 128)
    torch.cuda.synchronize()
    _log("oracle 128K score path")
    Qp_ref = numerics.bf16(W.as_f64(inp["x"][-128:]) @ W.as_f64(inp["wq"]).T).reshape(128, 32, 128)
    S_ref = pap.pap_scores(Qp_ref, W.as_f64(inp["k"]), 128 ** -0.5)
    assert_close(np64(S), S_ref, 1e-2, "probe scores 128K (chain)")
    idx = _check_selection(idx, k, 128, sh.n, S_ref)
    assert np.isin(inp["needle_pos"].numpy(), idx).mean() >= 0.95


def test_msdp_stack_small():
    """Pre-norm RoPE stack with MSDP on a reduced shape: GPU candidate sets
    nest exactly; they agree with the oracle's to the chain window."""
    sh = W.LayerShape(n=2048, d=512, Hq=8, Hkv=2, dh=128, f=1024, r=256, P=64)
    layers = 4
    st = W.make_stack(sh, layers, seed=0)
    budgets = [numerics.keep_count(r, sh.n) for r in (0.6, 0.35)]
    pts = pipeline.prune_points(0, (1, 3), budgets)
    cfg = pipeline.LayerConfig(Hq=8, Hkv=2, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, prenorm=True,
                               eps=1e-5, theta=500000.0)
    traces = []
    x0 = st["x"].to(DEV)
    x, pos = pipeline.msdp_stack(x0, [_gpu_w(w) for w in st["layers"]], cfg, pts, traces=traces)
    assert torch.equal(x0.cpu(), st["x"])                 # the stack never writes its input
    torch.cuda.synchronize()
    ocfg = dict(Hq=8, Hkv=2, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, prenorm=True, eps=1e-5,
                theta=500000.0)
    _log("oracle stack")
    ref, pos_ref, hist = olayer.msdp_stack(W.as_f64(st["x"]), [_f64_w(w) for w in st["layers"]], ocfg, pts)
    counts = olayer.candidate_counts(sh.n, layers, pts)
    # exact structure of the GPU's candidate sets
    prev = set(range(sh.n))
    for li, tr in enumerate(traces):
        cur = tr["pos"].cpu().numpy()
        assert len(cur) == counts[li] and np.all(np.diff(cur) > 0)
        assert set(cur.tolist()) <= prev
        assert set(range(sh.n - 64, sh.n)) <= set(cur.tolist())
        prev = set(cur.tolist())
    # first pruning decision against the oracle's score over all N
    assert window_violations(hist[0]["attn"]["S_full"], traces[0]["keep"].cpu().numpy(), budgets[0], 64,
                             rel=CHAIN_WINDOW) == 0
    final = pos.cpu().numpy()
    agree = len(np.intersect1d(final, pos_ref)) / len(pos_ref)
    assert agree > 0.95
    common, ig, io = np.intersect1d(final, pos_ref, return_indices=True)
    err = np.abs(np64(x)[ig] - ref[io]) / np.abs(ref[io]).max(axis=1, keepdims=True)
    assert np.median(err.max(axis=1)) <= BF16_REL



def test_dense_layers_and_schedule_small():
    """Dense prefill layers (every row computed) against the oracle's layer
    with every row kept, and the structure of a prefill schedule that runs
    dense layers before pruned SPTS layers."""
    sh = W.LayerShape(n=1024, d=512, Hq=8, Hkv=2, dh=128, f=1024, r=256, P=64)
    st = W.make_stack(sh, 2, seed=3)
    cfg = pipeline.LayerConfig(Hq=8, Hkv=2, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, prenorm=True,
                               eps=1e-5, theta=500000.0)
    ws = [_gpu_w(w) for w in st["layers"]]
    _log("dense prefill, 2 layers")
    x, pos = pipeline.prefill_schedule(st["x"].to(DEV), ws, cfg, n_layers=2, first_skip_layer=2, points={})
    torch.cuda.synchronize()
    ocfg = dict(Hq=8, Hkv=2, dh=128, P=64, keep_attn=1.0, keep_ffn=1.0, prenorm=True, eps=1e-5,
                theta=500000.0)
    ref = W.as_f64(st["x"])
    opos = np.arange(sh.n)
    for w in st["layers"]:
        ref, sa, sf = olayer.spts_layer(ref, opos, _f64_w(w), ocfg)
        assert len(sa["idx"]) == sh.n and len(sf["idx_f"]) == sh.n     # keep-all: the dense layer
    assert np.array_equal(pos.cpu().numpy(), opos)
    assert_close(np64(x), ref, BF16_REL, "dense prefill (2 layers)")
    _log("schedule: 2 dense + 4 SPTS layers, pruned at layers 2 and 4")
    pts = {2: 700, 4: 400}
    x2, pos2 = pipeline.prefill_schedule(st["x"].to(DEV), ws, cfg, n_layers=6, first_skip_layer=2, points=pts)
    torch.cuda.synchronize()
    p2 = pos2.cpu().numpy()
    assert x2.shape == (400, sh.d) and len(p2) == 400 and np.all(np.diff(p2) > 0)
    assert set(range(sh.n - 64, sh.n)) <= set(p2.tolist())
    assert torch.isfinite(x2.float()).all()


def test_msdp_stack_32k_full_size():
    """The timed workload itself: the 8-layer pre-norm RoPE stack at 32768
    tokens with the [SPTS] Sec. 3.3 stage schedule, in the configuration the
    benchmark runs.  Checked at full size:
      * structure that holds at any size: candidate counts per layer, nested
        ascending candidate sets that keep the probe rows, selection sizes,
        probe-score mass Hq*P, rows never selected passing through
        bit-identically;
      * the first pruning decision against the oracle's own probe score over
        all 32768 rows (window rule);
      * layer 0's attention output on sampled selected rows against the
        oracle's own projections, on rows before the first position where the
        two prune sets differ (causality makes those rows independent of it)."""
    from oracle.attention import reduced_attention
    from oracle.normrope import rmsnorm, rope
    from oracle.select import select_topk

    cfgd = W.CONFIGS["msdp_stack_32k"]
    sh = cfgd["shape"]
    N, P, Hq, Hkv, dh = sh.n, sh.P, sh.Hq, sh.Hkv, sh.dh
    _log("generate 32K stack inputs")
    st = W.make_stack(sh, cfgd["layers"], seed=cfgd["seed"])
    budgets = [numerics.keep_count(r, N) for r in cfgd["budget_ratios"]]
    pts = pipeline.prune_points(0, cfgd["stage_ends"], budgets)
    assert pts == olayer.prune_points(0, cfgd["stage_ends"], budgets)
    cfg = pipeline.LayerConfig(Hq=Hq, Hkv=Hkv, dh=dh, P=P, keep_attn=cfgd["keep_attn"], keep_ffn=cfgd["keep_ffn"],
                               w_fuse=cfgd["w_fuse"], prenorm=True, eps=cfgd["eps"], theta=cfgd["theta"])
    x0 = st["x"].to(DEV)
    traces = []
    _log("gpu 32K stack")
    x, pos = pipeline.msdp_stack(x0, [_gpu_w(w) for w in st["layers"]], cfg, pts, traces=traces)
    torch.cuda.synchronize()
    assert torch.equal(x0.cpu(), st["x"])                 # the stack never writes its input

    # ---- structure of every layer
    counts = olayer.candidate_counts(N, cfgd["layers"], pts)
    prev = np.arange(N)
    selected_pos = set()
    for li, tr in enumerate(traces):
        cur = tr["pos"].cpu().numpy().astype(np.int64)
        n = len(cur)
        assert n == counts[li] and np.all(np.diff(cur) > 0), li
        assert np.isin(cur, prev).all() and np.isin(np.arange(N - P, N), cur).all(), li
        assert abs(float(tr["S_pre"].double().sum()) - Hq * P) < 0.5, li
        k = numerics.keep_count(cfgd["keep_attn"], n)
        for name in ("idx", "idx_f"):
            sel = tr[name].cpu().numpy().astype(np.int64)
            assert len(sel) == k and np.all(np.diff(sel) > 0), (li, name)
            assert np.isin(np.arange(n - P, n), sel).all(), (li, name)
            selected_pos.update(cur[sel].tolist())
        prev = cur
    final = pos.cpu().numpy().astype(np.int64)
    assert np.array_equal(final, prev)
    got = np64(x)
    assert np.isfinite(got).all()
    x0_64 = W.as_f64(st["x"])
    untouched = ~np.isin(final, np.fromiter(selected_pos, dtype=np.int64))
    _log(f"final candidates never selected by any layer: {int(untouched.sum())}")
    assert np.array_equal(got[untouched], x0_64[final[untouched]])

    # ---- layer 0 against the oracle's own projections
    _log("oracle layer-0 projections at 32K")
    w0 = st["layers"][0]
    theta, scale = cfgd["theta"], dh ** -0.5
    xt = numerics.bf16(rmsnorm(x0_64, cfgd["eps"]))
    allpos = np.arange(N)

    def proj(rows, wname, heads, rope_pos):
        acc = numerics.f32(xt[rows] @ W.as_f64(w0[wname]).T).reshape(len(rows), heads, dh)
        return numerics.bf16(rope(acc, rope_pos, theta) if rope_pos is not None else acc)

    K = proj(allpos, "wk", Hkv, allpos)
    V = proj(allpos, "wv", Hkv, None)
    Qp = proj(allpos[-P:], "wq", Hq, allpos[-P:])
    S_ref = pap.pap_scores(Qp, K, scale)
    tr0 = traces[0]
    assert_close(np64(tr0["S_pre"]), S_ref, 1e-2, "layer-0 probe score over 32K (chain)")
    keep_gpu = tr0["keep"].cpu().numpy().astype(np.int64)
    assert window_violations(S_ref, keep_gpu, budgets[0], P, rel=CHAIN_WINDOW) == 0
    keep_ref = select_topk(numerics.f32(S_ref), budgets[0], P)
    differ = np.setxor1d(keep_gpu, keep_ref)
    first_diff = int(differ.min()) if len(differ) else N
    idx_ref = select_topk(numerics.f32(S_ref[keep_ref]), numerics.keep_count(cfgd["keep_attn"], budgets[0]), P)
    idx_gpu = tr0["idx"].cpu().numpy().astype(np.int64)
    rows_ref = keep_ref[idx_ref]                      # original positions of the oracle's queries
    rows_gpu = keep_gpu[idx_gpu]
    common = np.intersect1d(rows_ref[rows_ref < first_diff], rows_gpu)
    assert len(common) >= 64
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(common, size=32, replace=False))
    loc_ref = np.searchsorted(keep_ref, sample)       # query rows within the oracle's candidate set
    Qs = proj(sample, "wq", Hq, sample)
    O_ref = numerics.bf16(reduced_attention(Qs, loc_ref, K[keep_ref], V[keep_ref], scale))
    O_gpu = np64(tr0["O"]).reshape(-1, Hq, dh)[np.searchsorted(rows_gpu, sample)]
    assert_close(O_gpu, O_ref, BF16_REL, "layer-0 attention output, sampled rows at 32K")
