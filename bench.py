#!/usr/bin/env python3
"""SPTS prefill benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input
(inputs resident in HBM before timing starts):

  msdp_stack_32k (default): the 8-layer LLaMA-3.1-8B-shaped stack at 32768
      tokens -- RMSNorm, K/V/probe-Q projections with RoPE, PAP probe, MSDP
      stage pruning (budgets 0.6/0.45/0.35/0.25 of N every 2 layers), top-k,
      reduced attention, O projection + residual, LTP probe, fused top-k,
      reduced SwiGLU + residual -- every row of the hot path.
  layer_32k: one bare attention + FFN layer at 32768 tokens (PAP + LTP).

The metric is prefill tokens/s per layer: layers * N / seconds per step.
One JSON line is printed.  It also carries the roofline of the dominant
kernel (timed with HIP events on its own stream inside the timed region,
where no other call carries events), a per-call breakdown (from K steps with
every call bracketed, run before the timed ones), the single-layer figure and
the CPU oracle's rate on a bounded row sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_CALLS = {"kv_proj", "k_proj", "v_proj", "probe_q_proj", "q_proj", "reduced_attention", "o_proj_add",
              "ffn_gate_up", "ffn_down_add", "ltp_probe", "pap_probe", "o_proj", "reduced_ffn"}
SINGLE_KERNEL_CALLS = {"kv_proj", "k_proj", "v_proj", "probe_q_proj", "q_proj", "reduced_attention", "o_proj_add",
                       "ffn_gate_up", "ffn_down_add"}
KERNEL_OF_CALL = {"reduced_attention": "attn_bf16_kernel", "ffn_gate_up": "gemm_tn_kernel<EPI_SWIGLU,gather>",
                  "ffn_down_add": "gemm_tn_kernel<EPI_STORE,scatter>", "q_proj": "gemm_tn_kernel<EPI_ROPE/STORE,gather>",
                  "o_proj_add": "gemm_tn_kernel<EPI_STORE,scatter>", "k_proj": "gemm_tn_kernel",
                  "v_proj": "gemm_tn_kernel", "kv_proj": "gemm_tn_kernel<EPI_KV>"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="msdp_stack_32k", choices=["msdp_stack_32k", "layer_32k"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single-layer", action="store_true")
    ap.add_argument("--no-ttft", action="store_true", help="skip the 32-layer prefill schedule vs dense table")
    ap.add_argument("--no-hbm", action="store_true", help="skip the cold/warm gather and scatter-add table")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode / end-to-end table")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the 8K attention layer and the 128K score path / 16K prefix layer")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode table (prefill + decode at 32K), printed as one JSON line")
    ap.add_argument("--unfused", action="store_true", help="standalone gather/scatter kernels")
    ap.add_argument("--cpu-sample", type=float, default=1.0 / 32,
                    help="fraction of row-separable oracle work timed for the CPU baseline")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle's whole 32K layer unsampled (several minutes)")
    ap.add_argument("--probe-only", action="store_true",
                    help="only run the PAP probe on the 32K-stack shape (64 probes, 32768 keys) and the 128K shape "
                         "(128 probes, 131072 keys), 20 calls each, printing per-call times (for kernel profiles)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run spts_gather over 1 GiB with identity rows (a plain copy of known size, "
                         "to scale HBM byte counters) and exit")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------- inputs

def stack_inputs(dev, n_layers=8):
    import workloads as W
    cfgd = W.CONFIGS["msdp_stack_32k"]
    sh = cfgd["shape"]
    t0 = time.time()
    st = W.make_stack(sh, n_layers, seed=cfgd["seed"])
    keys = ["wq", "wk", "wv", "wo", "wg", "wu", "wd", "u_t", "v_t"]
    layers = [{k: w[k].to(dev) for k in keys} for w in st["layers"]]
    log(f"generated stack inputs in {time.time() - t0:.1f}s")
    return cfgd, sh, st, st["x"].to(dev), layers


# ------------------------------------------------------------------ timing

def dominant_call(summary):
    """The single-kernel call with the most time in a per-call summary."""
    cands = [(ms, name) for name, (calls, ms, work) in summary.items() if name in SINGLE_KERNEL_CALLS]
    return max(cands)[1] if cands else None


def timed(run_step, steps, warmup):
    """W untimed warm-up steps; K steps with every library call bracketed by
    events (the per-call breakdown, not timed as a whole); then the K timed
    steps, in which only the breakdown's dominant call carries events (its
    roofline), so the step time holds next to no instrumentation.
    Returns (timed ms, wall ms, breakdown summary, dominant-call summary)."""
    import torch
    from free_token_skipping_amd.pipeline import CallTimer, NO_TIMER
    for _ in range(warmup):
        run_step(NO_TIMER)
    torch.cuda.synchronize()
    full = CallTimer()
    for _ in range(steps):
        run_step(full)
    torch.cuda.synchronize()
    summ_full = full.summary()
    dom = dominant_call(summ_full)
    tm = CallTimer(only={dom}) if dom else NO_TIMER
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run_step(tm)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    return e0.elapsed_time(e1), wall_ms, summ_full, (tm.summary() if dom else {})


def breakdown(summary, steps):
    out = {}
    for name, (calls, ms, work) in sorted(summary.items(), key=lambda kv: -kv[1][1]):
        row = {"ms_per_step": round(ms / steps, 4), "calls_per_step": calls // steps}
        if ms > 0 and work:
            rate = work / (ms * 1e-3)
            if name in MFMA_CALLS:
                row["tflops"] = round(rate / 1e12, 1)
                row["frac_mfma_peak"] = round(rate / 1e12 / PEAK_BF16_TFLOPS, 4)
            else:
                row["gbs"] = round(rate / 1e9, 1)
                row["frac_hbm_peak"] = round(rate / 1e9 / PEAK_HBM_GBS, 4)
        out[name] = row
    return out


def measured_traffic(call):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary, if that summary was taken on the
    current kernel source (else None)."""
    import hashlib
    import re
    if call != "ffn_gate_up":
        return None
    path = os.path.join(ROOT, "profiles", "ffn_gate_up_gemm_traffic.md")
    src = os.path.join(ROOT, "free_token_skipping_amd", "csrc", "gemm.hip")
    try:
        text = open(path).read()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    m_sha = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text)
    m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    if not m_sha or not m_tr or m_sha.group(1) != sha:
        return None
    return float(m_tr.group(1))


# rocprofv3 kernel names behind a call (main kernel, tail fixup launch), as the
# committed kernel summary of the 8-layer stack lists them
ROCPROF_KERNELS = {"ffn_gate_up": ("gemm_tn_kernel<2, true>", "gemm_tail_fixup_kernel<2, true>"),
                   "reduced_attention": ("attn_bf16_kernel", None),
                   "kv_proj": ("gemm_tn_kernel<6, false>", "gemm_tail_fixup_kernel<6, false>")}
STACK_PROFILE = os.path.join(ROOT, "profiles", "msdp_stack_32k_kernel_stats.md")


def rocprof_per_call(call):
    """Average time per call of `call` from the committed rocprofv3 summary of
    the stack (main kernel plus its tail fixup launches, over the main
    kernel's launch count), or None."""
    import re
    names = ROCPROF_KERNELS.get(call)
    if not names:
        return None
    try:
        text = open(STACK_PROFILE).read()
    except OSError:
        return None
    rows = {}
    for m in re.finditer(r"^\|\s*([^|]+?)\s*\|\s*(\d+)\s*\|\s*([0-9.]+)\s*\|", text, re.M):
        rows[m.group(1)] = (int(m.group(2)), float(m.group(3)))
    main, fix = names
    if main not in rows:
        return None
    calls, total = rows[main]
    if fix and fix in rows:
        total += rows[fix][1]
    return {"avg_call_ms": round(total / calls, 4), "launches": calls,
            "source": "profiles/msdp_stack_32k_kernel_stats.md"}


def roofline(summary, steps, with_rocprof=False):
    """Dominant single-kernel call by time: achieved = algorithmic FLOPs per
    launch / average launch time (events on the launching stream).  With
    with_rocprof, the same figure from the committed rocprofv3 kernel summary
    of the stack is given beside it."""
    cands = [(ms, name, calls, work) for name, (calls, ms, work) in summary.items() if name in SINGLE_KERNEL_CALLS]
    ms, name, calls, work = max(cands)
    avg_ms = ms / calls
    flops_per_launch = work / calls
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    out = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
           "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(name),
           "kernel": KERNEL_OF_CALL.get(name, name), "call": name,
           "flops_per_launch": flops_per_launch, "avg_launch_ms": round(avg_ms, 4),
           "launches_per_step": calls // steps}
    if with_rocprof:
        rp = rocprof_per_call(name)
        if rp:
            a = flops_per_launch / (rp["avg_call_ms"] * 1e-3) / 1e12
            rp.update(achieved=round(a, 1), frac=round(a / PEAK_BF16_TFLOPS, 4))
        out["rocprof"] = rp
    return out


# ------------------------------------------------- 32-layer prefill schedule

# The LLaMA-3.1-8B schedule of [SPTS] Table B: 32 layers, layers 0-9 dense,
# stages ending at layers 13/18/23/28 with 9K/7K/4K/2K candidates, 1K after
# the last stage (K = 1024 tokens).
LLAMA_SCHEDULE = dict(n_layers=32, first_skip_layer=10, stage_ends=(13, 18, 23, 28),
                      budgets=(9216, 7168, 4096, 2048), final_budget=1024)


def ttft_table(x0, layers, cfg, reps=2):
    """Prefill time of the 32-layer schedule against the same 32 layers run
    dense, at 8K-32K tokens: a speed-only analogue of [SPTS] Table 4 (TTFT
    ratio vs the full model).  Both sides use this library's kernels; the
    32 layers cycle through the generated layers' weights (the work does not
    depend on the weight values)."""
    import torch
    from free_token_skipping_amd import pipeline
    sch = LLAMA_SCHEDULE
    pts = pipeline.prune_points(sch["first_skip_layer"], sch["stage_ends"], sch["budgets"], sch["final_budget"])
    rows = []
    for n in (8192, 16384, 24576, 32768):
        xs = x0[:n]
        ms = {}
        for mode in ("dense", "spts"):
            def run():
                pipeline.prefill_schedule(xs, layers, cfg, sch["n_layers"], sch["first_skip_layer"], pts,
                                          dense=(mode == "dense"))
            run()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            ms[mode] = e0.elapsed_time(e1) / reps
        rows.append({"tokens": n, "dense_ms": round(ms["dense"], 2), "spts_ms": round(ms["spts"], 2),
                     "ttft_ratio": round(ms["dense"] / ms["spts"], 3)})
        log(f"prefill {n}: dense {ms['dense']:.1f} ms, SPTS {ms['spts']:.1f} ms, ratio {ms['dense'] / ms['spts']:.2f}x")
    return {"schedule": "32 layers, dense 0-9, stage ends 13/18/23/28, candidates 9216/7168/4096/2048, "
                        "1024 after; keep 0.35 per skipping layer",
            "weights": f"{len(layers)} generated layers cycled", "reps": reps, "rows": rows}


def decode_table(x0, layers, cfg, tokens=16, gen=(32, 128, 512)):
    """Decode after the 32-layer prefill at 32K tokens: per-token latency with
    each layer's cache holding its candidates (SPTS, [SPTS] Table 5) against
    full caches (dense prefill), and end-to-end time for G generated tokens
    = prefill + G * per-token time (a speed-only analogue of the pages'
    end-to-end comparison).  A step is one spts_decode_step call (all 32
    layers); the per-call composition is timed beside it.  HBM rate: the
    algorithmic bytes of a token (every weight byte once, every cached K and
    V row once) over its time."""
    import torch
    from free_token_skipping_amd import capi, pipeline
    sch = LLAMA_SCHEDULE
    pts = pipeline.prune_points(sch["first_skip_layer"], sch["stage_ends"], sch["budgets"], sch["final_budget"])
    n = x0.shape[0]
    nl = sch["n_layers"]
    table = capi.spts_rope_table(n + 3 * tokens + 2, cfg.dh, cfg.theta, x0.device)
    wbytes = sum(layers[l % len(layers)][k].numel() * 2 for l in range(nl)
                 for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"))
    out = {}

    def clock(fn, count):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record()
        for t in range(count):
            fn(t)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / count, (time.perf_counter() - w0) * 1e3 / count

    for mode in ("dense", "spts"):
        kvs = []
        prefill_ms, _ = clock(lambda t: pipeline.prefill_schedule(
            x0, layers, cfg, nl, sch["first_skip_layer"], pts, dense=(mode == "dense"), kv_out=kvs), 1)
        caches = pipeline.DecodeCaches(kvs, 3 * tokens + 2)
        del kvs
        x = x0[n - 1].clone()
        pipeline.decode_step_native(x, n, layers, caches, cfg, table)                # warm-up token
        len0 = list(caches.lengths)
        tok_ms, wall = clock(lambda t: pipeline.decode_step_native(x, n + 1 + t, layers, caches, cfg, table), tokens)
        cache_read = sum(2 * (l0 + t + 1) * cfg.Hkv * cfg.dh * 2 for l0 in len0 for t in range(tokens)) / tokens
        per_call_ms, _ = clock(lambda t: pipeline.decode_step(x, n + 1 + tokens + t, layers, caches, cfg, table),
                               tokens)
        gbs = (wbytes + cache_read) / (tok_ms * 1e-3) / 1e9
        out[mode] = {"prefill_ms": round(prefill_ms, 2), "ms_per_token": round(tok_ms, 4),
                     "wall_ms_per_token": round(wall, 4), "per_call_ms_per_token": round(per_call_ms, 4),
                     "bytes_per_token": int(wbytes + cache_read), "hbm_gb_per_s": round(gbs, 1),
                     "hbm_frac": round(gbs / 8000.0, 4),
                     "cache_rows_first_last_layer": [len0[0], len0[-1]],
                     "cache_gib": round(caches.nbytes() / 2 ** 30, 3)}
        log(f"decode {mode}: prefill {prefill_ms:.1f} ms, {tok_ms:.3f} ms/token (wall {wall:.3f}, per-call "
            f"composition {per_call_ms:.3f}), {gbs:,.0f} GB/s, cache {caches.nbytes() / 2 ** 30:.2f} GiB")
        del caches
    e2e = []
    for g in gen:
        dm = out["dense"]["prefill_ms"] + g * out["dense"]["ms_per_token"]
        sm = out["spts"]["prefill_ms"] + g * out["spts"]["ms_per_token"]
        e2e.append({"generated": g, "dense_ms": round(dm, 1), "spts_ms": round(sm, 1), "ratio": round(dm / sm, 3)})
    out["tokens_timed"] = tokens
    out["prompt_tokens"] = n
    out["weights"] = f"{len(layers)} generated layers cycled over {nl}; {wbytes / 1e9:.2f} GB read per token"
    out["end_to_end"] = e2e
    return out


def other_workloads(dev, steps, warmup):
    """The remaining workloads, each timed like the headline (warm-up, then
    steps bracketed by events, per-call breakdown):
      attn_layer_8k     attention-only layer, 8192 tokens, 64 needles, P 64, keep 0.5
      long_128k_score   probe queries -> PAP score -> top-k at 131072 tokens (clustered
                        keys, 512 needles, P 128, keep 0.25)
      long_layer_128k   the whole 131072-token layer (attention + FFN, keep 0.25 / 0.25)
      long_16k_prefix   the 128K recipe as a full layer on a 16384-token prefix"""
    import torch
    import workloads as W
    from free_token_skipping_amd import capi, pipeline
    from free_token_skipping_amd.pipeline import LayerConfig, keep_count
    keys = ["wq", "wk", "wv", "wo", "wg", "wu", "wd", "u_t", "v_t"]
    out = {}

    def record(name, fn, tokens, extra):
        total_ms, _, summ, summ_dom = timed(fn, steps, warmup)
        ms = total_ms / steps
        out[name] = dict(extra, ms_per_step=round(ms, 4), tokens_per_s=round(tokens / (ms * 1e-3), 1),
                         breakdown=breakdown(summ, steps))
        if summ_dom and "layer" in name:
            out[name]["roofline"] = roofline(summ_dom, steps)
        log(f"{name}: {ms:.3f} ms/step, {tokens / (ms * 1e-3):,.0f} tokens/s")

    cfg8k = W.CONFIGS["attn_layer_8k"]
    sh = cfg8k["shape"]
    inp = W.make_layer(sh, seed=cfg8k["seed"], with_ffn=False, needles=cfg8k["needles"])
    w = {k: inp[k].to(dev) for k in ("wq", "wk", "wv", "wo")}
    x0 = inp["x"].to(dev)
    pos = torch.arange(sh.n, dtype=torch.int32, device=dev)
    cfg = LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfg8k["keep_attn"], keep_ffn=None)

    def step8k(tm):
        x = x0.clone()
        pipeline.spts_layer(x, pos, w, cfg, tm=tm)
    record("attn_layer_8k", step8k, sh.n, {"tokens": sh.n, "keep_attn": cfg8k["keep_attn"], "probes": sh.P,
                                           "needles": cfg8k["needles"]})
    del inp, w, x0

    cfg128k = W.CONFIGS["long_layer_128k"]
    sh = cfg128k["shape"]
    inp = W.make_layer(sh, seed=cfg128k["seed"], needles=cfg128k["needles"],
                       clustered_keys=(cfg128k["centroids"], cfg128k["sigma"]))
    xp = inp["x"][-sh.P:].to(dev).contiguous()
    wq = inp["wq"].to(dev)
    kk = inp["k"].to(dev)
    k = keep_count(cfg128k["keep_attn"], sh.n)

    def score128k(tm):
        with tm("probe_q_proj", 2.0 * sh.P * sh.d * sh.Hq * sh.dh):
            qp = capi.spts_linear(xp, wq)
        with tm("pap_probe", 2.0 * sh.Hq * sh.dh * sh.P * sh.n):
            S = capi.spts_probe_attention(qp.view(sh.P, sh.Hq, sh.dh), kk)
        with tm("select_attn", 4.0 * sh.n + 4.0 * k):
            capi.spts_score_topk(S, k, sh.P)
    record("long_128k_score", score128k, sh.n, {"tokens": sh.n, "probes": sh.P, "keep": cfg128k["keep_attn"],
                                                 "needles": cfg128k["needles"], "keys": "clustered"})
    # the whole 131072-token layer: PAP over the clustered keys, reduced
    # attention over 32768 selected queries, LTP, fused select, reduced FFN
    w = {k2: inp[k2].to(dev) for k2 in keys if k2 in inp}     # no Wk: the keys are given
    x0 = inp["x"].to(dev)
    pos = torch.arange(sh.n, dtype=torch.int32, device=dev)
    cfg = LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfg128k["keep_attn"],
                      keep_ffn=cfg128k["keep_ffn"], w_fuse=cfg128k["w_fuse"])

    def layer128k(tm):
        with tm("layer_setup", 4.0 * x0.numel()):
            x = x0.clone()
        pipeline.spts_layer(x, pos, w, cfg, k_given=kk, tm=tm)
    record("long_layer_128k", layer128k, sh.n, {"tokens": sh.n, "probes": sh.P, "keep": cfg128k["keep_attn"],
                                                 "needles": cfg128k["needles"], "keys": "clustered, given"})
    del inp, xp, wq, kk, w, x0

    shp = W.LayerShape(n=cfg128k["prefix"], P=sh.P)
    inp = W.make_layer(shp, seed=cfg128k["seed"], needles=64, clustered_keys=(cfg128k["centroids"], cfg128k["sigma"]))
    w = {k2: inp[k2].to(dev) for k2 in keys if k2 in inp}   # no Wk: the keys are given
    x0 = inp["x"].to(dev)
    kg = inp["k"].to(dev)
    pos = torch.arange(shp.n, dtype=torch.int32, device=dev)
    cfg = LayerConfig(Hq=shp.Hq, Hkv=shp.Hkv, dh=shp.dh, P=shp.P, keep_attn=cfg128k["keep_attn"], keep_ffn=cfg128k["keep_ffn"],
                      w_fuse=cfg128k["w_fuse"])

    def prefix16k(tm):
        x = x0.clone()
        pipeline.spts_layer(x, pos, w, cfg, k_given=kg, tm=tm)
    record("long_16k_prefix", prefix16k, shp.n, {"tokens": shp.n, "probes": shp.P, "keep": cfg128k["keep_attn"],
                                                  "keys": "clustered, given"})
    return out


def select_batched_table(dev, rows=256, n=32768, k=11469, nf=64, reps=10):
    """Capability micro-benchmark of the top-k kernel: one call holds only
    128 KiB of scores, so its time is latency, not bandwidth; a batch of
    independent 32K rows in one launch (one workgroup per row) shows the
    kernel's throughput.  Bytes: scores read + indices written."""
    import torch
    from free_token_skipping_amd import capi
    g = torch.Generator(device="cpu").manual_seed(0)
    s = torch.empty(rows, n).exponential_(generator=g).to(dev)
    idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    one = torch.empty(k, dtype=torch.int32, device=dev)

    def clock(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)       # keeps the GPU busy while the host enqueues the reps
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    ms_b = clock(lambda: capi.spts_score_topk_batched(s, k, nf, idx))
    ms_1 = clock(lambda: capi.spts_score_topk(s[0], k, nf, idx=one))
    nbytes = rows * n * 4 + rows * k * 4
    gbs = nbytes / (ms_b * 1e-3) / 1e9
    log(f"select: one 32K row {ms_1 * 1e3:.1f} us; {rows} rows in one launch {ms_b * 1e3:.1f} us, {gbs:,.0f} GB/s")
    return {"rows": rows, "n": n, "k": k, "forced": nf, "one_row_us": round(ms_1 * 1e3, 1),
            "batch_us": round(ms_b * 1e3, 1), "batch_bytes": nbytes, "batch_gbs": round(gbs, 1),
            "batch_frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


# ------------------------------------------------- HBM-bound row kernels

def hbm_table(x0, reps=5):
    """Standalone gather and scatter-add of the 32K layer's selected rows
    (11469 of 32768 rows of 4096 bf16): algorithmic bytes / time against the
    8 TB/s HBM peak.  Cold: a 1.5 GiB buffer is read before each rep, so the
    256 MB last-level cache holds none of the operands and no dirty lines of
    its own (a written flush buffer would be written back to HBM during the
    timed kernel); warm: four calls back to back.  Either way the call is
    enqueued while the GPU is still busy (with the flush read, or the call
    before), so the events time the kernel, not the binding's host work."""
    import numpy as np
    import torch
    from free_token_skipping_amd import capi
    N, d = x0.shape
    k = 11469
    rng = np.random.default_rng(0)
    idx = torch.from_numpy(np.sort(rng.choice(N, k, replace=False)).astype(np.int32)).to(x0.device)
    src = torch.empty((k, d), dtype=torch.bfloat16, device=x0.device)
    dst = x0.clone()
    flush = torch.ones(3 << 28, dtype=torch.float16, device=x0.device)      # 1.5 GiB
    row = d * 2
    cases = {"gather": (lambda: capi.spts_gather(x0, idx, src), 2.0 * k * row),
             "scatter_add": (lambda: capi.spts_scatter(src, idx, dst, accumulate=True), 3.0 * k * row)}
    out = {}
    for name, (fn, nbytes) in cases.items():
        fn()
        for mode in ("cold", "warm"):
            ts = []
            for r in range(reps):
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                # the GPU is kept busy while the host enqueues the timed call, so
                # the events bracket the kernel and not the call's host-side work
                if mode == "cold":
                    flush.amax()                          # reads every line of the flush buffer
                    e0.record()
                    fn()
                    e1.record()
                    reps_in = 1
                else:
                    fn()
                    e0.record()
                    for _ in range(4):
                        fn()
                    e1.record()
                    reps_in = 4
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) / reps_in)
            ms = sorted(ts)[len(ts) // 2]
            gbs = nbytes / (ms * 1e-3) / 1e9
            out[f"{name}_{mode}"] = {"us": round(ms * 1e3, 1), "bytes": int(nbytes), "gbs": round(gbs, 1),
                                     "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
            log(f"{name} {mode}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.0%} of HBM peak)")
    del flush
    return out


# ------------------------------------------------------------ CPU baseline

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return os.cpu_count()


def _oracle_layer_sampled(x, pos, w, cfg, frac, rng):
    """One oracle layer timed on the host as a CPU baseline (the oracle is
    test infrastructure; it runs here only to be timed).  Every step that
    needs all rows runs in full: pre-norm, K/V and probe-query projections,
    PAP score, selections, LTP score over every row, fused score.  The steps
    that are independent per selected row (Q projection + reduced attention +
    O projection + residual add; SwiGLU + residual add) run on about a
    fraction `frac` of the selected rows (attention: evenly spaced blocks of
    256 consecutive rows) and are scaled by the ratio of rows.
    Returns a dict of seconds: measured and estimated for the whole layer,
    and the projection + probe part (which scales with the candidates)."""
    import numpy as np
    from oracle import numerics, normrope, pap, select, attention, ltp, ffn
    from oracle.layer import project
    Hq, Hkv, dh, P = cfg["Hq"], cfg["Hkv"], cfg["dh"], cfg["P"]
    theta, prenorm, scale = cfg.get("theta"), cfg.get("prenorm", False), dh ** -0.5
    t0 = time.perf_counter()
    xt = numerics.bf16(normrope.rmsnorm(x)) if prenorm else x
    K = project(xt, w["wk"], Hkv, dh, pos, theta)
    V = project(xt, w["wv"], Hkv, dh)
    Qp = project(xt[-P:], w["wq"], Hq, dh, pos[-P:], theta)
    S = pap.pap_scores(Qp, K, scale)
    t_kvp = time.perf_counter() - t0
    n = x.shape[0]
    k_a = numerics.keep_count(0.35, n)
    idx = select.select_topk(numerics.f32(S), k_a, P)
    t_full = time.perf_counter() - t0
    # attention rows: evenly spaced blocks of 256 consecutive selected rows,
    # each one chunk of the oracle's attention loop as in the whole run (a
    # row's cost grows with its position, so the blocks' mean is the layer's)
    nb = min(max(2, int(round(k_a * frac / 256))), (k_a + 255) // 256)
    starts = np.unique(np.linspace(0, max(0, k_a - 256), nb).astype(np.int64))
    blocks = [idx[b0:b0 + 256] for b0 in starts]
    m = sum(len(b) for b in blocks)
    y = x.copy()
    t1 = time.perf_counter()
    for qi in blocks:
        Qs = project(xt[qi], w["wq"], Hq, dh, pos[qi], theta)
        O = numerics.bf16(attention.reduced_attention(Qs, qi, K, V, scale))
        y[qi] = numerics.bf16(x[qi] + numerics.bf16(O.reshape(len(qi), -1) @ w["wo"].T))
    t_rows = (time.perf_counter() - t1) * k_a / m
    t_meas = time.perf_counter() - t1
    t2 = time.perf_counter()
    z = numerics.bf16(normrope.rmsnorm(y)) if prenorm else y
    L = ltp.ltp_scores(z, w["u_t"], w["v_t"])
    idx_f = select.select_topk(select.fuse_maxnorm(numerics.f32(S), numerics.f32(L)), k_a, P)
    t_full += time.perf_counter() - t2
    mf = max(1, int(round(k_a * frac)))
    fi = idx_f[np.sort(rng.choice(k_a, mf, replace=False))]
    t3 = time.perf_counter()
    _, yv = ffn.swiglu_rows(z[fi], w["wg"], w["wu"], w["wd"])
    _ = numerics.bf16(y[fi] + yv)
    t_rows += (time.perf_counter() - t3) * k_a / mf
    t_meas += t_full + time.perf_counter() - t3
    return {"est": t_full + t_rows, "measured": t_meas, "kvp": t_kvp, "rows_sampled": m + mf, "rows": 2 * k_a}


def cpu_baseline(sh, st, n_layers, points, frac):
    """The CPU oracle timed on a bounded sample of the stack workload.

    Per MSDP stage (2 layers, c_s candidates) one oracle layer runs on c_s
    rows with that stage's first-layer weights (_oracle_layer_sampled: steps
    over all rows in full, per-row steps on a fraction of the selected rows,
    scaled).  The stage's first layer also projects and probes the c_{s-1}
    outgoing rows before its boundary, so the stage costs twice the layer
    plus the projection + probe part scaled by c_{s-1}/c_s - 1."""
    import numpy as np
    import workloads as W
    cfg = dict(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, prenorm=True, theta=500000.0)
    rng = np.random.default_rng(0)
    t_stack = measured = 0.0
    c_prev = sh.n
    for si, layer_idx in enumerate(sorted(points)):
        c = points[layer_idx]
        w = {k: W.as_f64(v) for k, v in st["layers"][layer_idx].items()}
        x = W.as_f64(st["x"][:c])
        r = _oracle_layer_sampled(x, np.arange(c), w, cfg, frac, rng)
        measured += r["measured"]
        t_stack += 2 * r["est"] + r["kvp"] * (c_prev / c - 1.0)
        c_prev = c
        log(f"cpu oracle stage {si}: {c} candidates, measured {r['measured']:.1f}s, layer est {r['est']:.1f}s")
    cores = _blas_threads()
    return {"value": round(n_layers * sh.n / t_stack, 1), "unit": "tokens/s/layer", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"the 8-layer 32K stack: one oracle layer per MSDP stage at its candidate count "
                       f"(19661/14746/11469/8192 of 32768 rows); the steps over all rows (RMSNorm, K/V and "
                       f"probe-query projections, PAP score, selections, LTP score, fused score) run in full, "
                       f"the per-row steps (Q projection + reduced attention + O projection, SwiGLU) on about "
                       f"{frac:.4f} of the selected rows (at least two 256-row blocks), scaled by the row ratio; "
                       f"stack = 2 x each stage's "
                       f"layer + the first layer's projections and probe over the outgoing rows; "
                       f"{measured:.1f}s measured on {cores} BLAS threads"),
            "seconds_per_step_est": round(t_stack, 2), "seconds_measured": round(measured, 2),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count(),
            "numpy": np.__version__}


def cpu_baseline_layer(x0, w0, n, frac, full=False):
    """The CPU oracle on the single 32K layer (attention + FFN, PAP + LTP,
    keep 0.35 / 0.35): the same sampling as the stack's, or (full=True) the
    oracle's whole layer run unsampled."""
    import numpy as np
    import workloads as W
    from oracle import layer as olayer
    w = {k: W.as_f64(v) for k, v in w0.items()}
    x = W.as_f64(x0)
    cores = _blas_threads()
    if full:
        t0 = time.perf_counter()
        olayer.spts_layer(x, np.arange(n), w, dict(Hq=32, Hkv=8, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35))
        sec = time.perf_counter() - t0
        return {"value": round(n / sec, 1), "unit": "tokens/s/layer", "cores": int(cores), "kind": "oracle",
                "sample": "the whole 32K layer, unsampled", "seconds_measured": round(sec, 2)}
    r = _oracle_layer_sampled(x, np.arange(n), w, dict(Hq=32, Hkv=8, dh=128, P=64), frac,
                              np.random.default_rng(1))
    return {"value": round(n / r["est"], 1), "unit": "tokens/s/layer", "cores": int(cores), "kind": "oracle",
            "sample": (f"the 32K layer: steps over all rows in full, per-row steps on {r['rows_sampled']} of "
                       f"{r['rows']} selected rows, scaled; {r['measured']:.1f}s measured"),
            "seconds_per_layer_est": round(r["est"], 2), "seconds_measured": round(r["measured"], 2)}


# --------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the SPTS path here runs on a "
              f"single GPU and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import torch
    from free_token_skipping_amd import capi, pipeline
    from free_token_skipping_amd.pipeline import LayerConfig, keep_count
    capi.lib()                                               # no library -> fail loudly
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fused = not args.unfused
    if args.probe_only:
        import workloads as W
        out = {}
        for n, P in ((32768, 64), (131072, 128)):
            q = W.randn((P, 32, 128), seed=1, std=1.28).to(dev)
            k = W.randn((n, 8, 128), seed=2, std=1.28).to(dev)
            S = torch.empty(n, dtype=torch.float32, device=dev)
            for _ in range(3):
                capi.spts_probe_attention(q, k, scores=S)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(50_000_000)              # the GPU stays busy while the calls are enqueued
            e0.record()
            for _ in range(20):
                capi.spts_probe_attention(q, k, scores=S)
            e1.record()
            torch.cuda.synchronize()
            out[f"n{n}_p{P}_us"] = round(e0.elapsed_time(e1) / 20 * 1e3, 1)
        print(json.dumps({"pap_probe": out}), flush=True)
        return
    if args.calibrate_copy:
        rows, width = 131072, 4096                       # 1 GiB of bf16 read + 1 GiB written
        src = torch.ones((rows, width), dtype=torch.bfloat16, device=dev)
        ident = torch.arange(rows, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            capi.spts_gather(src, ident, dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": rows * width * 2, "bytes_written": rows * width * 2,
                          "dispatches": 3}), flush=True)
        return

    cfgd, sh, st, x0, layers = stack_inputs(dev)
    N = sh.n
    if args.decode_only:
        cfg = LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"],
                          keep_ffn=cfgd["keep_ffn"], w_fuse=cfgd["w_fuse"], prenorm=True, eps=cfgd["eps"],
                          theta=cfgd["theta"])
        print(json.dumps({"decode_32_layers": decode_table(x0, layers, cfg)}), flush=True)
        return
    budgets = [keep_count(r, N) for r in cfgd["budget_ratios"]]
    points = pipeline.prune_points(0, cfgd["stage_ends"], budgets)
    stack_cfg = LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=cfgd["keep_attn"],
                            keep_ffn=cfgd["keep_ffn"], w_fuse=cfgd["w_fuse"], prenorm=True, eps=cfgd["eps"],
                            theta=cfgd["theta"])
    layer_cfg = LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=0.35, keep_ffn=0.35)
    pos0 = torch.arange(N, dtype=torch.int32, device=dev)
    n_layers = len(layers)

    def stack_step(tm):
        pipeline.msdp_stack(x0, layers, stack_cfg, points, fused=fused, tm=tm)

    def layer_step(tm):
        # one bare 32K layer (PAP + LTP); the layer-0 weights of the stack are the
        # 32K layer workload's inputs (same seed and draw order)
        with tm("layer_setup", 4.0 * x0.numel()):
            x = x0.clone()
        pipeline.spts_layer(x, pos0, layers[0], layer_cfg, fused=fused, tm=tm)

    # the pages' default scoring on the same layer: Multiply fusion and the
    # structured proxy (512 hidden channels, rank 256 per projection), its
    # factors drawn from layer 0's own feed-forward weights
    defaults_cfg = LayerConfig(Hq=sh.Hq, Hkv=sh.Hkv, dh=sh.dh, P=sh.P, keep_attn=0.35, keep_ffn=0.35,
                               fusion="multiply", proxy="structured")
    defaults_w = None
    if not args.no_single_layer:
        import workloads as W
        sp = W.structured_proxy(st["layers"][0]["wg"], st["layers"][0]["wu"], st["layers"][0]["wd"], 512, 256,
                                seed=cfgd["seed"])
        defaults_w = dict(layers[0])
        defaults_w["proxy_packed"] = capi.pack_structured_proxy(
            *[sp[k].to(dev) for k in ("a_g_t", "b_g_t", "a_u_t", "b_u_t", "c_t", "d_t")])

    def defaults_step(tm):
        with tm("layer_setup", 4.0 * x0.numel()):
            x = x0.clone()
        pipeline.spts_layer(x, pos0, defaults_w, defaults_cfg, fused=fused, tm=tm)

    results = {}
    for name, fn, nl in (("msdp_stack_32k", stack_step, n_layers), ("layer_32k", layer_step, 1),
                         ("layer_32k_page_defaults", defaults_step, 1)):
        if name != args.workload and (args.no_single_layer or name == "msdp_stack_32k"):
            continue
        if name == "layer_32k_page_defaults" and defaults_w is None:
            continue
        log(f"timing {name}: warmup {args.warmup}, steps {args.steps}")
        total_ms, wall_ms, summ, summ_dom = timed(fn, args.steps, args.warmup)
        ms = total_ms / args.steps
        results[name] = dict(ms_per_step=ms, wall_ms_per_step=wall_ms / args.steps,
                             tokens_per_s_per_layer=nl * N / (ms * 1e-3),
                             breakdown=breakdown(summ, args.steps),
                             roofline=roofline(summ_dom, args.steps, with_rocprof=(name == "msdp_stack_32k")))
        log(f"{name}: {ms:.3f} ms/step, {nl * N / (ms * 1e-3):,.0f} tokens/s/layer")

    head = results[args.workload]
    rec = {
        "metric": "SPTS prefill tokens/s per layer at 32K",
        "value": round(head["tokens_per_s_per_layer"], 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": ({"workload": "msdp_stack_32k", "tokens": N, "layers": n_layers, "stages": "2 layers each",
                    "candidate_budgets": budgets, "keep_attn": cfgd["keep_attn"], "keep_ffn": cfgd["keep_ffn"],
                    "probes": sh.P, "shape": "LLaMA-3.1-8B (d 4096, 32/8 heads, d_head 128, SwiGLU 14336)",
                    "ltp_rank": sh.r, "fused_gather_scatter": fused}
                   if args.workload == "msdp_stack_32k" else
                   {"workload": "layer_32k", "tokens": N, "layers": 1, "keep_attn": 0.35, "keep_ffn": 0.35,
                    "probes": sh.P, "ltp_rank": sh.r, "fused_gather_scatter": fused}),
        "roofline": head["roofline"],
        "breakdown": head["breakdown"],
        "wall_ms_per_step": round(head["wall_ms_per_step"], 4),
    }
    for name, r in results.items():
        if name != args.workload:
            rec.setdefault("also", {})[name] = {"tokens_per_s_per_layer": round(r["tokens_per_s_per_layer"], 1),
                                                "ms_per_step": round(r["ms_per_step"], 4),
                                                "roofline": r["roofline"], "breakdown": r["breakdown"]}
    if not args.no_hbm:
        log("timing the standalone gather / scatter-add, cold and warm")
        rec.setdefault("also", {})["hbm_row_kernels"] = hbm_table(x0)
        rec["also"]["select_batched"] = select_batched_table(dev)
    if not args.no_ttft:
        log("timing the 32-layer prefill schedule against dense")
        rec.setdefault("also", {})["prefill_32_layers"] = ttft_table(x0, layers, stack_cfg)
    if not args.no_other:
        log("timing the 8K attention layer, the 128K score path and the 16K prefix layer")
        rec.setdefault("also", {}).update(other_workloads(dev, args.steps, args.warmup))
    if not args.no_decode:
        log("timing decode after the 32-layer prefill, SPTS against full caches")
        rec.setdefault("also", {})["decode_32_layers"] = decode_table(x0, layers, stack_cfg)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(sh, st, n_layers, points, args.cpu_sample)
        log("timing the CPU oracle on the single 32K layer" + (" (unsampled)" if args.cpu_full else ""))
        rec.setdefault("also", {})["cpu_baseline_layer_32k"] = cpu_baseline_layer(
            st["x"], st["layers"][0], N, args.cpu_sample, full=args.cpu_full)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
