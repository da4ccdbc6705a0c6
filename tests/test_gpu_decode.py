"""Decode phase on the GPU against the oracle: one-row projections, the
split-key decode attention over a layer's cache, and whole decode steps after
a prefill (each side builds its own caches from the same seeded inputs)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import numerics, normrope, attention, layer as olayer, decode as odecode
from free_token_skipping_amd import capi, pipeline
from parity import np64, assert_close, BF16_REL

pytestmark = pytest.mark.gpu
DEV = "cuda"
WKEYS = ["wq", "wk", "wv", "wo", "wg", "wu", "wd", "u_t", "v_t"]


def _log(msg):
    print(msg, flush=True)


def _cuda(t):
    return t.to(DEV)


@pytest.mark.parametrize("kdim,n", [(4096, 1024), (14336, 512), (512, 256)])
def test_decode_linear_store_and_accumulate(kdim, n):
    _log(f"decode linear kdim={kdim} n={n}")
    x = W.randn((kdim,), seed=80)
    w = W.randn((n, kdim), seed=81, std=0.02)
    y = capi.spts_decode_linear(_cuda(x), _cuda(w))
    acc = numerics.f32(W.as_f64(w) @ W.as_f64(x))
    assert_close(np64(y), numerics.bf16(acc), BF16_REL, "decode linear")
    base = W.randn((n,), seed=82)
    out = _cuda(base).clone()
    capi.spts_decode_linear(_cuda(x), _cuda(w), out=out, accumulate=True)
    assert_close(np64(out), numerics.bf16(W.as_f64(base) + numerics.bf16(acc)), BF16_REL, "decode residual add")


def test_decode_linear_rope_and_swiglu():
    _log("decode rope / swiglu")
    kdim, n, pos, theta = 4096, 1024, 777, 500000.0
    x = W.randn((kdim,), seed=83)
    w = W.randn((n, kdim), seed=84, std=0.02)
    table = capi.spts_rope_table(4096, 128, theta, DEV)
    y = capi.spts_decode_linear_rope(_cuda(x), _cuda(w), pos, table)
    acc = numerics.f32(W.as_f64(w) @ W.as_f64(x)).reshape(1, n // 128, 128)
    ref = numerics.bf16(normrope.rope(acc, np.array([pos]), theta)).reshape(n)
    assert_close(np64(y), ref, BF16_REL, "decode rope")
    wg = W.randn((n, kdim), seed=85, std=0.02)
    wu = W.randn((n, kdim), seed=86, std=0.02)
    h = capi.spts_decode_swiglu(_cuda(x), _cuda(wg), _cuda(wu))
    g = numerics.f32(W.as_f64(wg) @ W.as_f64(x))
    u = numerics.f32(W.as_f64(wu) @ W.as_f64(x))
    assert_close(np64(h), numerics.bf16(g / (1.0 + np.exp(-g)) * u), BF16_REL, "decode swiglu")


@pytest.mark.parametrize("L", [1, 200, 256, 257, 3000, 4096, 9000, 16384, 32768])
def test_decode_attention(L):
    _log(f"decode attention L={L}")
    Hq, Hkv, dh, cap = 32, 8, 128, L + 37
    q = W.randn((Hq, dh), seed=87)
    k = W.randn((L, Hkv, dh), seed=88)
    v = W.randn((L, Hkv, dh), seed=89)
    kc = torch.full((cap, Hkv, dh), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full((cap, Hkv, dh), float("nan"), dtype=torch.bfloat16, device=DEV)
    kc[:L] = _cuda(k)
    vc[:L] = _cuda(v)
    o = capi.spts_decode_attention(_cuda(q), kc, vc, L)
    ref = attention.reduced_attention(W.as_f64(q)[None], np.array([L - 1]), W.as_f64(k), W.as_f64(v),
                                      1.0 / np.sqrt(dh))[0]
    got = np64(o)
    assert np.isfinite(got).all()                          # rows past L (NaN) are never read
    assert_close(got, numerics.bf16(ref), BF16_REL, "decode attention")


def _small_model(n=300):
    sh = W.LayerShape(n=n, d=512, Hq=8, Hkv=2, dh=128, f=1024, r=256, P=64)
    st = W.make_stack(sh, 2, seed=7)
    cfg = pipeline.LayerConfig(Hq=8, Hkv=2, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, prenorm=True,
                               eps=1e-5, theta=500000.0)
    ocfg = dict(Hq=8, Hkv=2, dh=128, P=64, keep_attn=1.0, keep_ffn=1.0, prenorm=True, eps=1e-5, theta=500000.0)
    return sh, st, cfg, ocfg


@pytest.mark.parametrize("native", [False, True])
def test_decode_after_dense_prefill(native):
    sh, st, cfg, ocfg = _small_model()
    step = pipeline.decode_step_native if native else pipeline.decode_step
    ws = [{k: w[k].to(DEV) for k in WKEYS} for w in st["layers"]]
    steps = 3
    new = W.randn((steps, sh.d), seed=90)
    _log(f"gpu dense prefill + decode (native step: {native})")
    kvs = []
    x, pos = pipeline.prefill_schedule(st["x"].to(DEV), ws, cfg, n_layers=2, first_skip_layer=2, points={},
                                       kv_out=kvs)
    caches = pipeline.DecodeCaches(kvs, steps)
    table = capi.spts_rope_table(sh.n + steps, 128, 500000.0, DEV)
    outs = []
    for s in range(steps):
        xr = _cuda(new[s]).clone()
        outs.append(np64(step(xr, sh.n + s, ws, caches, cfg, table)))
    assert caches.lengths == [sh.n + steps] * 2
    _log("oracle dense prefill + decode")
    ows = [{k: W.as_f64(w[k]) for k in WKEYS} for w in st["layers"]]
    ref = W.as_f64(st["x"])
    ocaches = []
    for w in ows:
        ref, sa, _ = olayer.spts_layer(ref, np.arange(sh.n), w, ocfg)
        ocaches.append([sa["K"], sa["V"]])
    for s in range(steps):
        r = odecode.decode_step(W.as_f64(new[s]), sh.n + s, ocaches, ows, ocfg)
        assert_close(outs[s], r, BF16_REL, f"decoded token {s}")


def test_decode_after_spts_prefill_structure():
    """SPTS caches hold each layer's candidates (MSDP budget); decode runs on them."""
    sh, st, cfg, _ = _small_model(n=700)
    ws = [{k: w[k].to(DEV) for k in WKEYS} for w in st["layers"]]
    kvs = []
    pipeline.prefill_schedule(st["x"].to(DEV), ws, cfg, n_layers=2, first_skip_layer=0, points={0: 500, 1: 300},
                              kv_out=kvs)
    assert [k.shape[0] for k, _ in kvs] == [500, 300]
    caches = pipeline.DecodeCaches(kvs, 2)
    table = capi.spts_rope_table(sh.n + 2, 128, 500000.0, DEV)
    x = pipeline.decode_step(_cuda(W.randn((sh.d,), seed=91)).clone(), sh.n, ws, caches, cfg, table)
    assert caches.lengths == [501, 301]
    assert torch.isfinite(x.float()).all()


def test_native_step_matches_per_call_step_after_spts_prefill():
    """The one-call step (fused norms, one QKV launch) against the per-call
    composition on the same SPTS caches: outputs and the cache rows written."""
    sh, st, cfg, _ = _small_model(n=700)
    ws = [{k: w[k].to(DEV) for k in WKEYS} for w in st["layers"]]
    kvs = []
    pipeline.prefill_schedule(st["x"].to(DEV), ws, cfg, n_layers=2, first_skip_layer=0, points={0: 500, 1: 300},
                              kv_out=kvs)
    steps = 3
    a, b = pipeline.DecodeCaches(kvs, steps), pipeline.DecodeCaches(kvs, steps)
    table = capi.spts_rope_table(sh.n + steps, 128, 500000.0, DEV)
    for s in range(steps):
        x0 = _cuda(W.randn((sh.d,), seed=92 + s))
        xa = pipeline.decode_step(x0.clone(), sh.n + s, ws, a, cfg, table)
        xb = pipeline.decode_step_native(x0.clone(), sh.n + s, ws, b, cfg, table)
        assert_close(np64(xb), np64(xa), BF16_REL, f"native step {s}")
    assert a.lengths == b.lengths == [503, 303]
    for li in range(2):
        L = a.lengths[li]
        assert_close(np64(b.k[li][:L]), np64(a.k[li][:L]), BF16_REL, f"layer {li} k cache")
        assert_close(np64(b.v[li][:L]), np64(a.v[li][:L]), BF16_REL, f"layer {li} v cache")


def test_native_step_rejects_a_full_cache():
    sh, st, cfg, _ = _small_model()
    ws = [{k: w[k].to(DEV) for k in WKEYS} for w in st["layers"]]
    kvs = [(torch.zeros((10, 2, 128), dtype=torch.bfloat16, device=DEV),) * 2 for _ in range(2)]
    caches = pipeline.DecodeCaches(kvs, 1)
    table = capi.spts_rope_table(16, 128, 500000.0, DEV)
    x = _cuda(W.randn((sh.d,), seed=95))
    pipeline.decode_step_native(x, 10, ws, caches, cfg, table)
    assert caches.lengths == [11, 11]
    with pytest.raises(capi.SptsError, match="cache holds 11 of 11"):
        pipeline.decode_step_native(x, 11, ws, caches, cfg, table)
    assert caches.lengths == [11, 11]


def test_decode_step_full_llama_shape():
    """One decode step at the LLaMA-3.1-8B layer shape (d 4096, 32/8 heads,
    d_head 128, SwiGLU 14336), two layers whose caches hold different row
    counts (as after MSDP), through the one-call step and the per-call step,
    against the oracle's decode of the same caches."""
    sh = W.LayerShape(n=64)
    st = W.make_stack(sh, 2, seed=11)
    ws = [{k: w[k].to(DEV) for k in WKEYS} for w in st["layers"]]
    cfg = pipeline.LayerConfig(Hq=32, Hkv=8, dh=128, P=64, keep_attn=0.35, keep_ffn=0.35, prenorm=True, eps=1e-5,
                               theta=500000.0)
    ocfg = dict(Hq=32, Hkv=8, dh=128, prenorm=True, eps=1e-5, theta=500000.0)
    lens, pos = [3000, 700], 5000
    kvs = [(W.randn((L, 8, 128), seed=100 + 2 * i), W.randn((L, 8, 128), seed=101 + 2 * i)) for i, L in enumerate(lens)]
    x = W.randn((4096,), seed=99)
    _log("oracle decode at the LLaMA shape")
    ows = [{k: W.as_f64(w[k]) for k in WKEYS} for w in st["layers"]]
    ocaches = [[W.as_f64(k), W.as_f64(v)] for k, v in kvs]
    ref = odecode.decode_step(W.as_f64(x), pos, ocaches, ows, ocfg)
    table = capi.spts_rope_table(pos + 1, 128, 500000.0, DEV)
    for native in (True, False):
        _log(f"gpu decode at the LLaMA shape (native step: {native})")
        caches = pipeline.DecodeCaches([(k.to(DEV), v.to(DEV)) for k, v in kvs], 1)
        step = pipeline.decode_step_native if native else pipeline.decode_step
        out = step(_cuda(x).clone(), pos, ws, caches, cfg, table)
        assert caches.lengths == [3001, 701]
        assert_close(np64(out), ref, BF16_REL, f"decode output (native {native})")
        for li in range(2):
            assert_close(np64(caches.k[li][lens[li]]), ocaches[li][0][-1], BF16_REL, f"layer {li} new key")
            assert_close(np64(caches.v[li][lens[li]]), ocaches[li][1][-1], BF16_REL, f"layer {li} new value")
