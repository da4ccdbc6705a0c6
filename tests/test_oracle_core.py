"""Pins of the CPU oracle against facts fixed by the pages and by mathematics
(closed forms, brute force, library routines, printed tables).  CPU only."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import numerics, pap, select, attention, ltp, ffn, normrope, layer, costs
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ numerics

def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        [0.0, -0.0, 1.0, -2.0, np.inf, -np.inf, 3.0e38, 1e-40, -1e-42],
        1.0 + np.arange(0, 64) * 2.0 ** -9,          # exact ties and near-ties
    ])
    ours = numerics.to_bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_known_patterns():
    bits = numerics.to_bf16_bits(np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0, np.nan]))
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x7FC0]
    assert numerics.from_bf16_bits(np.array([0x3F80, 0x4049], np.uint16)).tolist() == [1.0, 3.140625]


def test_keep_counts():
    assert numerics.keep_count(0.35, 32768) == 11469
    assert numerics.keep_count(0.5, 8192) == 4096
    assert [numerics.keep_count(r, 32768) for r in (0.6, 0.45, 0.35, 0.25)] == [19661, 14746, 11469, 8192]
    assert numerics.keep_count(0.25, 131072) == 32768
    assert numerics.keep_count(1.0, 7) == 7 and numerics.keep_count(0.0, 7) == 0


# ------------------------------------------------------------------------ PAP

def _pap_brute(q, k, scale):
    P, Hq, dh = q.shape
    n, Hkv, _ = k.shape
    S = [0.0] * n
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for p in range(P):
            row = n - P + p
            logits = [scale * sum(q[p, h, e] * k[j, g, e] for e in range(dh)) for j in range(row + 1)]
            mx = max(logits)
            ex = [math.exp(t - mx) for t in logits]
            tot = sum(ex)
            for j in range(row + 1):
                S[j] += ex[j] / tot
    return np.array(S)


def test_pap_brute_force():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((5, 4, 8))
    k = rng.standard_normal((20, 2, 8))
    got = pap.pap_scores(q, k, 0.3)
    assert np.allclose(got, _pap_brute(q, k, 0.3), rtol=1e-12, atol=1e-14)


def test_pap_mass_is_heads_times_probes():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((16, 8, 32))
    k = rng.standard_normal((300, 2, 32))
    S = pap.pap_scores(q, k, 1 / math.sqrt(32))
    assert abs(S.sum() - 8 * 16) < 1e-10
    assert (S >= 0).all()


def test_pap_single_probe_is_torch_softmax():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((40, 1, 16))
    logits = torch.from_numpy(0.25 * (k[:, 0, :] @ q[0, 0]))
    ref = torch.softmax(logits, dim=-1).numpy()
    assert np.allclose(pap.pap_scores(q, k, 0.25), ref, rtol=1e-13, atol=1e-15)


def test_pap_gqa_groups_are_contiguous():
    # Hq=4, Hkv=2: heads 0,1 read key head 0; heads 2,3 read key head 1.
    n, dh = 12, 4
    k = np.zeros((n, 2, dh))
    k[3, 0, 0] = 50.0            # key head 0 peaks at token 3
    k[7, 1, 1] = 50.0            # key head 1 peaks at token 7
    q = np.zeros((1, 4, dh))
    q[0, :, 0] = 1.0
    q[0, :, 1] = 1.0
    S = pap.pap_scores(q, k, 1.0)
    assert abs(S[3] - 2.0) < 1e-12 and abs(S[7] - 2.0) < 1e-12


def test_pap_is_causal():
    # The last key would dominate every probe, but only the last probe sees it.
    n, dh = 10, 2
    k = np.zeros((n, 1, dh))
    k[-1, 0, 0] = 100.0
    q = np.zeros((2, 3, dh))
    q[:, :, 0] = 1.0
    S = pap.pap_scores(q, k, 1.0)
    assert abs(S[-1] - 3.0) < 1e-12          # 3 heads x weight ~1 from the last probe
    assert abs(S[:-1].sum() - 3.0) < 1e-12   # the other probe row spreads over 9 keys
    assert np.allclose(S[:-1], 3.0 / 9.0)


# ---------------------------------------------------------------------- select

def _select_by_dominance(s, k, nf):
    """Independent definition: the chosen free rows beat every unchosen free
    row under (larger score, then lower index); searched exhaustively."""
    n = len(s)
    if k >= n:
        return [list(range(n))]
    free = list(range(n - nf))
    sols = []
    for combo in itertools.combinations(free, k - nf):
        c = set(combo)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in c for j in free if j not in c)
        if ok:
            sols.append(sorted(c | set(range(n - nf, n))))
    return sols


@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_select_brute_force_all_tie_patterns(n):
    rng = np.random.default_rng(n)
    patterns = list(itertools.product([0.0, 1.0, 2.0], repeat=n)) if n <= 5 else \
        [tuple(rng.integers(0, 3, n).astype(float)) for _ in range(60)]
    for pat in patterns:
        s = np.array(pat)
        for nf in range(0, min(n, 2) + 1):
            for k in range(nf, n + 2):
                sols = _select_by_dominance(s, k, nf)
                assert len(sols) == 1
                assert select.select_topk(s, k, nf).tolist() == sols[0]


def test_select_special_values():
    s = np.array([np.nan, 1.0, -0.0, 0.0, 5.0, 2.0])
    assert select.select_topk(s, 3, 1).tolist() == [1, 4, 5]
    # -0.0 and +0.0 tie: the lower index wins
    assert select.select_topk(np.array([-0.0, 0.0, 1.0]), 2, 0).tolist() == [0, 2]
    assert select.select_topk(np.array([-0.0, 0.0, 1.0]), 2, 1).tolist() == [0, 2]
    assert select.select_topk(s, 1, 1).tolist() == [5]
    with pytest.raises(ValueError):
        select.select_topk(s, 1, 2)


def test_fuse_maxnorm_pins():
    rng = np.random.default_rng(5)
    a = rng.exponential(size=1000).astype(np.float32)
    b = rng.exponential(size=1000).astype(np.float32) * np.float32(1e-3)
    c = select.fuse_maxnorm(a, b)
    assert c.dtype == np.float32
    # identical inputs with weights 1/2 + 1/2 reproduce the normalised score exactly
    assert np.array_equal(select.fuse_maxnorm(a, a), (a / a.max()).astype(np.float32))
    # the normalisation is by the maximum: the argmax of both scores fuses to 1
    a2, b2 = a.copy(), b.copy()
    b2[a.argmax()] = b.max() * np.float32(2)
    assert select.fuse_maxnorm(a2, b2)[a.argmax()] == np.float32(1.0)
    # one weight zero: only the other normalised score remains
    assert np.array_equal(select.fuse_maxnorm(a, b, 1.0, 0.0), (a / a.max()).astype(np.float32))
    # value agrees with the float64 definition to fp32 rounding
    ref = 0.5 * a.astype(np.float64) / a.max() + 0.5 * b.astype(np.float64) / b.max()
    assert np.allclose(c, ref, rtol=3e-7, atol=0)
    # a zero maximum contributes nothing
    assert np.array_equal(select.fuse_maxnorm(a, np.zeros_like(a)), (np.float32(0.5) * (a / a.max())).astype(np.float32))
    # a NaN score: the maxima skip it, so every other row keeps the value it
    # has without the NaN (the float64 definition over the remaining rows),
    # and the NaN row's own fused value is NaN, which ranks lowest
    a3 = a.copy()
    a3[17] = np.nan
    c3 = select.fuse_maxnorm(a3, b)
    rest = np.arange(1000) != 17
    mx = np.max(a[rest].astype(np.float64))
    ref3 = 0.5 * a[rest].astype(np.float64) / mx + 0.5 * b[rest].astype(np.float64) / b.max()
    assert np.allclose(c3[rest], ref3, rtol=3e-7, atol=0) and np.isnan(c3[17])
    assert 17 not in select.select_topk(c3, 999, 0).tolist()
    # all-NaN score: no positive maximum, the term is 0
    nan_all = np.full_like(a, np.nan)
    assert np.array_equal(select.fuse_maxnorm(nan_all, b, 0.5, 0.5),
                          (np.float32(0.5) * (b / b.max())).astype(np.float32))


def test_fuse_multiply_pins():
    rng = np.random.default_rng(6)
    a = rng.exponential(size=1000).astype(np.float32)
    b = rng.exponential(size=1000).astype(np.float32)
    c = select.fuse_multiply(a, b)
    assert c.dtype == np.float32
    # a product of two fp32 values is exact in float64 (24 + 24 < 53 bits), so
    # the correctly rounded fp32 product is that float64 value rounded once
    assert np.array_equal(c, (a.astype(np.float64) * b.astype(np.float64)).astype(np.float32))
    # powers of two scale exactly and leave the ranking unchanged
    c2 = select.fuse_multiply(a * np.float32(4), b * np.float32(0.5))
    assert np.array_equal(c2, c * np.float32(2))
    assert np.array_equal(select.select_topk(c2, 100, 8), select.select_topk(c, 100, 8))
    # a zero factor gives zero
    assert np.all(select.fuse_multiply(a, np.zeros_like(b)) == 0)
    # Multiply and MaxNorm-Add rank differently: a lopsided row wins the sum,
    # a balanced row wins the product
    sa = np.array([1.0, 0.5, 0.01], np.float32)
    sb = np.array([0.01, 0.5, 1.0], np.float32)
    assert select.select_topk(select.fuse_maxnorm(sa, sb), 1, 0).tolist() == [0]
    assert select.select_topk(select.fuse_multiply(sa, sb), 1, 0).tolist() == [1]


# ------------------------------------------------------------------- attention

def _sdpa_gqa(q, k, v, scale):
    """Dense causal attention from torch (float64), GQA by contiguous groups."""
    n, Hq, dh = q.shape
    G = Hq // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_reduced_attention_all_rows_is_dense_causal():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((50, 4, 16))
    k = rng.standard_normal((50, 2, 16))
    v = rng.standard_normal((50, 2, 16))
    o = attention.reduced_attention(q, np.arange(50), k, v, 0.25, row_chunk=7)
    assert np.allclose(o, _sdpa_gqa(q, k, v, 0.25), rtol=1e-10, atol=1e-12)


def test_reduced_attention_rows_are_dense_rows():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((40, 8, 8))
    k = rng.standard_normal((40, 2, 8))
    v = rng.standard_normal((40, 2, 8))
    dense = _sdpa_gqa(q, k, v, 0.4)
    idx = np.array([0, 3, 4, 17, 39])
    o = attention.reduced_attention(q[idx], idx, k, v, 0.4, row_chunk=2)
    assert np.allclose(o, dense[idx], rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------------- LTP

def test_ltp_full_rank_equals_linear_delta():
    rng = np.random.default_rng(8)
    d = 48
    m = rng.standard_normal((d, d)) * 0.02
    u_t, v_t = workloads.proxy_factors(m, d)
    assert np.allclose(u_t.T @ v_t.T, m, rtol=0, atol=1e-13)
    z = rng.standard_normal((30, d))
    assert np.allclose(ltp.ltp_scores(z, u_t, v_t), np.linalg.norm(z @ m, axis=1), rtol=1e-11)


def test_ltp_truncation_keeps_top_singular_values():
    rng = np.random.default_rng(9)
    d, r = 64, 10
    m = rng.standard_normal((d, d))
    u_t, v_t = workloads.proxy_factors(m, r)
    sv = np.linalg.svd(m, compute_uv=False)
    err = np.linalg.norm(m - u_t.T @ v_t.T) ** 2
    assert abs(err - (sv[r:] ** 2).sum()) < 1e-9 * (sv ** 2).sum()
    # the large-d path (partial eigensolve) agrees with the plain SVD path
    big = rng.standard_normal((1100, 1100)) * 0.02
    u1, v1 = workloads.proxy_factors(big, 16)
    a, s, bt = np.linalg.svd(big)
    assert np.allclose(u1.T @ v1.T, (a[:, :16] * s[:16]) @ bt[:16], atol=1e-12)


def test_ltp_exact_low_rank_matrix_is_reproduced():
    rng = np.random.default_rng(10)
    d, r = 40, 6
    m = rng.standard_normal((d, r)) @ rng.standard_normal((r, d))
    u_t, v_t = workloads.proxy_factors(m, r)
    z = rng.standard_normal((9, d))
    assert np.allclose(ltp.ltp_scores(z, u_t, v_t), np.linalg.norm(z @ m, axis=1), rtol=1e-10)


def test_structured_proxy_full_rank_is_swiglu():
    rng = np.random.default_rng(11)
    d, f = 16, 24
    wg, wu, wd = (rng.standard_normal(s) * 0.3 for s in ((f, d), (f, d), (d, f)))
    z = rng.standard_normal((5, d))
    ch = np.arange(f)
    delta = ltp.structured_proxy_delta(z, [wg[ch].T], [wu[ch].T], [wd[:, ch].T], ch)
    ref = (F.silu(torch.from_numpy(z @ wg.T)) * torch.from_numpy(z @ wu.T)).numpy() @ wd.T
    assert np.allclose(delta, ref, rtol=1e-12, atol=1e-13)


def test_structured_scores_exact_factors_are_swiglu_norm():
    # each projection given as (weight, identity): the score is ||SwiGLU(z)||
    rng = np.random.default_rng(13)
    d, f = 16, 24
    wg, wu, wd = (rng.standard_normal(s) * 0.3 for s in ((f, d), (f, d), (d, f)))
    z = rng.standard_normal((7, d))
    L = ltp.ltp_structured_scores(z, wg, np.eye(f), wu, np.eye(f), np.eye(f), wd)
    ref = (F.silu(torch.from_numpy(z @ wg.T)) * torch.from_numpy(z @ wu.T)).numpy() @ wd.T
    assert np.allclose(L, np.linalg.norm(ref, axis=1), rtol=1e-12)


def test_structured_proxy_generator_full_rank():
    rng = np.random.default_rng(14)
    d, f, d_low = 64, 96, 32
    wg, wu, wd = (workloads.to_bf16(rng.standard_normal(s) * 0.05) for s in ((f, d), (f, d), (d, f)))
    sp = workloads.structured_proxy(wg, wu, wd, d_low, d_low, seed=3)
    ch = sp["channels"]
    assert len(ch) == d_low and np.all(np.diff(ch) > 0)
    f64 = workloads.as_f64
    # at rank d_low each factor pair reproduces the restricted map up to the bf16 storage of the factors
    for a, b, ref in ((sp["a_g_t"], sp["b_g_t"], f64(wg)[ch].T), (sp["a_u_t"], sp["b_u_t"], f64(wu)[ch].T),
                      (sp["c_t"], sp["d_t"], f64(wd)[:, ch].T)):
        rec = f64(a).T @ f64(b).T
        assert np.abs(rec - ref).max() <= 1e-2 * np.abs(ref).max()


def test_decode_of_token_n_is_row_n_of_dense_prefill():
    # two pre-norm RoPE layers, every token cached: decoding token N from the
    # N-token caches reproduces row N of a dense prefill over N + 1 tokens
    from oracle import decode
    sh = workloads.LayerShape(n=97, d=256, Hq=8, Hkv=2, dh=32, f=384, r=32, P=4)
    st = workloads.make_stack(sh, 2, seed=21)
    cfg = dict(Hq=8, Hkv=2, dh=32, P=4, keep_attn=1.0, keep_ffn=1.0, prenorm=True, eps=1e-5, theta=10000.0)
    ws = [{k: workloads.as_f64(v) for k, v in w.items() if hasattr(v, "numpy")} for w in st["layers"]]
    X = workloads.as_f64(st["x"])
    N = sh.n - 1
    full, pre = X, X[:N]
    caches = []
    for w in ws:
        full, _, _ = layer.spts_layer(full, np.arange(N + 1), w, cfg)
        pre, sa, _ = layer.spts_layer(pre, np.arange(N), w, cfg)
        caches.append([sa["K"], sa["V"]])
    out = decode.decode_step(X[N], N, caches, ws, cfg)
    assert np.allclose(out, full[N], rtol=0, atol=1e-9 * np.abs(full[N]).max())
    assert caches[0][0].shape == (N + 1, 2, 32) and caches[1][1].shape == (N + 1, 2, 32)


# ------------------------------------------------------------------------- FFN

def test_swiglu_against_torch():
    rng = np.random.default_rng(12)
    d, f = 64, 160
    z = numerics.bf16(rng.standard_normal((20, d)))
    wg, wu, wd = (numerics.bf16(rng.standard_normal(s) * 0.1) for s in ((f, d), (f, d), (d, f)))
    H, y = ffn.swiglu_rows(z, wg, wu, wd)
    zt = torch.from_numpy(z)
    ref = ((F.silu(zt @ torch.from_numpy(wg).T) * (zt @ torch.from_numpy(wu).T)) @ torch.from_numpy(wd).T).numpy()
    assert np.abs(y - ref).max() <= 1e-2 * np.abs(ref).max()
    assert np.array_equal(numerics.bf16(H), H) and np.array_equal(numerics.bf16(y), y)
    t = np.linspace(-20, 20, 101)
    assert np.allclose(ffn.silu(t), F.silu(torch.from_numpy(t)).numpy(), rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------- RMSNorm / RoPE

def test_rmsnorm_against_torch():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((7, 96)) * 3
    ref = F.rms_norm(torch.from_numpy(x), (96,), eps=1e-5).numpy()
    assert np.allclose(normrope.rmsnorm(x, 1e-5), ref, rtol=1e-13)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(14)
    rows, H, dh, theta = 6, 3, 16, 500000.0
    x = rng.standard_normal((rows, H, dh))
    pos = np.array([0, 1, 5, 100, 4095, 131071])
    got = normrope.rope(x, pos, theta)
    half = dh // 2
    zc = x[..., :half] + 1j * x[..., half:]
    freq = theta ** (-np.arange(half) * 2.0 / dh)
    rot = zc * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    assert np.allclose(got[..., :half], rot.real, atol=1e-12)
    assert np.allclose(got[..., half:], rot.imag, atol=1e-12)
    assert np.allclose(got[0], x[0], atol=0)        # position 0 is the identity
    q, k = x[:1], x[1:2]
    a = (normrope.rope(q, [7], theta) * normrope.rope(k, [3], theta)).sum()
    b = (normrope.rope(q, [1007], theta) * normrope.rope(k, [1003], theta)).sum()
    assert abs(a - b) < 1e-9                          # depends on the offset only


# --------------------------------------------------------------------- layers

def _small_weights(rng, d, Hq, Hkv, dh, f, r, std=0.05):
    b = numerics.bf16
    w = dict(wq=b(rng.standard_normal((Hq * dh, d)) * std),
             wk=b(rng.standard_normal((Hkv * dh, d)) * std),
             wv=b(rng.standard_normal((Hkv * dh, d)) * std),
             wo=b(rng.standard_normal((d, Hq * dh)) * std),
             wg=b(rng.standard_normal((f, d)) * std),
             wu=b(rng.standard_normal((f, d)) * std),
             wd=b(rng.standard_normal((d, f)) * std))
    u_t, v_t = workloads.proxy_factors(rng.standard_normal((d, d)) * std, r)
    w["u_t"], w["v_t"] = b(u_t), b(v_t)
    return w


def _dense_layer_torch(x, pos, w, cfg):
    """A dense LLaMA-style block written with torch library ops, float64."""
    Hq, Hkv, dh = cfg["Hq"], cfg["Hkv"], cfg["dh"]
    X = torch.from_numpy(x)
    T = {k: torch.from_numpy(v) for k, v in w.items()}
    xt = F.rms_norm(X, (X.shape[1],), eps=cfg["eps"]) if cfg.get("prenorm") else X
    q = (xt @ T["wq"].T).reshape(-1, Hq, dh).numpy()
    k = (xt @ T["wk"].T).reshape(-1, Hkv, dh).numpy()
    v = (xt @ T["wv"].T).reshape(-1, Hkv, dh).numpy()
    if cfg.get("theta") is not None:
        half = dh // 2
        fr = cfg["theta"] ** (-np.arange(half) * 2.0 / dh)
        rot = np.exp(1j * np.asarray(pos)[:, None, None] * fr[None, None, :])
        for a in (q, k):
            zc = (a[..., :half] + 1j * a[..., half:]) * rot
            a[..., :half], a[..., half:] = zc.real, zc.imag
    o = _sdpa_gqa(q, k, v, 1 / math.sqrt(dh)).reshape(len(x), -1)
    h = X + torch.from_numpy(o) @ T["wo"].T
    z = F.rms_norm(h, (h.shape[1],), eps=cfg["eps"]) if cfg.get("prenorm") else h
    y = (F.silu(z @ T["wg"].T) * (z @ T["wu"].T)) @ T["wd"].T
    return (h + y).numpy()


@pytest.mark.parametrize("prenorm", [False, True])
def test_layer_keep_all_is_dense(prenorm):
    rng = np.random.default_rng(15)
    n, d, Hq, Hkv, dh, f, r = 40, 64, 4, 2, 16, 96, 8
    w = _small_weights(rng, d, Hq, Hkv, dh, f, r)
    x = numerics.bf16(rng.standard_normal((n, d)))
    cfg = dict(Hq=Hq, Hkv=Hkv, dh=dh, P=4, keep_attn=1.0, keep_ffn=1.0, prenorm=prenorm,
               eps=1e-5, theta=10000.0 if prenorm else None)
    pos = np.arange(n)
    out, st_a, st_f = layer.spts_layer(x, pos, w, cfg)
    ref = _dense_layer_torch(x, pos, w, cfg)
    assert len(st_a["idx"]) == n and len(st_f["idx_f"]) == n
    assert np.abs(out - ref).max() <= 2e-2 * np.abs(ref).max()


def test_layer_skipped_rows_pass_through_bit_exact():
    rng = np.random.default_rng(16)
    n, d, Hq, Hkv, dh, f, r = 64, 64, 4, 2, 16, 96, 8
    w = _small_weights(rng, d, Hq, Hkv, dh, f, r)
    x = numerics.bf16(rng.standard_normal((n, d)))
    cfg = dict(Hq=Hq, Hkv=Hkv, dh=dh, P=4, keep_attn=0.35, keep_ffn=0.35)
    y, st_a = layer.attention_block(x, np.arange(n), w, cfg)
    skipped = np.setdiff1d(np.arange(n), st_a["idx"])
    assert len(st_a["idx"]) == numerics.keep_count(0.35, n)
    assert np.array_equal(y[skipped], x[skipped])
    assert not np.array_equal(y[st_a["idx"]], x[st_a["idx"]])
    assert set(range(n - 4, n)) <= set(st_a["idx"].tolist())
    out, st_f = layer.ffn_block(y, st_a["S"], w, cfg)
    skipped_f = np.setdiff1d(np.arange(n), st_f["idx_f"])
    assert np.array_equal(out[skipped_f], y[skipped_f])


def test_msdp_candidate_sets_are_nested():
    rng = np.random.default_rng(17)
    n, d, Hq, Hkv, dh, f, r = 96, 64, 4, 2, 16, 96, 8
    ws = [_small_weights(rng, d, Hq, Hkv, dh, f, r) for _ in range(6)]
    x0 = numerics.bf16(rng.standard_normal((n, d)))
    cfg = dict(Hq=Hq, Hkv=Hkv, dh=dh, P=4, keep_attn=0.35, keep_ffn=0.35, prenorm=True,
               eps=1e-5, theta=500000.0)
    pts = layer.prune_points(0, (1, 3, 5), (70, 50, 30))
    x, pos, hist = layer.msdp_stack(x0, ws, cfg, pts)
    counts = layer.candidate_counts(n, 6, pts)
    assert counts == [70, 70, 50, 50, 30, 30]
    prev = set(range(n))
    for hst, c in zip(hist, counts):
        cur = hst["pos"].tolist()
        assert len(cur) == c and cur == sorted(cur)
        assert set(cur) <= prev
        assert set(range(n - 4, n)) <= set(cur)
        prev = set(cur)
    assert x.shape == (30, d) and pos.tolist() == hist[-1]["pos"].tolist()


# --------------------------------------------------------------- page tables

def test_table5_kv_cache_reproduced():
    g = json.load(open(os.path.join(GOLDEN, "table5_kv_cache.json")))
    pts = layer.prune_points(g["first_skip_layer"], g["stage_end_layers"], g["budgets"], g["final_budget"])
    gib = 2.0 ** 30

    def half_up(v, nd):                      # the page rounds 4.125 to 4.13
        return math.floor(v * 10 ** nd + 0.5) / 10 ** nd

    for n, full, spts, saving in zip(g["context_tokens"], g["full_cache_gb"], g["spts_cache_gb"], g["saving_pct"]):
        f_b = costs.kv_cache_bytes(n, g["n_layers"], {})
        s_b = costs.kv_cache_bytes(n, g["n_layers"], pts)
        assert half_up(f_b / gib, 2) == full
        assert half_up(s_b / gib, 2) == spts
        assert half_up(100 * (1 - s_b / f_b), 1) == saving


def test_table_a_proxy_cost_reproduced():
    g = json.load(open(os.path.join(GOLDEN, "table_a_proxy_cost.json")))
    for row in g["rows"]:
        k = round(costs.proxy_macs(row["d_low"], row["rank"], g["d_model"]) / 1000)
        if row.get("garbled"):
            assert k != row["printed_k"]     # the page's value disagrees with every other row's rule
        else:
            assert k == row["printed_k"]
