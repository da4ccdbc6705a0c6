"""Per-call parity of the HIP library against the CPU oracle.

Both sides receive the same seeded inputs from `workloads`; the oracle never
sees a value produced by the GPU.  Small cases span several tiles and a
ragged tail and are compared element by element; full-size cases (the 32K
and 128K workloads) compare every output the oracle can afford, or sampled
rows computed one by one."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import numerics, pap, select, attention, ltp, ffn, normrope
from free_token_skipping_amd import capi
from parity import np64, assert_close, window_violations, BF16_REL, F32_REL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cuda(t):
    return t.to(DEV).contiguous()


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------------ PAP

@pytest.mark.parametrize("n,P,Hq,Hkv", [(1000, 64, 8, 2), (333, 32, 4, 1), (4096, 128, 8, 1)])
def test_probe_bf16_small(n, P, Hq, Hkv):
    _log(f"probe bf16 n={n} P={P} Hq={Hq} Hkv={Hkv}")
    q = W.randn((P, Hq, 128), seed=1, std=1.3)
    k = W.randn((n, Hkv, 128), seed=2, std=1.3)
    S = capi.spts_probe_attention(_cuda(q), _cuda(k))
    ref = pap.pap_scores(W.as_f64(q), W.as_f64(k), 128 ** -0.5)
    got = np64(S)
    assert_close(got, ref, F32_REL, "probe scores")
    assert abs(got.sum() - Hq * P) < 1e-3 * Hq * P


def test_probe_bf16_growing_logits():
    """Keys whose norm grows 30x along the sequence: the late logits pass an
    early reference by far more than 64 exp2 units (their weights overflow
    against it), so the kernel's reference has to move many times per chunk."""
    n, P, Hq, Hkv = 3000, 64, 8, 2
    _log(f"probe bf16 growing logits n={n}")
    q = W.randn((P, Hq, 128), seed=7, std=1.3)
    k = W.randn((n, Hkv, 128), seed=8, std=1.3)
    ramp = (1.0 + 30.0 * torch.arange(n, dtype=torch.float32) / n).view(n, 1, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    S = capi.spts_probe_attention(_cuda(q), _cuda(k))
    ref = pap.pap_scores(W.as_f64(q), W.as_f64(k), 128 ** -0.5)
    assert np.isfinite(np64(S)).all()
    assert_close(np64(S), ref, F32_REL, "probe scores, growing logits")


def test_probe_bf16_full_32k_and_select_window():
    n, P, Hq, Hkv = 32768, 64, 32, 8
    _log("probe bf16 full 32K")
    q = W.randn((P, Hq, 128), seed=3, std=1.28)
    k = W.randn((n, Hkv, 128), seed=4, std=1.28)
    S = capi.spts_probe_attention(_cuda(q), _cuda(k))
    ref = pap.pap_scores(W.as_f64(q), W.as_f64(k), 128 ** -0.5)
    assert_close(np64(S), ref, F32_REL, "probe scores 32K")
    k_a = numerics.keep_count(0.35, n)
    idx = capi.spts_score_topk(S, k_a, P)
    assert window_violations(ref, idx.cpu().numpy(), k_a, P) == 0


def test_probe_bf16_full_128k_clustered_and_select_window():
    n, P, Hq, Hkv = 131072, 128, 32, 8
    _log("probe bf16 full 128K clustered keys")
    q = W.randn((P, Hq, 128), seed=5, std=1.28)
    k = W.clustered_keys(n, Hkv, 128, 256, 0.3, seed=6)
    S = capi.spts_probe_attention(_cuda(q), _cuda(k))
    ref = pap.pap_scores(W.as_f64(q), W.as_f64(k), 128 ** -0.5)
    assert_close(np64(S), ref, F32_REL, "probe scores 128K")
    k_a = numerics.keep_count(0.25, n)
    idx = capi.spts_score_topk(S, k_a, P)
    assert window_violations(ref, idx.cpu().numpy(), k_a, P) == 0


@pytest.mark.parametrize("n,P", [(131072, 64), (100000, 128)])
def test_probe_bf16_long_chunks(n, P):
    """Chunks longer than 1024 keys: 131072 keys at 64 probes run 2048-key
    chunks (the limit at two workgroups per CU); 100000 keys at 128 probes run
    3136-key chunks, the last one partly filled."""
    Hq, Hkv = 32, 8
    _log(f"probe bf16 long chunks n={n} P={P}")
    q = W.randn((P, Hq, 128), seed=11, std=1.28)
    k = W.randn((n, Hkv, 128), seed=12, std=1.28)
    S = capi.spts_probe_attention(_cuda(q), _cuda(k))
    ref = pap.pap_scores(W.as_f64(q), W.as_f64(k), 128 ** -0.5)
    assert_close(np64(S), ref, F32_REL, "probe scores, long chunks")
    assert abs(float(np64(S).sum()) - Hq * P) < 1e-3 * Hq * P


def test_probe_f32_tiny_config():
    _log("probe fp32 tiny (N=256, 4 heads, d_head 64, P=16)")
    t = W.make_pap_tiny()
    P = 16
    qp = t["q"][-P:].contiguous()
    S = capi.spts_probe_attention(_cuda(qp), _cuda(t["k"]), scale=1 / 8)
    ref = pap.pap_scores(W.as_f64(qp), W.as_f64(t["k"]), 1 / 8)
    assert_close(np64(S), ref, F32_REL, "fp32 probe")
    idx = capi.spts_score_topk(S, 64, P)
    assert window_violations(ref, idx.cpu().numpy(), 64, P) == 0


# --------------------------------------------------------------------- select

@pytest.mark.parametrize("n,k,nf,dist,ties", [
    (1, 1, 1, "exp", 0), (2, 1, 0, "exp", 0), (17, 5, 2, "few", 0), (1000, 350, 64, "exp", 40),
    (1000, 999, 64, "few", 0), (1000, 64, 64, "exp", 0), (1000, 1000, 64, "exp", 0),
    (1000, 1200, 10, "exp", 0), (32768, 11469, 64, "exp", 500), (32768, 11469, 64, "few", 0),
    (131072, 32768, 128, "exp", 2000), (4097, 2049, 0, "few", 0),
    # more than 8192 keys share the threshold's first digit: workgroup passes finish
    (32768, 16384, 64, "band", 0), (32768, 16384, 64, "band", 300), (32768, 11469, 64, "few3", 0),
    (131072, 65536, 128, "band", 0),
    # each keys-per-lane width of the one-workgroup select (12, 16, 20, 24, 32), at its
    # smallest and largest n and at the MSDP stack's candidate counts
    (8193, 2868, 64, "exp", 30), (11469, 4014, 64, "exp", 100), (12288, 4300, 64, "few", 0),
    (12289, 4301, 64, "band", 0), (14746, 5161, 64, "exp", 200), (16384, 8192, 64, "band", 50),
    (19661, 6881, 64, "exp", 300), (20480, 10240, 64, "band", 0), (20481, 7168, 64, "few3", 0),
    (24576, 8602, 64, "exp", 0), (24577, 8602, 64, "band", 100),
    # above 32K scores a plain selection runs on many workgroups
    (32769, 11469, 64, "exp", 500), (40000, 10000, 0, "few", 0), (65536, 32768, 128, "band", 300),
    (50000, 64, 64, "exp", 0), (50000, 65, 64, "few3", 0), (70001, 70000, 64, "exp", 0),
    (70001, 80000, 64, "exp", 0), (100000, 25000, 128, "band", 0), (1048576, 262144, 128, "exp", 5000)])
def test_select_bit_exact(n, k, nf, dist, ties):
    _log(f"select n={n} k={k} nf={nf} {dist}")
    s = W.make_scores(n, seed=n + k, ties=ties, dist=dist)
    idx = capi.spts_score_topk(_cuda(s), k, nf)
    ref = select.select_topk(s.numpy(), k, nf)
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("n", [32769, 131072])
def test_select_many_workgroups_nan_zero(n):
    """NaN ranks lowest and -0 equals +0 on the many-workgroup path too."""
    s = W.make_scores(n, seed=7, ties=300, dist="exp")
    s[::97] = float("nan")
    s[::89] = -0.0
    s[::83] = 0.0
    for k in (n // 4, n - 2000):
        idx = capi.spts_score_topk(_cuda(s), k, 64)
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), select.select_topk(s.numpy(), k, 64))


def test_select_special_values():
    s = torch.tensor([float("nan"), 1.0, -0.0, 0.0, 5.0, 2.0, -1.0, float("inf")], dtype=torch.float32)
    for k, nf in [(3, 1), (5, 0), (4, 2)]:
        idx = capi.spts_score_topk(_cuda(s), k, nf)
        assert idx.cpu().numpy().tolist() == select.select_topk(s.numpy(), k, nf).tolist()


@pytest.mark.parametrize("n,k,nf,batch", [(1000, 350, 64, 5), (32768, 11469, 64, 3), (700, 900, 16, 2),
                                          (8193, 4097, 0, 4)])
def test_select_batched_bit_exact(n, k, nf, batch):
    _log(f"batched select n={n} k={k} nf={nf} batch={batch}")
    rows = [W.make_scores(n, seed=100 * b + n, ties=(b % 2) * 30, dist="exp" if b % 3 else "few") for b in range(batch)]
    s = torch.stack(rows)
    idx = capi.spts_score_topk_batched(_cuda(s), k, nf).cpu().numpy().astype(np.int64)
    assert idx.shape == (batch, min(k, n))
    for b in range(batch):
        assert np.array_equal(idx[b], select.select_topk(rows[b].numpy(), k, nf)), f"row {b}"


@pytest.mark.parametrize("n,k,nf,nan", [(1000, 350, 64, False), (32768, 11469, 64, False),
                                         (131072, 32768, 128, False), (1000, 350, 64, True),
                                         (131072, 32768, 128, True), (19661, 6881, 64, False),
                                         (14746, 5161, 64, True), (11469, 4014, 64, False),
                                         (40000, 39000, 64, True), (65537, 70000, 64, True)])
def test_select_fused_bit_exact(n, k, nf, nan):
    # n > 32768 runs on many workgroups, the maxima in a pass of their own; k >= n
    # still writes every fused score
    _log(f"fused select n={n} nan={nan}")
    a = W.make_scores(n, seed=7)
    b = W.make_scores(n, seed=8) * 1e-3
    b[5] = b[9]                                            # a tie in the second score
    if nan:                                                # NaN in each score: the maxima skip it
        a[3] = float("nan")
        b[n // 2] = float("nan")
    fused = torch.empty(n, dtype=torch.float32, device=DEV)
    idx = capi.spts_score_topk(_cuda(a), k, nf, s_b=_cuda(b), w_a=0.5, w_b=0.5, fused_out=fused)
    ref_c = select.fuse_maxnorm(a.numpy(), b.numpy(), 0.5, 0.5)
    assert np.array_equal(fused.cpu().numpy(), ref_c, equal_nan=True)
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), select.select_topk(ref_c, k, nf))


@pytest.mark.parametrize("n,k,nf", [(1000, 350, 64), (32768, 11469, 64), (19661, 6881, 64),
                                    (131072, 32768, 128), (50000, 64, 64)])
def test_select_multiply_bit_exact(n, k, nf):
    _log(f"multiply select n={n}")
    a = W.make_scores(n, seed=9)
    b = W.make_scores(n, seed=10) * 3.0
    b[5] = b[9]
    a[11] = 0.0                                            # a zero factor
    fused = torch.empty(n, dtype=torch.float32, device=DEV)
    idx = capi.spts_score_topk_multiply(_cuda(a), _cuda(b), k, nf, fused_out=fused)
    ref_c = select.fuse_multiply(a.numpy(), b.numpy())
    assert np.array_equal(fused.cpu().numpy(), ref_c)
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), select.select_topk(ref_c, k, nf))


# ------------------------------------------------------------ gather / scatter

# 1040-byte, 3 KiB, 8 KiB and 16 KiB rows (1, 1, 2 and 4 units of 16 bytes per
# thread and row; 4, 4, 2 and 1 rows per workgroup), and 24 KiB rows (grid-stride)
@pytest.mark.parametrize("width", [520, 1536, 4096, 8192, 12296])
def test_gather_scatter_bit_exact(width):
    _log(f"gather / scatter width={width}")
    x = W.randn((777, width), seed=9)
    idx = W.sorted_rows(777, 301, 16, seed=10)
    g = capi.spts_gather(_cuda(x), _cuda(idx))
    assert torch.equal(g.cpu(), x[idx.long()])
    src = W.randn((301, width), seed=11)
    dst = _cuda(x).clone()
    capi.spts_scatter(_cuda(src), _cuda(idx), dst, accumulate=False)
    ref = x.clone()
    ref[idx.long()] = src
    assert torch.equal(dst.cpu(), ref)
    dst = _cuda(x).clone()
    capi.spts_scatter(_cuda(src), _cuda(idx), dst, accumulate=True)
    ref = W.as_f64(x).copy()
    ref[idx.long().numpy()] = numerics.bf16(ref[idx.long().numpy()] + W.as_f64(src))
    assert np.array_equal(np64(dst), ref)                  # one bf16 rounding of the fp32 sum
    skipped = np.setdiff1d(np.arange(777), idx.numpy())
    assert torch.equal(dst.cpu()[skipped], x[skipped])
    # 4-byte rows (positions) and fp32 rows
    pos = torch.arange(777, dtype=torch.int32)
    assert torch.equal(capi.spts_gather(_cuda(pos), _cuda(idx)).cpu(), pos[idx.long()])
    f = W.randn((777, 3), seed=12, bf16=False)
    assert torch.equal(capi.spts_gather(_cuda(f), _cuda(idx)).cpu(), f[idx.long()])


# ----------------------------------------------------------- reduced attention

@pytest.mark.parametrize("n,kq,Hq,Hkv", [(1000, 350, 8, 2), (300, 300, 4, 1), (2500, 97, 8, 1), (1, 1, 4, 1), (65, 1, 8, 2), (129, 65, 32, 8)])
def test_reduced_attention_bf16(n, kq, Hq, Hkv):
    _log(f"reduced attention bf16 n={n} kq={kq}")
    q = W.randn((kq, Hq, 128), seed=13, std=1.3)
    k = W.randn((n, Hkv, 128), seed=14, std=1.3)
    v = W.randn((n, Hkv, 128), seed=15)
    idx = W.sorted_rows(n, kq, min(64, kq), seed=16)
    o = capi.spts_reduced_attention(_cuda(q), _cuda(idx), _cuda(k), _cuda(v))
    ref = attention.reduced_attention(W.as_f64(q), idx.numpy(), W.as_f64(k), W.as_f64(v), 128 ** -0.5)
    assert_close(np64(o), ref, BF16_REL, "attention")
    # also per row: every query row within the bf16 bar of its own scale
    per_row = np.abs(np64(o) - ref).max(axis=(1, 2)) / np.abs(ref).max(axis=(1, 2))
    assert per_row.max() <= BF16_REL


def test_reduced_attention_growing_logits():
    """Keys whose norm grows 30x along the sequence: later tiles' logits pass
    the softmax reference by far more than 64 exp2 units (their weights
    overflow against it), so the kernel moves its reference many times."""
    n, kq, Hq, Hkv = 3000, 700, 8, 2
    _log(f"reduced attention bf16 growing logits n={n} kq={kq}")
    q = W.randn((kq, Hq, 128), seed=17, std=1.3)
    k = W.randn((n, Hkv, 128), seed=18, std=1.3)
    ramp = (1.0 + 30.0 * torch.arange(n, dtype=torch.float32) / n).view(n, 1, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    v = W.randn((n, Hkv, 128), seed=19)
    idx = W.sorted_rows(n, kq, 64, seed=20)
    o = capi.spts_reduced_attention(_cuda(q), _cuda(idx), _cuda(k), _cuda(v))
    ref = attention.reduced_attention(W.as_f64(q), idx.numpy(), W.as_f64(k), W.as_f64(v), 128 ** -0.5)
    got = np64(o)
    assert np.isfinite(got).all()
    per_row = np.abs(got - ref).max(axis=(1, 2)) / np.abs(ref).max(axis=(1, 2))
    assert per_row.max() <= BF16_REL, per_row.max()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reduced_attention_unsorted_idx(dtype):
    """Query rows in shuffled order (and one row twice): each query's causal
    range follows its own row, on both dtypes."""
    n, kq, Hq, Hkv = 1500, 400, 8, 2
    _log(f"reduced attention {dtype}, shuffled rows")
    rows = W.sorted_rows(n, kq, 8, seed=80).numpy().copy()
    np.random.default_rng(81).shuffle(rows)
    rows[7] = rows[300]
    idx = torch.from_numpy(rows.astype(np.int32))
    bf = dtype == "bf16"
    dh = 128 if bf else 64
    q = W.randn((kq, Hq, dh), seed=82, std=1.3, bf16=bf)
    k = W.randn((n, Hkv, dh), seed=83, std=1.3, bf16=bf)
    v = W.randn((n, Hkv, dh), seed=84, bf16=bf)
    o = capi.spts_reduced_attention(_cuda(q), _cuda(idx), _cuda(k), _cuda(v))
    ref = attention.reduced_attention(W.as_f64(q), rows, W.as_f64(k), W.as_f64(v), dh ** -0.5)
    got = np64(o)
    tol = BF16_REL if bf else F32_REL
    per_row = np.abs(got - ref).max(axis=(1, 2)) / np.abs(ref).max(axis=(1, 2))
    assert per_row.max() <= tol, per_row.max()


def test_reduced_attention_full_32k_sampled():
    n, kq, Hq, Hkv = 32768, 11469, 32, 8
    _log("reduced attention bf16 full 32K (sampled rows)")
    q = W.randn((kq, Hq, 128), seed=17, std=1.28)
    k = W.randn((n, Hkv, 128), seed=18, std=1.28)
    v = W.randn((n, Hkv, 128), seed=19)
    idx = W.sorted_rows(n, kq, 64, seed=20)
    o = capi.spts_reduced_attention(_cuda(q), _cuda(idx), _cuda(k), _cuda(v))
    rows = np.unique(np.concatenate([np.random.default_rng(0).choice(kq, 48, replace=False),
                                     [0, 1, 63, 64, kq - 65, kq - 1]]))
    ref = attention.reduced_attention(W.as_f64(q)[rows], idx.numpy()[rows], W.as_f64(k), W.as_f64(v), 128 ** -0.5)
    assert_close(np64(o)[rows], ref, BF16_REL, "attention 32K sampled")


def test_reduced_attention_f32_tiny_config():
    _log("reduced attention fp32 tiny")
    t = W.make_pap_tiny()
    idx = W.sorted_rows(256, 64, 16, seed=21)
    qs = t["q"][idx.long()].contiguous()
    o = capi.spts_reduced_attention(_cuda(qs), _cuda(idx), _cuda(t["k"]), _cuda(t["v"]), scale=1 / 8)
    ref = attention.reduced_attention(W.as_f64(qs), idx.numpy(), W.as_f64(t["k"]), W.as_f64(t["v"]), 1 / 8)
    assert_close(np64(o), ref, F32_REL, "fp32 attention")


# --------------------------------------------------------------- projections

def _linear_ref(a, w):
    return numerics.bf16(W.as_f64(a) @ W.as_f64(w).T)


@pytest.mark.parametrize("m,kd,n", [(777, 512, 256), (256, 64, 512), (1, 128, 256), (300, 4096, 1024)])
def test_linear_plain(m, kd, n):
    _log(f"linear m={m} k={kd} n={n}")
    a = W.randn((m, kd), seed=22)
    w = W.randn((n, kd), seed=23, std=0.05)
    out = capi.spts_linear(_cuda(a), _cuda(w))
    ref = _linear_ref(a, w)
    assert_close(np64(out), ref, BF16_REL, "linear")
    ulp = np.abs(np64(out) - ref) / np.maximum(np.abs(ref), 1e-30)
    assert (ulp <= 2 ** -7).mean() > 0.999                 # almost all within one bf16 ulp


def test_linear_gather_scatter_accumulate():
    _log("linear with gathered rows and scatter-add")
    a = W.randn((900, 512), seed=24)
    w = W.randn((512, 512), seed=25, std=0.05)
    rows = W.sorted_rows(900, 333, 8, seed=26)
    out = capi.spts_linear(_cuda(a), _cuda(w), a_rows=_cuda(rows))
    ref = _linear_ref(a[rows.long()], w)
    assert_close(np64(out), ref, BF16_REL, "gathered linear")
    resid = W.randn((900, 512), seed=27)
    dst = _cuda(resid).clone()
    src = W.randn((333, 512), seed=28)
    capi.spts_linear(_cuda(src), _cuda(w), out=dst, out_rows=_cuda(rows), accumulate=True)
    r = rows.long().numpy()
    ref = W.as_f64(resid).copy()
    ref[r] = numerics.bf16(ref[r] + _linear_ref(src, w))
    assert_close(np64(dst), ref, BF16_REL, "scatter-add linear")
    skipped = np.setdiff1d(np.arange(900), r)
    assert torch.equal(dst.cpu()[skipped], resid[skipped])


def test_linear_rope():
    _log("linear + rope")
    m, kd, n, theta = 500, 256, 512, 500000.0
    a = W.randn((m, kd), seed=29)
    w = W.randn((n, kd), seed=30, std=0.05)
    pos = torch.from_numpy(np.sort(np.random.default_rng(1).choice(131072, m, replace=False)).astype(np.int32))
    table = capi.spts_rope_table(131072, 128, theta, DEV)
    out = capi.spts_linear_rope(_cuda(a), _cuda(w), _cuda(pos), table)
    acc = numerics.f32(W.as_f64(a) @ W.as_f64(w).T).reshape(m, n // 128, 128)
    ref = numerics.bf16(normrope.rope(acc, pos.numpy(), theta)).reshape(m, n)
    assert_close(np64(out), ref, BF16_REL, "linear rope")
    rows = W.sorted_rows(m, 100, 4, seed=31)
    out2 = capi.spts_linear_rope(_cuda(a), _cuda(w), _cuda(pos), table, a_rows=_cuda(rows))
    assert_close(np64(out2), ref[rows.long().numpy()], BF16_REL, "gathered linear rope")


@pytest.mark.parametrize("m,kd,n", [(64, 4096, 4096), (1, 64, 256), (65, 192, 512), (128, 4096, 1024),
                                    (17, 1024, 768), (129, 256, 512)])
def test_linear_few_rows(m, kd, n):
    """Few rows (the probe queries' shape, 64 or 128 rows): one partly
    filled 256-row tile, split along k with fp32 pieces."""
    _log(f"linear few rows m={m} k={kd} n={n}")
    a = W.randn((m, kd), seed=32)
    w = W.randn((n, kd), seed=33, std=0.05)
    out = capi.spts_linear(_cuda(a), _cuda(w))
    ref = _linear_ref(a, w)
    assert_close(np64(out), ref, BF16_REL, "few-rows linear")
    ulp = np.abs(np64(out) - ref) / np.maximum(np.abs(ref), 1e-30)
    assert (ulp <= 2 ** -7).mean() > 0.999


@pytest.mark.parametrize("m,kd,n", [(64, 4096, 4096), (128, 4096, 4096), (37, 512, 256), (1, 128, 256)])
def test_linear_rope_few_rows(m, kd, n):
    """RoPE on few rows (the probe queries' projection), through the
    split-K reduce's RoPE epilogue."""
    _log(f"linear rope few rows m={m} k={kd} n={n}")
    theta = 500000.0
    a = W.randn((m, kd), seed=34)
    w = W.randn((n, kd), seed=35, std=0.05)
    pos = torch.from_numpy(np.sort(np.random.default_rng(2).choice(131072, m, replace=False)).astype(np.int32))
    table = capi.spts_rope_table(131072, 128, theta, DEV)
    out = capi.spts_linear_rope(_cuda(a), _cuda(w), _cuda(pos), table)
    acc = numerics.f32(W.as_f64(a) @ W.as_f64(w).T).reshape(m, n // 128, 128)
    ref = numerics.bf16(normrope.rope(acc, pos.numpy(), theta)).reshape(m, n)
    assert_close(np64(out), ref, BF16_REL, "few-rows linear rope")
    ulp = np.abs(np64(out) - ref) / np.maximum(np.abs(ref), 1e-30)
    assert (ulp <= 2 ** -7).mean() > 0.995


@pytest.mark.parametrize("rope", [True, False])
def test_linear_kv(rope):
    _log(f"linear kv rope={rope}")
    m, kd, nk, nv, theta = 600, 256, 512, 256, 500000.0
    a = W.randn((m, kd), seed=70)
    wk = W.randn((nk, kd), seed=71, std=0.05)
    wv = W.randn((nv, kd), seed=72, std=0.05)
    pos = torch.from_numpy(np.sort(np.random.default_rng(7).choice(131072, m, replace=False)).astype(np.int32))
    table = capi.spts_rope_table(131072, 128, theta, DEV) if rope else None
    k_out, v_out = capi.spts_linear_kv(_cuda(a), _cuda(wk), _cuda(wv), _cuda(pos) if rope else None, table)
    kacc = numerics.f32(W.as_f64(a) @ W.as_f64(wk).T)
    kref = numerics.bf16(normrope.rope(kacc.reshape(m, nk // 128, 128), pos.numpy(), theta).reshape(m, nk)
                         if rope else kacc)
    vref = numerics.bf16(W.as_f64(a) @ W.as_f64(wv).T)
    assert_close(np64(k_out), kref, BF16_REL, "kv: K")
    assert_close(np64(v_out), vref, BF16_REL, "kv: V")
    rows = W.sorted_rows(m, 300, 4, seed=73)
    k2, v2 = capi.spts_linear_kv(_cuda(a), _cuda(wk), _cuda(wv), _cuda(pos) if rope else None, table,
                                 a_rows=_cuda(rows))
    r = rows.long().numpy()
    assert_close(np64(k2), kref[r], BF16_REL, "kv gathered: K")
    assert_close(np64(v2), vref[r], BF16_REL, "kv gathered: V")


def test_linear_full_size_sampled():
    m, kd, n = 11469, 4096, 4096
    _log("linear full size (sampled rows)")
    a = W.randn((32768, kd), seed=32)
    w = W.randn((n, kd), seed=33, std=0.02)
    rows = W.sorted_rows(32768, m, 64, seed=34)
    out = capi.spts_linear(_cuda(a), _cuda(w), a_rows=_cuda(rows))
    pick = np.random.default_rng(2).choice(m, 40, replace=False)
    ref = numerics.bf16(W.as_f64(a[rows.long()[pick]]) @ W.as_f64(w).T)
    assert_close(np64(out)[pick], ref, BF16_REL, "linear 32K sampled")


@pytest.mark.parametrize("d", [4096, 520, 12296])      # in registers, a partly filled group, past 8192 columns
def test_rmsnorm(d):
    x = W.randn((333, d), seed=35, std=2.0)
    out = capi.spts_rmsnorm(_cuda(x), 1e-5)
    ref = numerics.bf16(normrope.rmsnorm(W.as_f64(x), 1e-5))
    assert_close(np64(out), ref, BF16_REL, "rmsnorm")


def test_rope_table():
    t = capi.spts_rope_table(131072, 128, 500000.0, DEV).cpu().numpy().astype(np.float64)
    p = np.array([0, 1, 777, 131071])[:, None]
    c = np.arange(64)[None, :]
    ang = p * 500000.0 ** (-2.0 * c / 128)
    assert np.abs(t[p[:, 0], :, 0] - np.cos(ang)).max() < 1e-7
    assert np.abs(t[p[:, 0], :, 1] - np.sin(ang)).max() < 1e-7


# ------------------------------------------------------------------------ LTP

@pytest.mark.parametrize("n,d,r", [(1000, 512, 256), (300, 1024, 512)])
def test_ltp_probe(n, d, r):
    _log(f"ltp n={n} d={d} r={r}")
    z = W.randn((n, d), seed=36)
    m = np.random.default_rng(37).standard_normal((d, d)) * 0.02
    u_t, v_t = W.proxy_factors(m, r)
    u_t, v_t = W.to_bf16(u_t), W.to_bf16(v_t)
    L = capi.spts_ltp_probe(_cuda(z), _cuda(u_t), _cuda(v_t))
    ref = ltp.ltp_scores(W.as_f64(z), W.as_f64(u_t), W.as_f64(v_t))
    got = np64(L)
    assert_close(got, ref, F32_REL, "ltp")
    assert (np.abs(got - ref) / ref).max() < 2e-5         # per row, not only at the max


@pytest.mark.parametrize("n", [32768, 19661])          # the 32K input and the first MSDP stage
def test_ltp_full_size_sampled(n):
    d, r = 4096, 256
    _log(f"ltp full size n={n} (sampled rows)")
    z = W.randn((n, d), seed=38)
    u_t = W.randn((r, d), seed=39, std=0.3)
    v_t = W.randn((d, r), seed=40, std=0.06)
    L = capi.spts_ltp_probe(_cuda(z), _cuda(u_t), _cuda(v_t))
    pick = np.concatenate([np.random.default_rng(3).choice(n, 256, replace=False), [n - 1]])
    ref = ltp.ltp_scores(W.as_f64(z[pick]), W.as_f64(u_t), W.as_f64(v_t))
    got = np64(L)[pick]
    assert (np.abs(got - ref) / ref).max() < 2e-5


def test_ltp_gram_operand():
    """spts_ltp_gram: rows [hi | hi | lo] of G = V V^T, hi + lo within the
    two-term bf16 bound of G, G symmetric bit for bit."""
    d, r = 4096, 256
    v_t = W.randn((d, r), seed=41, std=0.06)
    g = capi.spts_ltp_gram(_cuda(v_t))
    torch.cuda.synchronize()
    gb = g.cpu()
    hi = gb[:, :r].float().numpy().astype(np.float64)
    assert torch.equal(gb[:, :r], gb[:, r:2 * r])
    lo = gb[:, 2 * r:].float().numpy().astype(np.float64)
    v = W.as_f64(v_t)
    ref = v.T @ v
    assert np.array_equal(hi, hi.T) and np.array_equal(lo, lo.T)
    scale = np.abs(ref).max()
    assert np.abs(hi + lo - ref).max() <= 2.0 ** -16 * scale
    assert np.all(np.abs(lo) <= 2.0 ** -8 * np.abs(hi) + 1e-30)


@pytest.mark.parametrize("n,d,r", [(1000, 512, 256), (300, 1024, 512), (1, 512, 256), (257, 768, 256)])
def test_ltp_probe_gram(n, d, r):
    """sqrt(t G t^T) against the oracle's ||(z U) V|| (ragged row tails, one
    row, two 256-column tiles of G at r = 512)."""
    _log(f"ltp gram n={n} d={d} r={r}")
    z = W.randn((n, d), seed=36)
    m = np.random.default_rng(37).standard_normal((d, d)) * 0.02
    u_t, v_t = W.proxy_factors(m, r)
    u_t, v_t = W.to_bf16(u_t), W.to_bf16(v_t)
    gram = capi.spts_ltp_gram(_cuda(v_t))
    L = capi.spts_ltp_probe_gram(_cuda(z), _cuda(u_t), gram)
    ref = ltp.ltp_scores(W.as_f64(z), W.as_f64(u_t), W.as_f64(v_t))
    got = np64(L)
    assert (np.abs(got - ref) / ref).max() < 2e-5


def test_ltp_probe_gram_zero_rows():
    """A zero row scores exactly 0 (no NaN from a form rounding below 0); an
    empty input is a no-op."""
    n, d, r = 600, 512, 256
    z = W.randn((n, d), seed=42)
    z[::7] = 0
    u_t = W.randn((r, d), seed=43, std=0.3)
    v_t = W.randn((d, r), seed=44, std=0.06)
    gram = capi.spts_ltp_gram(_cuda(v_t))
    got = np64(capi.spts_ltp_probe_gram(_cuda(z), _cuda(u_t), gram))
    assert np.all(got[::7] == 0.0)
    ref = ltp.ltp_scores(W.as_f64(z), W.as_f64(u_t), W.as_f64(v_t))
    keep = np.ones(n, bool)
    keep[::7] = False
    assert (np.abs(got[keep] - ref[keep]) / ref[keep]).max() < 2e-5
    e = capi.spts_ltp_probe_gram(_cuda(z[:0]), _cuda(u_t), gram)
    assert e.shape == (0,)


@pytest.mark.parametrize("n,factors", [(32768, "random"), (19661, "random"), (32768, "svd")])
def test_ltp_gram_full_size_sampled(n, factors):
    """The Gram form at the 32K input and the first MSDP stage, on random
    factors (G far from diagonal) and on the truncated-SVD proxy."""
    d, r = 4096, 256
    _log(f"ltp gram full size n={n} {factors} (sampled rows)")
    z = W.randn((n, d), seed=38)
    if factors == "random":
        u_t = W.randn((r, d), seed=39, std=0.3)
        v_t = W.randn((d, r), seed=40, std=0.06)
    else:
        m = np.random.default_rng(45).standard_normal((d, d)) * 0.02
        u_t, v_t = (W.to_bf16(a) for a in W.proxy_factors(m, r))
    gram = capi.spts_ltp_gram(_cuda(v_t))
    L = capi.spts_ltp_probe_gram(_cuda(z), _cuda(u_t), gram)
    pick = np.concatenate([np.random.default_rng(3).choice(n, 256, replace=False), [0, n - 1]])
    ref = ltp.ltp_scores(W.as_f64(z[pick]), W.as_f64(u_t), W.as_f64(v_t))
    got = np64(L)[pick]
    assert (np.abs(got - ref) / ref).max() < 2e-5


def _structured_case(n, d, f, d_low, r, seed):
    z = W.randn((n, d), seed=seed)
    wg = W.randn((f, d), seed=seed + 1, std=0.05)
    wu = W.randn((f, d), seed=seed + 2, std=0.05)
    wd = W.randn((d, f), seed=seed + 3, std=0.05)
    return z, W.structured_proxy(wg, wu, wd, d_low, r, seed=seed + 4)


_SP_KEYS = ("a_g_t", "b_g_t", "a_u_t", "b_u_t", "c_t", "d_t")


@pytest.mark.parametrize("form", ["direct", "gram"])
@pytest.mark.parametrize("n,d,f,d_low,r", [(1000, 512, 1024, 512, 256), (777, 1024, 2048, 256, 256),
                                           (300, 512, 1024, 512, 512)])
def test_ltp_structured(n, d, f, d_low, r, form):
    """Both forms of the last factor (D itself, or its Gram matrix D D^T)."""
    _log(f"structured ltp n={n} d={d} d_low={d_low} r={r} {form}")
    z, sp = _structured_case(n, d, f, d_low, r, seed=60)
    packed = capi.pack_structured_proxy(*[_cuda(sp[k]) for k in _SP_KEYS])
    gram = capi.spts_ltp_gram(packed["d_t"]) if form == "gram" else None
    L = capi.spts_ltp_probe_structured(_cuda(z), packed, gram=gram)
    ref = ltp.ltp_structured_scores(W.as_f64(z), *[W.as_f64(sp[k]) for k in _SP_KEYS])
    got = np64(L)
    assert_close(got, ref, F32_REL, "structured ltp")
    assert (np.abs(got - ref) / ref).max() < 5e-5          # per row: three hi/lo stages of ~16 bits


@pytest.mark.parametrize("form", ["direct", "gram"])
def test_ltp_structured_full_size_sampled(form):
    n, d, f, d_low, r = 32768, 4096, 14336, 512, 256
    _log(f"structured ltp full size (sampled rows) {form}")
    z, sp = _structured_case(n, d, f, d_low, r, seed=66)
    packed = capi.pack_structured_proxy(*[_cuda(sp[k]) for k in _SP_KEYS])
    gram = capi.spts_ltp_gram(packed["d_t"]) if form == "gram" else None
    L = capi.spts_ltp_probe_structured(_cuda(z), packed, gram=gram)
    pick = np.random.default_rng(4).choice(n, 128, replace=False)
    ref = ltp.ltp_structured_scores(W.as_f64(z[pick]), *[W.as_f64(sp[k]) for k in _SP_KEYS])
    got = np64(L)[pick]
    assert (np.abs(got - ref) / ref).max() < 5e-5


# ------------------------------------------------------------------------ FFN

@pytest.mark.parametrize("k,d,f", [(333, 512, 1024), (64, 256, 384)])
def test_reduced_ffn(k, d, f):
    _log(f"ffn k={k} d={d} f={f}")
    z = W.randn((k + 50, d), seed=41)
    wg = W.randn((f, d), seed=42, std=0.05)
    wu = W.randn((f, d), seed=43, std=0.05)
    wd = W.randn((d, f), seed=44, std=0.05)
    rows = W.sorted_rows(k + 50, k, 4, seed=45)
    y = capi.spts_reduced_ffn(_cuda(z), _cuda(wg), _cuda(wu), _cuda(wd), rows=_cuda(rows))
    H, ref = ffn.swiglu_rows(W.as_f64(z)[rows.long().numpy()], W.as_f64(wg), W.as_f64(wu), W.as_f64(wd))
    assert_close(np64(y), ref, BF16_REL, "ffn")
    # fused residual add into the selected rows
    h = _cuda(z).clone()
    capi.spts_reduced_ffn(h, _cuda(wg), _cuda(wu), _cuda(wd), rows=_cuda(rows), y=h, y_rows=_cuda(rows),
                          accumulate=True)
    r = rows.long().numpy()
    exp = W.as_f64(z).copy()
    exp[r] = numerics.bf16(exp[r] + ref)
    assert_close(np64(h), exp, BF16_REL, "ffn residual")
    skipped = np.setdiff1d(np.arange(k + 50), r)
    assert torch.equal(h.cpu()[skipped], z[skipped])


def test_reduced_ffn_full_size_sampled():
    k, d, f = 11469, 4096, 14336
    _log("ffn full size (sampled rows)")
    z = W.randn((k, d), seed=46)
    wg = W.randn((f, d), seed=47, std=0.02)
    wu = W.randn((f, d), seed=48, std=0.02)
    wd = W.randn((d, f), seed=49, std=0.02)
    y = capi.spts_reduced_ffn(_cuda(z), _cuda(wg), _cuda(wu), _cuda(wd))
    pick = np.random.default_rng(4).choice(k, 24, replace=False)
    _, ref = ffn.swiglu_rows(W.as_f64(z[pick]), W.as_f64(wg), W.as_f64(wu), W.as_f64(wd))
    assert_close(np64(y)[pick], ref, BF16_REL, "ffn 32K sampled")


# ----------------------------------------------------------------------- MSDP

def test_msdp_stage_bit_exact():
    _log("msdp stage")
    n, budget, P, d = 5000, 2999, 64, 512
    s = W.make_scores(n, seed=50, ties=100)
    pos = torch.from_numpy(np.sort(np.random.default_rng(5).choice(40000, n, replace=False)).astype(np.int32))
    x = W.randn((n, d), seed=51)
    keep, pos_new, x_new = capi.spts_msdp_stage(_cuda(s), budget, P, _cuda(pos), _cuda(x))
    ref = select.select_topk(s.numpy(), budget, P)
    assert np.array_equal(keep.cpu().numpy(), ref)
    assert np.array_equal(pos_new.cpu().numpy(), pos.numpy()[ref])
    assert torch.equal(x_new.cpu(), x[ref])


def test_linear_swiglu():
    _log("swiglu GEMM")
    a = W.randn((600, 512), seed=52)
    wg = W.randn((384, 512), seed=53, std=0.05)
    wu = W.randn((384, 512), seed=54, std=0.05)
    rows = W.sorted_rows(600, 301, 4, seed=55)
    h = capi.spts_linear_swiglu(_cuda(a), _cuda(wg), _cuda(wu), a_rows=_cuda(rows))
    z = W.as_f64(a)[rows.long().numpy()]
    g = numerics.f32(z @ W.as_f64(wg).T)
    u = numerics.f32(z @ W.as_f64(wu).T)
    ref = numerics.bf16(ffn.silu(g) * u)
    assert_close(np64(h), ref, BF16_REL, "swiglu GEMM")
