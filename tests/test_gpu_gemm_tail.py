"""Parity of the projections when the launcher splits the last, partly
filled round of output tiles along k (equal pieces, or heads and ends) and a
second launch adds the fp32 pieces.  Shapes are chosen so each mode runs;
the host test test_gemm_split_plans pins which plan each shape gets.
Sampled rows (two per 256-row tile, plus the last row) are compared in full
with the oracle, so every output tile, split or not, is checked."""

import functools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import numerics, ffn, normrope
from free_token_skipping_amd import capi
from parity import np64, assert_close, BF16_REL

pytestmark = pytest.mark.gpu
DEV = "cuda"
THETA = 500000.0
TILE = 256 * 256 * 4


def _cuda(t):
    return t.to(DEV).contiguous()


def _log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=None)
def _mat(rows, cols, seed, std=1.0):
    return W.randn((rows, cols), seed=seed, std=std)


def _a(kd):
    """The shared activation matrix of a test at inner size kd."""
    return _mat(5200, 4096, 90) if kd == 4096 else _mat(2500, 8192, 92)


def _pick(m, seed):
    rng = np.random.default_rng(seed)
    rows = [int(rng.integers(t * 256, min(m, t * 256 + 256))) for t in range((m + 255) // 256) for _ in range(2)]
    return np.unique(np.array(rows + [m - 1]))


def _pos(n, seed):
    return torch.from_numpy(np.sort(np.random.default_rng(seed).choice(131072, n, replace=False)).astype(np.int32))


def _check_rows(got, ref, what):
    assert_close(got, ref, BF16_REL, what)
    ulp = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
    assert (ulp <= 2 ** -7).mean() > 0.995, what


@pytest.mark.parametrize("m,kd,n,plan", [(5161, 4096, 4096, 80 * 3), (2000, 4096, 8448, 8 * 32),
                                         (2227, 8192, 4096, 144 * 2)])
def test_tail_linear(m, kd, n, plan):
    _log(f"tail linear m={m} k={kd} n={n}")
    assert capi.lib().spts_linear_workspace(m, kd, n) == plan * TILE
    a = _a(kd)[:m]
    w = _mat(n, kd, 91, 0.02)
    out = capi.spts_linear(_cuda(a), _cuda(w))
    pick = _pick(m, 1)
    ref = numerics.bf16(W.as_f64(a[pick]) @ W.as_f64(w).T)
    _check_rows(np64(out)[pick], ref, "tail linear")


def test_tail_linear_gather_scatter_add():
    m, kd, n = 2227, 8192, 4096                       # heads and ends
    _log("tail linear, gathered rows, scatter-add")
    a = _a(kd)
    w = _mat(n, kd, 91, 0.02)
    rows = W.sorted_rows(2500, m, 8, seed=93)
    out_rows = W.sorted_rows(2600, m, 8, seed=94)
    resid = _mat(2600, n, 95)
    dst = _cuda(resid).clone()
    capi.spts_linear(_cuda(a), _cuda(w), a_rows=_cuda(rows), out=dst, out_rows=_cuda(out_rows), accumulate=True)
    pick = _pick(m, 2)
    r_in, r_out = rows.long().numpy()[pick], out_rows.long().numpy()[pick]
    ref = numerics.bf16(W.as_f64(resid)[r_out] + numerics.bf16(W.as_f64(a)[r_in] @ W.as_f64(w).T))
    _check_rows(np64(dst)[r_out], ref, "tail scatter-add")
    skipped = np.setdiff1d(np.arange(2600), out_rows.long().numpy())
    assert torch.equal(dst.cpu()[skipped], resid[skipped])


@pytest.mark.parametrize("m,n", [(5161, 4096), (2000, 8448)])
def test_tail_linear_rope_gather(m, n):
    kd = 4096
    _log(f"tail linear rope m={m} n={n}")
    a = _a(kd)
    w = _mat(n, kd, 96, 0.02)
    rows = W.sorted_rows(5200, m, 8, seed=97)
    pos = _pos(5200, 9)
    table = capi.spts_rope_table(131072, 128, THETA, DEV)
    out = capi.spts_linear_rope(_cuda(a), _cuda(w), _cuda(pos), table, a_rows=_cuda(rows))
    pick = _pick(m, 3)
    r = rows.long().numpy()[pick]
    acc = numerics.f32(W.as_f64(a)[r] @ W.as_f64(w).T).reshape(len(pick), n // 128, 128)
    ref = numerics.bf16(normrope.rope(acc, pos.numpy()[r], THETA)).reshape(len(pick), n)
    _check_rows(np64(out)[pick], ref, "tail rope")


@pytest.mark.parametrize("m,kd,plan", [(5161, 4096, 80 * 3), (2500, 8192, 160 * 2)])
def test_tail_swiglu_gather(m, kd, plan):
    f = 2048
    _log(f"tail swiglu m={m} k={kd} f={f}")
    assert capi.lib().spts_linear_swiglu_workspace(m, kd, f) == plan * TILE
    a = _a(kd)
    wg = _mat(f, kd, 98, 0.02)
    wu = _mat(f, kd, 99, 0.02)
    rows = W.sorted_rows(a.shape[0], m, 8, seed=100)
    h = capi.spts_linear_swiglu(_cuda(a), _cuda(wg), _cuda(wu), a_rows=_cuda(rows))
    pick = _pick(m, 4)
    z = W.as_f64(a)[rows.long().numpy()[pick]]
    g = numerics.f32(z @ W.as_f64(wg).T)
    u = numerics.f32(z @ W.as_f64(wu).T)
    _check_rows(np64(h)[pick], numerics.bf16(ffn.silu(g) * u), "tail swiglu")


@pytest.mark.parametrize("m,kd,plan", [(5161, 4096, 80 * 3), (2500, 8192, 160 * 2)])
def test_tail_kv_rope(m, kd, plan):
    nk = nv = 2048
    _log(f"tail kv m={m} k={kd}")
    assert capi.lib().spts_linear_kv_workspace(m, kd, nk, nv) == plan * TILE
    a = _a(kd)
    wk = _mat(nk, kd, 98, 0.02)
    wv = _mat(nv, kd, 99, 0.02)
    rows = W.sorted_rows(a.shape[0], m, 8, seed=101)
    pos = _pos(a.shape[0], 10)
    table = capi.spts_rope_table(131072, 128, THETA, DEV)
    k_out, v_out = capi.spts_linear_kv(_cuda(a), _cuda(wk), _cuda(wv), _cuda(pos), table, a_rows=_cuda(rows))
    pick = _pick(m, 5)
    r = rows.long().numpy()[pick]
    z = W.as_f64(a)[r]
    kacc = numerics.f32(z @ W.as_f64(wk).T).reshape(len(pick), nk // 128, 128)
    kref = numerics.bf16(normrope.rope(kacc, pos.numpy()[r], THETA)).reshape(len(pick), nk)
    _check_rows(np64(k_out)[pick], kref, "tail kv: K")
    _check_rows(np64(v_out)[pick], numerics.bf16(z @ W.as_f64(wv).T), "tail kv: V")


def test_tail_shape_without_workspace_runs_unsplit():
    """A caller that gives less workspace than the tail split needs gets the
    unsplit launch: same oracle bar, and the documented status."""
    import ctypes
    m, kd, n = 5161, 4096, 4096                       # 80 tail tiles in 3 pieces with room
    _log("tail shape, 1 MiB workspace")
    L = capi.lib()
    assert L.spts_linear_workspace(m, kd, n) > (1 << 20)
    a = _cuda(_a(kd)[:m])
    w = _cuda(_mat(n, kd, 91, 0.02))
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    h = ctypes.c_void_p()
    assert L.spts_create(ctypes.byref(h), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    try:
        assert L.spts_set_workspace(h, ctypes.c_void_p(ws.data_ptr()), ws.numel()) == 0
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        assert L.spts_linear(h, P(a), None, m, kd, P(w), n, P(out), None, 0) == 0
        assert L.spts_check(h) == 0
    finally:
        L.spts_destroy(h)
    pick = _pick(m, 6)
    ref = numerics.bf16(W.as_f64(_a(kd)[:m][pick]) @ W.as_f64(_mat(n, kd, 91, 0.02)).T)
    _check_rows(np64(out)[pick], ref, "unsplit fallback")
    split = capi.spts_linear(a, w)                     # with room: the tail split
    diff = (split.float() - out.float()).abs()
    assert diff.max().item() <= 2 ** -6 * out.float().abs().max().item()   # one bf16 rounding apart at most
