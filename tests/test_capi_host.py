"""The C-ABI library on the host: it loads, exports every function that
include/spts.h declares, and rejects bad arguments with the documented
status before launching anything.  No GPU is touched: every call below
fails validation (fake but aligned pointers never reach a kernel)."""

import ctypes
import os
import re

import pytest

from free_token_skipping_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spts.h")

OK, INVALID, SHAPE, DTYPE, ALIGN, NOMEM, HIP, UNSUPPORTED = range(8)
FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced
MIS = ctypes.c_void_p(0x10002)        # misaligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spts_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return capi.lib()


@pytest.fixture
def ctx(L):
    h = ctypes.c_void_p()
    assert L.spts_create(ctypes.byref(h), None) == OK
    yield h
    assert L.spts_destroy(h) == OK


def test_every_declared_function_is_exported(L):
    declared = header_functions()
    assert len(declared) >= 20
    assert sorted(capi.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_status_names(L):
    assert L.spts_status_name(SHAPE) == b"SPTS_ERR_SHAPE"
    assert L.spts_status_name(OK) == b"SPTS_OK"
    assert L.spts_create(None, None) == INVALID
    assert L.spts_destroy(None) == INVALID


def test_workspace_queries(L):
    assert L.spts_score_topk_workspace(32768) >= 32768 * 4
    assert L.spts_reduced_ffn_workspace(11469, 4096, 14336) >= 11469 * 14336 * 2
    assert L.spts_ltp_probe_workspace(100, 4096, 256) >= 100 * 512 * 2
    assert L.spts_probe_attention_workspace(0, 64, 32) == 0


def test_gemm_split_plans(L):
    """The split the GEMM launcher picks, read from the workspace it asks for:
    split-K into ks slices needs ks*m*n fp32, a tail split T*np fp32 tiles of
    256 x 256 (T tiles of the last, partly filled round over 256 CUs, each
    cut into np pieces).  Shapes are the MSDP stack's at 32K tokens."""
    tile = 256 * 256 * 4
    lin, kv, swi = L.spts_linear_workspace, L.spts_linear_kv_workspace, L.spts_linear_swiglu_workspace
    # FFN down projection, kept rows of the four stages (14336 -> 4096)
    assert lin(6881, 14336, 4096) == 176 * 2 * tile       # 432 tiles: heads and ends
    assert lin(5161, 14336, 4096) == 80 * 3 * tile        # 336 tiles: 3 equal pieces
    assert lin(4014, 14336, 4096) == 0                    # 256 tiles: one whole round
    assert lin(2867, 14336, 4096) == 192 * 2 * tile       # 192 tiles: heads and ends
    # Q / O projections (4096 -> 4096): only the 336-tile stage pays
    assert lin(6881, 4096, 4096) == 0
    assert lin(5161, 4096, 4096) == 80 * 3 * tile
    assert lin(2867, 4096, 4096) == 0
    assert lin(64, 4096, 4096) == 16 * 64 * 4096 * 4      # probe queries: split-K, 16 slices
    # gate/up (4096 -> 2 x 14336)
    assert swi(6881, 4096, 14336) == 0                    # 3024 tiles: the tail is nearly full
    assert swi(5161, 4096, 14336) == 48 * 5 * tile
    assert swi(2867, 4096, 14336) == 64 * 4 * tile
    # K/V over all candidates (4096 -> 1024 + 1024)
    assert kv(19661, 4096, 1024, 1024) == 104 * 2 * tile
    assert kv(32768, 4096, 1024, 1024) == 0
    assert kv(0, 4096, 1024, 1024) == 0 and swi(10, 4096, 0) == 0


def test_probe_validation(L, ctx):
    f = L.spts_probe_attention
    assert f(ctx, capi.BF16, None, FAKE, 100, 64, 32, 8, 128, 0.1, FAKE) == INVALID
    assert f(ctx, capi.BF16, FAKE, FAKE, 50, 64, 32, 8, 128, 0.1, FAKE) == SHAPE          # P > n
    assert f(ctx, capi.BF16, FAKE, FAKE, 100, 64, 30, 8, 128, 0.1, FAKE) == SHAPE         # Hq % Hkv
    assert f(ctx, capi.BF16, MIS, FAKE, 100, 64, 32, 8, 128, 0.1, FAKE) == ALIGN
    assert f(ctx, capi.BF16, FAKE, FAKE, 100, 64, 32, 8, 128, 0.1, FAKE) == NOMEM         # no workspace
    L.spts_set_workspace(ctx, FAKE, 1 << 30)
    assert f(ctx, capi.BF16, FAKE, FAKE, 100, 64, 32, 8, 64, 0.1, FAKE) == UNSUPPORTED    # dh
    assert f(ctx, capi.BF16, FAKE, FAKE, 100, 48, 32, 8, 128, 0.1, FAKE) == UNSUPPORTED   # P
    assert f(ctx, capi.BF16, FAKE, FAKE, 100, 64, 8, 8, 128, 0.1, FAKE) == UNSUPPORTED    # group of 1
    assert f(ctx, 7, FAKE, FAKE, 100, 64, 32, 8, 128, 0.1, FAKE) == DTYPE
    assert b"dtype" in L.spts_last_error(ctx)


def test_select_validation(L, ctx):
    f = L.spts_score_topk
    assert f(ctx, None, None, 0.5, 0.5, 10, 4, 1, FAKE, None) == INVALID
    assert f(ctx, FAKE, None, 0.5, 0.5, 10, 4, 5, FAKE, None) == SHAPE     # forced > k
    assert f(ctx, FAKE, None, 0.5, 0.5, 0, 0, 0, FAKE, None) == SHAPE      # n = 0
    assert f(ctx, FAKE, None, 0.5, 0.5, 10, 4, 1, FAKE, None) == NOMEM
    assert f(ctx, FAKE, MIS, 0.5, 0.5, 10, 4, 1, FAKE, None) == ALIGN
    na = L.spts_score_topk_noalloc
    assert na(ctx, None, None, 0.5, 0.5, 10, 4, 1, FAKE, None) == INVALID
    assert na(ctx, FAKE, None, 0.5, 0.5, 10, 4, 5, FAKE, None) == SHAPE
    assert na(ctx, FAKE, None, 0.5, 0.5, (1 << 20) + 1, 4, 1, FAKE, None) == UNSUPPORTED   # beyond its scratch
    assert b"static scratch" in L.spts_last_error(ctx)
    m = L.spts_score_topk_multiply
    assert m(ctx, FAKE, None, 10, 4, 1, FAKE, None) == INVALID            # s_b required
    assert m(ctx, FAKE, FAKE, 10, 4, 5, FAKE, None) == SHAPE
    assert m(ctx, FAKE, FAKE, 0, 0, 0, FAKE, None) == SHAPE
    assert m(ctx, FAKE, FAKE, 10, 4, 1, FAKE, None) == NOMEM
    assert m(ctx, FAKE, MIS, 10, 4, 1, FAKE, None) == ALIGN
    assert L.spts_msdp_stage(ctx, FAKE, 100, 120, 4, FAKE, FAKE, FAKE, None, None, 0) == SHAPE
    assert L.spts_msdp_stage(ctx, FAKE, 100, 50, 60, FAKE, FAKE, FAKE, None, None, 0) == SHAPE
    # more than 2^30 scores: row indices and grid strides of the selection stay in 32 bits
    big = (1 << 30) + 1
    assert f(ctx, FAKE, None, 0.5, 0.5, big, 4, 1, FAKE, None) == UNSUPPORTED
    assert b"at most 2^30" in L.spts_last_error(ctx)
    assert m(ctx, FAKE, FAKE, big, 4, 1, FAKE, None) == UNSUPPORTED
    assert L.spts_msdp_stage(ctx, FAKE, big, 50, 4, FAKE, FAKE, FAKE, None, None, 0) == UNSUPPORTED


def test_gemm_family_validation(L, ctx):
    assert L.spts_linear(ctx, FAKE, None, 100, 100, FAKE, 256, FAKE, None, 0) == UNSUPPORTED   # k % 64
    assert L.spts_linear(ctx, FAKE, None, 100, 128, FAKE, 200, FAKE, None, 0) == UNSUPPORTED   # n % 256
    assert L.spts_linear(ctx, FAKE, None, 100, 128, FAKE, 256, FAKE, None, 2) == INVALID
    assert L.spts_linear(ctx, None, None, 100, 128, FAKE, 256, FAKE, None, 0) == INVALID
    assert L.spts_linear(ctx, FAKE, None, 0, 128, FAKE, 256, FAKE, None, 0) == OK             # empty: no-op
    # a weight of 4 GiB or more is refused (the GEMM forms weight-row offsets in 32 bits)
    assert L.spts_linear(ctx, FAKE, None, 10, 4096, FAKE, 524288, FAKE, None, 0) == UNSUPPORTED
    assert L.spts_linear_swiglu(ctx, FAKE, None, 10, 8192, FAKE, FAKE, 262144, FAKE) == UNSUPPORTED
    assert L.spts_linear_kv(ctx, FAKE, None, 10, 8192, FAKE, 262144, FAKE, 256, FAKE, FAKE, None, None) == UNSUPPORTED
    assert L.spts_reduced_ffn(ctx, FAKE, None, FAKE, FAKE, FAKE, 10, 8192, 262144, FAKE, None, 0) == UNSUPPORTED
    assert L.spts_ltp_probe(ctx, FAKE, FAKE, FAKE, 10, 8388608, 256, FAKE) == UNSUPPORTED
    assert b"4 GiB" in L.spts_last_error(ctx)
    assert L.spts_ltp_probe(ctx, FAKE, FAKE, FAKE, 10, 4096, 100, FAKE) == UNSUPPORTED
    assert L.spts_ltp_probe(ctx, FAKE, FAKE, FAKE, 10, 4096, 256, FAKE) == NOMEM
    assert L.spts_reduced_ffn(ctx, FAKE, None, FAKE, FAKE, FAKE, 10, 4096, 100, FAKE, None, 0) == UNSUPPORTED
    assert L.spts_reduced_ffn(ctx, FAKE, None, FAKE, FAKE, FAKE, 10, 4096, 14336, FAKE, None, 0) == NOMEM
    assert L.spts_reduced_ffn(ctx, FAKE, None, FAKE, FAKE, FAKE, 0, 4096, 14336, FAKE, None, 0) == OK
    assert L.spts_rmsnorm(ctx, FAKE, 10, 12, 1e-5, FAKE) == SHAPE
    st = L.spts_ltp_probe_structured
    assert st(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 4096, 192, 512, FAKE) == UNSUPPORTED   # r % 256
    assert st(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 4096, 256, 300, FAKE) == UNSUPPORTED   # d_low % 256
    assert st(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 4096, 256, 512, FAKE) == NOMEM
    assert st(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4096, 256, 512, FAKE) == OK             # empty
    assert st(ctx, FAKE, None, FAKE, FAKE, FAKE, FAKE, 10, 4096, 256, 512, FAKE) == INVALID
    assert L.spts_ltp_structured_workspace(100, 4096, 256, 512) > 0
    kv = L.spts_linear_kv
    assert kv(ctx, FAKE, None, 100, 128, FAKE, 1024, FAKE, 200, FAKE, FAKE, None, None) == UNSUPPORTED  # nv % 256
    assert kv(ctx, FAKE, None, 100, 96, FAKE, 1024, FAKE, 1024, FAKE, FAKE, None, None) == UNSUPPORTED   # k % 64
    assert kv(ctx, FAKE, None, 100, 128, FAKE, 0, FAKE, 1024, FAKE, FAKE, None, None) == SHAPE
    assert kv(ctx, FAKE, None, 100, 128, FAKE, 1024, FAKE, 1024, FAKE, FAKE, FAKE, None) == INVALID       # pos w/o table
    assert kv(ctx, FAKE, None, 100, 128, FAKE, 1024, FAKE, 1024, None, FAKE, None, None) == INVALID
    assert kv(ctx, FAKE, None, 0, 128, FAKE, 1024, FAKE, 1024, FAKE, FAKE, None, None) == OK             # empty: no-op


def test_ltp_gram_validation(L, ctx):
    """The Gram-form LTP calls: sizes, alignment, empty input, the workspace
    refusal, and the Gram operand's own size check."""
    g = L.spts_ltp_gram
    assert g(ctx, FAKE, 4096, 192, FAKE) == UNSUPPORTED                                # r % 256
    assert g(ctx, FAKE, 0, 256, FAKE) == SHAPE
    assert g(ctx, MIS, 4096, 256, FAKE) == ALIGN
    assert g(ctx, FAKE, 4096, 256, None) == INVALID
    assert g(ctx, FAKE, 8388608, 256, FAKE) == UNSUPPORTED                              # v_t of 4 GiB
    pg = L.spts_ltp_probe_gram
    assert pg(ctx, FAKE, FAKE, FAKE, 10, 4096, 100, FAKE) == UNSUPPORTED                 # r % 256
    assert pg(ctx, FAKE, FAKE, FAKE, 10, 1000, 256, FAKE) == UNSUPPORTED                 # d % 256
    assert pg(ctx, FAKE, FAKE, FAKE, -1, 4096, 256, FAKE) == SHAPE
    assert pg(ctx, FAKE, FAKE, FAKE, 0, 4096, 256, FAKE) == OK                           # empty: no-op
    assert pg(ctx, FAKE, FAKE, None, 10, 4096, 256, FAKE) == INVALID
    assert pg(ctx, FAKE, FAKE, MIS, 10, 4096, 256, FAKE) == ALIGN
    assert pg(ctx, FAKE, FAKE, FAKE, 10, 4096, 256, FAKE) == NOMEM                       # no workspace bound
    assert pg(ctx, FAKE, FAKE, FAKE, 10, 4096, 65536, FAKE) == UNSUPPORTED               # gram of 4 GiB x 3
    assert L.spts_ltp_gram_workspace(100, 4096, 256) >= 100 * 3 * 256 * 2 + 256 * 256 * 4
    assert L.spts_ltp_gram_workspace(0, 4096, 256) == 0
    sg = L.spts_ltp_probe_structured_gram
    assert sg(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 4096, 192, 512, FAKE) == UNSUPPORTED   # r % 256
    assert sg(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 4096, 256, 512, FAKE) == NOMEM
    assert sg(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4096, 256, 512, FAKE) == OK             # empty
    assert sg(ctx, FAKE, FAKE, FAKE, FAKE, FAKE, None, 10, 4096, 256, 512, FAKE) == INVALID


def test_attention_and_rows_validation(L, ctx):
    f = L.spts_reduced_attention
    assert f(ctx, capi.BF16, FAKE, FAKE, FAKE, FAKE, 10, 5, 32, 8, 128, 0.1, FAKE) == SHAPE   # kq > n
    assert f(ctx, capi.BF16, FAKE, FAKE, FAKE, FAKE, 5, 10, 32, 8, 64, 0.1, FAKE) == UNSUPPORTED
    assert f(ctx, capi.BF16, FAKE, FAKE, FAKE, FAKE, 0, 10, 32, 8, 128, 0.1, FAKE) == OK       # empty
    # K/V of 2^31 elements or more (32-bit staging offsets): refused before any launch
    assert f(ctx, capi.BF16, FAKE, FAKE, FAKE, FAKE, 5, 1 << 21, 32, 8, 128, 0.1, FAKE) == UNSUPPORTED
    assert f(ctx, capi.I32, FAKE, FAKE, FAKE, FAKE, 5, 10, 32, 8, 128, 0.1, FAKE) == DTYPE
    assert L.spts_gather(ctx, 9, FAKE, FAKE, 4, 8, FAKE) == DTYPE
    assert L.spts_gather(ctx, capi.BF16, FAKE, FAKE, 0, 8, FAKE) == OK
    assert L.spts_scatter(ctx, capi.BF16, FAKE, FAKE, 4, 8, FAKE, 3) == INVALID
    assert L.spts_scatter(ctx, capi.BF16, FAKE, MIS, 4, 8, FAKE, 1) == ALIGN


def test_select_batched_validation(L, ctx):
    b = L.spts_score_topk_batched
    assert b(ctx, FAKE, 32768, 4, 32769, 10, 1, FAKE, 16) == UNSUPPORTED                  # row too long
    assert b(ctx, FAKE, 100, 4, 100, 10, 11, FAKE, 16) == SHAPE                           # forced > k
    assert b(ctx, FAKE, 96, 4, 100, 10, 1, FAKE, 16) == SHAPE                             # stride < n
    assert b(ctx, FAKE, 100, 4, 100, 10, 1, FAKE, 9) == SHAPE                             # idx stride < k
    assert b(ctx, MIS, 100, 4, 100, 10, 1, FAKE, 16) == ALIGN
    assert b(ctx, None, 100, 4, 100, 10, 1, FAKE, 16) == INVALID
    assert b(ctx, None, 100, 0, 100, 10, 1, None, 16) == OK                               # empty batch


def test_decode_validation(L, ctx):
    assert L.spts_decode_linear(ctx, FAKE, FAKE, 4000, 64, FAKE, 0) == UNSUPPORTED        # kdim % 512
    assert L.spts_decode_linear(ctx, FAKE, FAKE, 32768, 64, FAKE, 0) == UNSUPPORTED       # kdim > 16384
    assert L.spts_decode_linear(ctx, FAKE, FAKE, 4096, 0, FAKE, 0) == SHAPE
    assert L.spts_decode_linear(ctx, FAKE, FAKE, 4096, 64, FAKE, 2) == INVALID
    assert L.spts_decode_linear(ctx, None, FAKE, 4096, 64, FAKE, 0) == INVALID
    assert L.spts_decode_linear(ctx, MIS, FAKE, 4096, 64, FAKE, 0) == ALIGN
    r = L.spts_decode_linear_rope
    assert r(ctx, FAKE, FAKE, 4096, 192, FAKE, 3, FAKE) == UNSUPPORTED                    # 128-wide heads
    assert r(ctx, FAKE, FAKE, 4096, 256, FAKE, -1, FAKE) == SHAPE
    assert r(ctx, FAKE, FAKE, 4096, 256, FAKE, 3, None) == INVALID
    assert L.spts_decode_swiglu(ctx, FAKE, None, FAKE, 4096, 256, FAKE) == INVALID
    assert L.spts_decode_swiglu(ctx, FAKE, FAKE, MIS, 4096, 256, FAKE) == ALIGN
    a = L.spts_decode_attention
    assert a(ctx, FAKE, FAKE, FAKE, 0, 32, 8, 128, 0.1, FAKE) == SHAPE                    # empty cache
    assert a(ctx, FAKE, FAKE, FAKE, 10, 32, 16, 128, 0.1, FAKE) == UNSUPPORTED            # group of 2
    assert a(ctx, FAKE, FAKE, FAKE, 10, 32, 8, 64, 0.1, FAKE) == UNSUPPORTED
    assert a(ctx, FAKE, FAKE, FAKE, 10, 32, 8, 128, 0.1, FAKE) == NOMEM                   # no workspace
    assert L.spts_decode_attention_workspace(32768, 32) >= 128 * 32 * 130 * 4
    L.spts_set_workspace(ctx, FAKE, 1 << 20)
    assert a(ctx, FAKE, MIS, FAKE, 10, 32, 8, 128, 0.1, FAKE) == ALIGN


def test_decode_step_validation(L, ctx):
    lay = (capi.DecodeLayer * 2)()
    for i in range(2):
        lay[i] = capi.DecodeLayer(*([FAKE] * 9), 100)
    lens = (ctypes.c_int * 2)(10, 99)
    f = L.spts_decode_step
    args = lambda **kw: dict(dict(x=FAKE, d=4096, pos=5, layers=lay, n=2, lens=lens, Hq=32, Hkv=8, dh=128, f=14336,
                                  eps=1e-5, pre=1, table=FAKE, rows=64, scale=0.1), **kw)
    call = lambda a: f(ctx, a["x"], a["d"], a["pos"], a["layers"], a["n"], a["lens"], a["Hq"], a["Hkv"], a["dh"],
                       a["f"], a["eps"], a["pre"], a["table"], a["rows"], a["scale"])
    assert call(args()) == NOMEM                                        # every check passed, no workspace
    assert call(args(d=4000)) == UNSUPPORTED
    assert call(args(Hkv=16)) == UNSUPPORTED
    assert call(args(pre=2)) == INVALID
    assert call(args(pos=64)) == SHAPE                                  # outside the RoPE table
    assert call(args(pos=64, table=None)) == NOMEM                      # no RoPE: no table bound
    assert call(args(x=MIS)) == ALIGN
    assert call(args(n=0, layers=None, lens=None)) == OK                # no layers: no-op
    lens[1] = 100                                                       # layer 1 full
    assert call(args()) == SHAPE
    assert b"layer 1" in L.spts_last_error(ctx)
    lens[1] = 50
    lay[1].w_up = None
    assert call(args()) == INVALID
    lay[1].w_up = MIS
    assert call(args()) == ALIGN
    assert list(lens) == [10, 50]                                       # unchanged on every error
    assert L.spts_decode_step_workspace(32769, 32, 14336) >= L.spts_decode_attention_workspace(32769, 32)


def test_product_path_has_no_cpu_fallback():
    """The binding refuses CPU tensors instead of computing on the host."""
    import torch
    with pytest.raises(ValueError):
        capi.spts_rmsnorm(torch.zeros(4, 8, dtype=torch.bfloat16))
