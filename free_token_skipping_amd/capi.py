"""Thin Python binding of libspts.so (the C ABI in include/spts.h).

Argument marshalling only: every function checks that its torch tensors sit
on the GPU with the dtype and contiguity the C call expects, passes their
device pointers and the current HIP stream, and raises SptsError on a
non-OK status.  All computation happens in the library's HIP kernels; there
is no CPU fallback -- without the built library every call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspts.so")

BF16, F32, I32 = 0, 1, 2
_DTYPE = {torch.bfloat16: BF16, torch.float32: F32, torch.int32: I32}

# Every function the header declares (checked against include/spts.h by the tests).
EXPORTS = [
    "spts_create", "spts_destroy", "spts_set_stream", "spts_set_workspace", "spts_last_error",
    "spts_status_name", "spts_check",
    "spts_probe_attention_workspace", "spts_score_topk_workspace", "spts_ltp_probe_workspace",
    "spts_reduced_ffn_workspace", "spts_msdp_stage_workspace", "spts_linear_workspace",
    "spts_linear_kv_workspace", "spts_linear_swiglu_workspace",
    "spts_ltp_structured_workspace", "spts_ltp_probe_structured",
    "spts_ltp_gram_workspace", "spts_ltp_gram", "spts_ltp_probe_gram", "spts_ltp_probe_structured_gram",
    "spts_decode_attention_workspace", "spts_decode_linear", "spts_decode_linear_rope", "spts_decode_swiglu",
    "spts_decode_attention", "spts_decode_step_workspace", "spts_decode_step",
    "spts_probe_attention", "spts_score_topk", "spts_score_topk_multiply", "spts_score_topk_batched",
    "spts_score_topk_noalloc", "spts_gather", "spts_scatter",
    "spts_reduced_attention", "spts_ltp_probe", "spts_reduced_ffn", "spts_msdp_stage",
    "spts_linear", "spts_linear_rope", "spts_linear_kv", "spts_linear_swiglu", "spts_rope_table",
    "spts_rmsnorm",
]

_c = ctypes
_P, _I, _F, _D, _SZ = _c.c_void_p, _c.c_int, _c.c_float, _c.c_double, _c.c_size_t
_SIGS = {
    "spts_create": (_I, [_c.POINTER(_P), _P]),
    "spts_destroy": (_I, [_P]),
    "spts_set_stream": (_I, [_P, _P]),
    "spts_set_workspace": (_I, [_P, _P, _SZ]),
    "spts_last_error": (_c.c_char_p, [_P]),
    "spts_status_name": (_c.c_char_p, [_I]),
    "spts_check": (_I, [_P]),
    "spts_probe_attention_workspace": (_SZ, [_I, _I, _I]),
    "spts_score_topk_workspace": (_SZ, [_I]),
    "spts_ltp_probe_workspace": (_SZ, [_I, _I, _I]),
    "spts_ltp_gram_workspace": (_SZ, [_I, _I, _I]),
    "spts_ltp_gram": (_I, [_P, _P, _I, _I, _P]),
    "spts_ltp_probe_gram": (_I, [_P, _P, _P, _P, _I, _I, _I, _P]),
    "spts_reduced_ffn_workspace": (_SZ, [_I, _I, _I]),
    "spts_msdp_stage_workspace": (_SZ, [_I]),
    "spts_linear_workspace": (_SZ, [_I, _I, _I]),
    "spts_linear_kv_workspace": (_SZ, [_I, _I, _I, _I]),
    "spts_linear_swiglu_workspace": (_SZ, [_I, _I, _I]),
    "spts_ltp_structured_workspace": (_SZ, [_I, _I, _I, _I]),
    "spts_decode_attention_workspace": (_SZ, [_I, _I]),
    "spts_decode_linear": (_I, [_P, _P, _P, _I, _I, _P, _I]),
    "spts_decode_linear_rope": (_I, [_P, _P, _P, _I, _I, _P, _I, _P]),
    "spts_decode_swiglu": (_I, [_P, _P, _P, _P, _I, _I, _P]),
    "spts_decode_attention": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P]),
    "spts_decode_step_workspace": (_SZ, [_I, _I, _I]),
    "spts_decode_step": (_I, [_P, _P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _F, _I, _P, _I, _F]),
    "spts_ltp_probe_structured": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "spts_ltp_probe_structured_gram": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "spts_probe_attention": (_I, [_P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "spts_score_topk": (_I, [_P, _P, _P, _F, _F, _I, _I, _I, _P, _P]),
    "spts_score_topk_multiply": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "spts_score_topk_noalloc": (_I, [_P, _P, _P, _F, _F, _I, _I, _I, _P, _P]),
    "spts_score_topk_batched": (_I, [_P, _P, _c.c_int64, _I, _I, _I, _I, _P, _c.c_int64]),
    "spts_gather": (_I, [_P, _I, _P, _P, _I, _I, _P]),
    "spts_scatter": (_I, [_P, _I, _P, _P, _I, _I, _P, _I]),
    "spts_reduced_attention": (_I, [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "spts_ltp_probe": (_I, [_P, _P, _P, _P, _I, _I, _I, _P]),
    "spts_reduced_ffn": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _I]),
    "spts_msdp_stage": (_I, [_P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _I]),
    "spts_linear": (_I, [_P, _P, _P, _I, _I, _P, _I, _P, _P, _I]),
    "spts_linear_rope": (_I, [_P, _P, _P, _I, _I, _P, _I, _P, _P, _P]),
    "spts_linear_kv": (_I, [_P, _P, _P, _I, _I, _P, _I, _P, _I, _P, _P, _P, _P]),
    "spts_linear_swiglu": (_I, [_P, _P, _P, _I, _I, _P, _P, _I, _P]),
    "spts_rope_table": (_I, [_P, _I, _I, _D, _P]),
    "spts_rmsnorm": (_I, [_P, _P, _I, _I, _F, _P]),
}

_lib = None


class SptsError(RuntimeError):
    def __init__(self, status, name, message):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name


def lib():
    """Load libspts.so, building it in-tree first if it is not there (hipcc
    for gfx950); raises if it cannot be built or loaded -- there is no
    fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build(verbose=False)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m free_token_skipping_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ------------------------------------------------------------------- context

class Context:
    """One spts_ctx bound to the current torch stream, with a growable
    workspace tensor (torch allocates it; the library only borrows it)."""

    def __init__(self):
        self.handle = _P()
        st = lib().spts_create(ctypes.byref(self.handle), None)
        if st != 0:
            raise SptsError(st, "spts_create", "failed")
        self.ws = None

    def __del__(self):
        try:
            if self.handle and _lib is not None:
                _lib.spts_destroy(self.handle)
        except Exception:
            pass

    def bind(self, ws_bytes=0, device=None):
        if device is None or torch.device(device).type != "cuda":
            raise ValueError("libspts works on GPU tensors only (got device %s)" % (device,))
        L = lib()
        stream = torch.cuda.current_stream(device).cuda_stream
        L.spts_set_stream(self.handle, _P(stream))
        if ws_bytes:
            if self.ws is None or self.ws.numel() < ws_bytes or self.ws.device != device:
                self.ws = torch.empty(int(ws_bytes), dtype=torch.uint8, device=device)
            _check(self, L.spts_set_workspace(self.handle, _P(self.ws.data_ptr()), self.ws.numel()), "workspace")
        return self.handle

    def check(self):
        _check(self, lib().spts_check(self.handle), "spts_check")


_ctxs = {}


def context():
    """The context of the current torch stream: each stream has its own, so
    calls on two streams never share a workspace."""
    key = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    ctx = _ctxs.get(key)
    if ctx is None:
        ctx = _ctxs[key] = Context()
    return ctx


def _check(ctx, status, what):
    if status != 0:
        L = lib()
        name = L.spts_status_name(status).decode()
        msg = L.spts_last_error(ctx.handle).decode() if ctx is not None else ""
        raise SptsError(status, name, f"{what}: {msg}")


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _P(t.data_ptr())


def _dt(t):
    if t.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


# -------------------------------------------------------------- entry points

def spts_probe_attention(q_probe, k, scale=None, scores=None):
    """q_probe [P,Hq,dh], k [n,Hkv,dh] (bf16 or fp32) -> scores [n] fp32."""
    P, Hq, dh = q_probe.shape
    n, Hkv, _ = k.shape
    scale = float(dh ** -0.5) if scale is None else float(scale)
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=k.device)
    ctx = context()
    h = ctx.bind(lib().spts_probe_attention_workspace(n, P, Hq), k.device)
    _check(ctx, lib().spts_probe_attention(h, _dt(k), _ptr(q_probe, k.dtype, "q_probe"), _ptr(k, name="k"),
                                           n, P, Hq, Hkv, dh, scale, _ptr(scores, torch.float32, "scores")),
           "spts_probe_attention")
    return scores


def spts_score_topk(s_a, k, n_forced, s_b=None, w_a=0.5, w_b=0.5, idx=None, fused_out=None):
    """Ascending int32 indices of the k kept rows (see include/spts.h)."""
    n = s_a.shape[0]
    if idx is None:
        idx = torch.empty(min(k, n), dtype=torch.int32, device=s_a.device)
    ctx = context()
    h = ctx.bind(lib().spts_score_topk_workspace(n), s_a.device)
    _check(ctx, lib().spts_score_topk(h, _ptr(s_a, torch.float32, "s_a"), _ptr(s_b, torch.float32, "s_b"),
                                      float(w_a), float(w_b), n, int(k), int(n_forced),
                                      _ptr(idx, torch.int32, "idx"), _ptr(fused_out, torch.float32, "fused_out")),
           "spts_score_topk")
    return idx


def spts_score_topk_noalloc(s_a, k, n_forced, idx, s_b=None, w_a=0.5, w_b=0.5, fused_out=None):
    """spts_score_topk without a workspace: the library's static per-GPU
    scratch holds the keys (n <= 1048576); idx (and fused_out) are the
    caller's.  Calls overlapping on one GPU race on that scratch."""
    n = s_a.shape[0]
    ctx = context()
    h = ctx.bind(0, s_a.device)
    _check(ctx, lib().spts_score_topk_noalloc(h, _ptr(s_a, torch.float32, "s_a"), _ptr(s_b, torch.float32, "s_b"),
                                              float(w_a), float(w_b), n, int(k), int(n_forced),
                                              _ptr(idx, torch.int32, "idx"),
                                              _ptr(fused_out, torch.float32, "fused_out")),
           "spts_score_topk_noalloc")
    return idx


def spts_score_topk_batched(s, k, n_forced, idx=None):
    """Top-k of every row of s [batch, n] fp32 (no fusion) in one launch -> idx [batch, min(k, n)] int32."""
    batch, n = s.shape
    kk = min(k, n)
    if idx is None:
        idx = torch.empty((batch, kk), dtype=torch.int32, device=s.device)
    ctx = context()
    h = ctx.bind(0, s.device)
    _check(ctx, lib().spts_score_topk_batched(h, _ptr(s, torch.float32, "s"), s.stride(0), batch, n, int(k),
                                              int(n_forced), _ptr(idx, torch.int32, "idx"), idx.stride(0)),
           "spts_score_topk_batched")
    return idx


def spts_score_topk_multiply(s_a, s_b, k, n_forced, idx=None, fused_out=None):
    """Top-k of the Multiply fusion fl(s_a * s_b), probes forced, ascending int32 indices."""
    n = s_a.shape[0]
    if idx is None:
        idx = torch.empty(min(k, n), dtype=torch.int32, device=s_a.device)
    ctx = context()
    h = ctx.bind(lib().spts_score_topk_workspace(n), s_a.device)
    _check(ctx, lib().spts_score_topk_multiply(h, _ptr(s_a, torch.float32, "s_a"), _ptr(s_b, torch.float32, "s_b"),
                                               n, int(k), int(n_forced), _ptr(idx, torch.int32, "idx"),
                                               _ptr(fused_out, torch.float32, "fused_out")),
           "spts_score_topk_multiply")
    return idx


def _row_elems(t):
    return int(t[0].numel()) if t.dim() > 1 else 1


def spts_gather(src, idx, dst=None):
    k = idx.shape[0]
    if dst is None:
        dst = torch.empty((k,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    ctx = context()
    h = ctx.bind(0, src.device)
    _check(ctx, lib().spts_gather(h, _dt(src), _ptr(src, name="src"), _ptr(idx, torch.int32, "idx"), k,
                                  _row_elems(src), _ptr(dst, src.dtype, "dst")), "spts_gather")
    return dst


def spts_scatter(src, idx, dst, accumulate=False):
    k = idx.shape[0]
    ctx = context()
    h = ctx.bind(0, dst.device)
    _check(ctx, lib().spts_scatter(h, _dt(dst), _ptr(src, dst.dtype, "src"), _ptr(idx, torch.int32, "idx"), k,
                                   _row_elems(dst), _ptr(dst, name="dst"), int(bool(accumulate))), "spts_scatter")
    return dst


def spts_reduced_attention(q_sel, idx, k, v, scale=None, o_sel=None):
    kq, Hq, dh = q_sel.shape
    n, Hkv, _ = k.shape
    scale = float(dh ** -0.5) if scale is None else float(scale)
    if o_sel is None:
        o_sel = torch.empty_like(q_sel)
    ctx = context()
    h = ctx.bind(0, k.device)
    _check(ctx, lib().spts_reduced_attention(h, _dt(k), _ptr(q_sel, k.dtype, "q_sel"), _ptr(idx, torch.int32, "idx"),
                                             _ptr(k, name="k"), _ptr(v, k.dtype, "v"), kq, n, Hq, Hkv, dh, scale,
                                             _ptr(o_sel, k.dtype, "o_sel")), "spts_reduced_attention")
    return o_sel


def spts_ltp_probe(z, u_t, v_t, score=None):
    n, d = z.shape
    r = u_t.shape[0]
    if score is None:
        score = torch.empty(n, dtype=torch.float32, device=z.device)
    ctx = context()
    h = ctx.bind(lib().spts_ltp_probe_workspace(n, d, r), z.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_ltp_probe(h, _ptr(z, bf, "z"), _ptr(u_t, bf, "u_t"), _ptr(v_t, bf, "v_t"), n, d, r,
                                     _ptr(score, torch.float32, "score")), "spts_ltp_probe")
    return score


def spts_ltp_gram(v_t, gram=None):
    """Offline Gram operand of the proxy's second factor: v_t [d, r] ->
    gram [r, 3r] bf16, rows [hi(G) | hi(G) | lo(G)] of G = V V^T."""
    d, r = v_t.shape
    if gram is None:
        gram = torch.empty(r, 3 * r, dtype=torch.bfloat16, device=v_t.device)
    ctx = context()
    h = ctx.bind(0, v_t.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_ltp_gram(h, _ptr(v_t, bf, "v_t"), d, r, _ptr(gram, bf, "gram")), "spts_ltp_gram")
    return gram


def spts_ltp_probe_gram(z, u_t, gram, score=None):
    """LTP score ||(z U) V|| per row as sqrt(t G t^T), t = z U, with the gram
    operand from spts_ltp_gram."""
    n, d = z.shape
    r = u_t.shape[0]
    if score is None:
        score = torch.empty(n, dtype=torch.float32, device=z.device)
    ctx = context()
    h = ctx.bind(lib().spts_ltp_gram_workspace(n, d, r), z.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_ltp_probe_gram(h, _ptr(z, bf, "z"), _ptr(u_t, bf, "u_t"), _ptr(gram, bf, "gram"), n, d,
                                          r, _ptr(score, torch.float32, "score")), "spts_ltp_probe_gram")
    return score


def pack_structured_proxy(a_g_t, b_g_t, a_u_t, b_u_t, c_t, d_t):
    """Arrange the structured proxy's factors (nn.Linear layout: a_g_t, a_u_t
    [r, d]; b_g_t, b_u_t [d_low, r]; c_t [r, d_low]; d_t [d, r]) in the block
    layout spts_ltp_probe_structured reads.  Layout only: concatenation and
    zero blocks."""
    z = torch.zeros_like(b_g_t)
    return {"a_gu_t": torch.cat([a_g_t, a_u_t], 0).contiguous(),
            "b_gate": torch.cat([b_g_t, z, b_g_t, z], 1).contiguous(),
            "b_up": torch.cat([z, b_u_t, z, b_u_t], 1).contiguous(),
            "c_t": c_t.contiguous(), "d_t": d_t.contiguous()}


def spts_ltp_probe_structured(z, packed, score=None, gram=None):
    """Structured LTP score ||(silu((zA_g)B_g) * ((zA_u)B_u)) C D|| per row;
    with gram (spts_ltp_gram of packed["d_t"]) the last factor enters through
    its Gram matrix (spts_ltp_probe_structured_gram)."""
    n, d = z.shape
    r = packed["c_t"].shape[0]
    d_low = packed["c_t"].shape[1]
    if score is None:
        score = torch.empty(n, dtype=torch.float32, device=z.device)
    ctx = context()
    h = ctx.bind(lib().spts_ltp_structured_workspace(n, d, r, d_low), z.device)
    bf = torch.bfloat16
    fn, name = ((lib().spts_ltp_probe_structured_gram, "spts_ltp_probe_structured_gram") if gram is not None
                else (lib().spts_ltp_probe_structured, "spts_ltp_probe_structured"))
    last = _ptr(gram, bf, "gram") if gram is not None else _ptr(packed["d_t"], bf, "d_t")
    _check(ctx, fn(h, _ptr(z, bf, "z"), _ptr(packed["a_gu_t"], bf, "a_gu_t"), _ptr(packed["b_gate"], bf, "b_gate"),
                   _ptr(packed["b_up"], bf, "b_up"), _ptr(packed["c_t"], bf, "c_t"), last, n, d, r, d_low,
                   _ptr(score, torch.float32, "score")), name)
    return score


def spts_decode_linear(x, w, out=None, accumulate=False):
    """One token row x [kdim] through w [n, kdim]; accumulate adds into out (residual)."""
    n, kdim = w.shape
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=x.device)
    ctx = context()
    h = ctx.bind(0, x.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_decode_linear(h, _ptr(x, bf, "x"), _ptr(w, bf, "w"), kdim, n, _ptr(out, bf, "out"),
                                         int(bool(accumulate))), "spts_decode_linear")
    return out


def spts_decode_linear_rope(x, w, pos, table, out=None):
    n, kdim = w.shape
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=x.device)
    ctx = context()
    h = ctx.bind(0, x.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_decode_linear_rope(h, _ptr(x, bf, "x"), _ptr(w, bf, "w"), kdim, n, _ptr(out, bf, "out"),
                                              int(pos), _ptr(table, torch.float32, "table")), "spts_decode_linear_rope")
    return out


def spts_decode_swiglu(x, w_gate, w_up, out=None):
    f, kdim = w_gate.shape
    if out is None:
        out = torch.empty(f, dtype=torch.bfloat16, device=x.device)
    ctx = context()
    h = ctx.bind(0, x.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_decode_swiglu(h, _ptr(x, bf, "x"), _ptr(w_gate, bf, "w_gate"), _ptr(w_up, bf, "w_up"),
                                         kdim, f, _ptr(out, bf, "out")), "spts_decode_swiglu")
    return out


class DecodeLayer(ctypes.Structure):
    """struct spts_decode_layer: one layer's weight and cache pointers."""
    _fields_ = [("wq", _P), ("wk", _P), ("wv", _P), ("wo", _P), ("w_gate", _P), ("w_up", _P), ("w_down", _P),
                ("k_cache", _P), ("v_cache", _P), ("cap", _I)]


def decode_layer_table(weights, k_caches, v_caches):
    """ctypes array of spts_decode_layer for layer l = 0 .. len(k_caches)-1,
    layer l taking weights[l % len(weights)] (dicts of bf16 GPU tensors
    wq, wk, wv, wo, wg, wu, wd) and caches [cap, Hkv, dh] bf16."""
    bf = torch.bfloat16
    arr = (DecodeLayer * len(k_caches))()
    for l, (kc, vc) in enumerate(zip(k_caches, v_caches)):
        w = weights[l % len(weights)]
        if kc.shape != vc.shape:
            raise ValueError("k and v caches differ in shape")
        arr[l] = DecodeLayer(_ptr(w["wq"], bf, "wq"), _ptr(w["wk"], bf, "wk"), _ptr(w["wv"], bf, "wv"),
                             _ptr(w["wo"], bf, "wo"), _ptr(w["wg"], bf, "wg"), _ptr(w["wu"], bf, "wu"),
                             _ptr(w["wd"], bf, "wd"), _ptr(kc, bf, "k_cache"), _ptr(vc, bf, "v_cache"),
                             int(kc.shape[0]))
    return arr


def spts_decode_step(x, pos, layer_table, lengths, Hq, Hkv, dh, f, eps, prenorm, rope_table=None, scale=None):
    """One whole decode step in one library call: x [d] bf16 (updated in place)
    through every layer of layer_table (decode_layer_table); lengths is a
    Python list of per-layer cache lengths, incremented on success."""
    d = x.shape[0]
    n = len(layer_table)
    if len(lengths) != n:
        raise ValueError("one cache length per layer")
    scale = float(dh ** -0.5) if scale is None else float(scale)
    lens = (ctypes.c_int * n)(*lengths)
    ctx = context()
    h = ctx.bind(lib().spts_decode_step_workspace(max(lengths) + 1 if n else 1, Hq, f), x.device)
    table_rows = rope_table.shape[0] if rope_table is not None else 0
    _check(ctx, lib().spts_decode_step(h, _ptr(x, torch.bfloat16, "x"), d, int(pos), layer_table, n, lens, Hq, Hkv,
                                       dh, f, float(eps), int(bool(prenorm)),
                                       _ptr(rope_table, torch.float32, "rope_table"), table_rows, scale),
           "spts_decode_step")
    lengths[:] = list(lens)
    return x


def spts_decode_attention(q, k_cache, v_cache, L, scale=None, o=None):
    """q [Hq, dh] against the first L rows of k_cache, v_cache [cap, Hkv, dh]."""
    Hq, dh = q.shape
    Hkv = k_cache.shape[1]
    scale = float(dh ** -0.5) if scale is None else float(scale)
    if o is None:
        o = torch.empty_like(q)
    ctx = context()
    h = ctx.bind(lib().spts_decode_attention_workspace(int(L), Hq), q.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_decode_attention(h, _ptr(q, bf, "q"), _ptr(k_cache, bf, "k_cache"),
                                            _ptr(v_cache, bf, "v_cache"), int(L), Hq, Hkv, dh, scale,
                                            _ptr(o, bf, "o")), "spts_decode_attention")
    return o


def spts_reduced_ffn(z, w_gate, w_up, w_down, rows=None, y=None, y_rows=None, accumulate=False):
    d = z.shape[1]
    f = w_gate.shape[0]
    k = rows.shape[0] if rows is not None else z.shape[0]
    if y is None:
        y = torch.empty((k, d), dtype=torch.bfloat16, device=z.device)
    ctx = context()
    h = ctx.bind(lib().spts_reduced_ffn_workspace(k, d, f), z.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_reduced_ffn(h, _ptr(z, bf, "z"), _ptr(rows, torch.int32, "rows"), _ptr(w_gate, bf, "w_gate"),
                                       _ptr(w_up, bf, "w_up"), _ptr(w_down, bf, "w_down"), k, d, f,
                                       _ptr(y, bf, "y"), _ptr(y_rows, torch.int32, "y_rows"),
                                       int(bool(accumulate))), "spts_reduced_ffn")
    return y


def spts_msdp_stage(scores, budget, n_forced, pos_prev, x_prev=None, keep=None, pos_new=None, x_new=None):
    n_prev = scores.shape[0]
    dev = scores.device
    if keep is None:
        keep = torch.empty(budget, dtype=torch.int32, device=dev)
    if pos_new is None:
        pos_new = torch.empty(budget, dtype=torch.int32, device=dev)
    d = 0
    if x_prev is not None:
        d = x_prev.shape[1]
        if x_new is None:
            x_new = torch.empty((budget, d), dtype=x_prev.dtype, device=dev)
    ctx = context()
    h = ctx.bind(lib().spts_msdp_stage_workspace(n_prev), dev)
    bf = torch.bfloat16
    _check(ctx, lib().spts_msdp_stage(h, _ptr(scores, torch.float32, "scores"), n_prev, int(budget), int(n_forced),
                                      _ptr(pos_prev, torch.int32, "pos_prev"), _ptr(keep, torch.int32, "keep"),
                                      _ptr(pos_new, torch.int32, "pos_new"), _ptr(x_prev, bf, "x_prev"),
                                      _ptr(x_new, bf, "x_new"), d), "spts_msdp_stage")
    return keep, pos_new, x_new


def spts_linear(a, w, a_rows=None, out=None, out_rows=None, accumulate=False):
    kdim = a.shape[1]
    n = w.shape[0]
    m = a_rows.shape[0] if a_rows is not None else a.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    ctx = context()
    h = ctx.bind(lib().spts_linear_workspace(m, kdim, n), a.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_linear(h, _ptr(a, bf, "a"), _ptr(a_rows, torch.int32, "a_rows"), m, kdim,
                                  _ptr(w, bf, "w"), n, _ptr(out, bf, "out"), _ptr(out_rows, torch.int32, "out_rows"),
                                  int(bool(accumulate))), "spts_linear")
    return out


def spts_linear_rope(a, w, pos, table, a_rows=None, out=None):
    kdim = a.shape[1]
    n = w.shape[0]
    m = a_rows.shape[0] if a_rows is not None else a.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    ctx = context()
    h = ctx.bind(lib().spts_linear_workspace(m, kdim, n), a.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_linear_rope(h, _ptr(a, bf, "a"), _ptr(a_rows, torch.int32, "a_rows"), m, kdim,
                                       _ptr(w, bf, "w"), n, _ptr(out, bf, "out"), _ptr(pos, torch.int32, "pos"),
                                       _ptr(table, torch.float32, "table")), "spts_linear_rope")
    return out


def spts_linear_kv(a, wk, wv, pos=None, table=None, a_rows=None):
    """K = RoPE(A Wk^T) (plain if table is None) and V = A Wv^T in one launch."""
    kdim = a.shape[1]
    nk, nv = wk.shape[0], wv.shape[0]
    m = a_rows.shape[0] if a_rows is not None else a.shape[0]
    k_out = torch.empty((m, nk), dtype=torch.bfloat16, device=a.device)
    v_out = torch.empty((m, nv), dtype=torch.bfloat16, device=a.device)
    ctx = context()
    h = ctx.bind(lib().spts_linear_kv_workspace(m, kdim, nk, nv), a.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_linear_kv(h, _ptr(a, bf, "a"), _ptr(a_rows, torch.int32, "a_rows"), m, kdim,
                                     _ptr(wk, bf, "wk"), nk, _ptr(wv, bf, "wv"), nv, _ptr(k_out, bf, "k_out"),
                                     _ptr(v_out, bf, "v_out"), _ptr(pos, torch.int32, "pos"),
                                     _ptr(table, torch.float32, "table")), "spts_linear_kv")
    return k_out, v_out


def spts_linear_swiglu(a, w_gate, w_up, a_rows=None, out=None):
    kdim = a.shape[1]
    f = w_gate.shape[0]
    m = a_rows.shape[0] if a_rows is not None else a.shape[0]
    if out is None:
        out = torch.empty((m, f), dtype=torch.bfloat16, device=a.device)
    ctx = context()
    h = ctx.bind(lib().spts_linear_swiglu_workspace(m, kdim, f), a.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_linear_swiglu(h, _ptr(a, bf, "a"), _ptr(a_rows, torch.int32, "a_rows"), m, kdim,
                                         _ptr(w_gate, bf, "w_gate"), _ptr(w_up, bf, "w_up"), f,
                                         _ptr(out, bf, "out")), "spts_linear_swiglu")
    return out


def spts_rope_table(max_pos, dh, theta, device, table=None):
    if table is None:
        table = torch.empty((max_pos, dh // 2, 2), dtype=torch.float32, device=device)
    ctx = context()
    h = ctx.bind(0, device)
    _check(ctx, lib().spts_rope_table(h, int(max_pos), int(dh), float(theta), _ptr(table, torch.float32, "table")),
           "spts_rope_table")
    return table


def spts_rmsnorm(x, eps=1e-5, out=None):
    n, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    ctx = context()
    h = ctx.bind(0, x.device)
    bf = torch.bfloat16
    _check(ctx, lib().spts_rmsnorm(h, _ptr(x, bf, "x"), n, d, float(eps), _ptr(out, bf, "out")), "spts_rmsnorm")
    return out
