"""Decode phase: one new token per step -- test infrastructure only.

[SPTS] Table 5 and Fig. A(c): after prefill each layer keeps the keys and
values of its own candidates (every token for a dense layer, the MSDP
candidate set for a skipping layer).  A generated token then runs through
every layer: its K and V are appended to that layer's cache, and its query
attends to every cached row (all of them precede it).  The block is the same
pre-norm LLaMA layer as the prefill stack, with the same storage points:
projections accumulate in float64, are rounded to fp32, rotated, then stored
as bf16; the attention output, the O projection, the residual, the SwiGLU
hidden state and the FFN output are bf16.

The reading that pins it: with every token cached (a dense prefill), the
decode of token N equals row N of a dense prefill over N + 1 tokens.
"""

import numpy as np

from .numerics import bf16
from .normrope import rmsnorm
from .attention import reduced_attention
from .ffn import swiglu_rows
from .layer import _proj


def decode_layer(x, pos, cache_k, cache_v, w, cfg):
    """x [d] residual of the new token (bf16 values) at original position pos;
    cache_k, cache_v [L, Hkv, dh] (keys already rotated at their positions).
    Returns (x_out [d], k_new [Hkv, dh], v_new [Hkv, dh])."""
    Hq, Hkv, dh = cfg["Hq"], cfg["Hkv"], cfg["dh"]
    theta = cfg.get("theta")
    eps = cfg.get("eps", 1e-5)
    x = np.asarray(x, dtype=np.float64)[None, :]
    p = np.array([pos], dtype=np.int64)
    xt = bf16(rmsnorm(x, eps)) if cfg.get("prenorm") else x
    q = _proj(xt, w["wq"], Hq, dh, p, theta)
    k = _proj(xt, w["wk"], Hkv, dh, p, theta)
    v = _proj(xt, w["wv"], Hkv, dh)
    K = np.concatenate([np.asarray(cache_k, dtype=np.float64), k], axis=0)
    V = np.concatenate([np.asarray(cache_v, dtype=np.float64), v], axis=0)
    L = K.shape[0] - 1
    O = bf16(reduced_attention(q, np.array([L]), K, V, 1.0 / np.sqrt(dh)))   # row L sees rows 0..L
    y = bf16(x + bf16(O.reshape(1, Hq * dh) @ np.asarray(w["wo"], dtype=np.float64).T))
    z = bf16(rmsnorm(y, eps)) if cfg.get("prenorm") else y
    _, f = swiglu_rows(z, w["wg"], w["wu"], w["wd"])
    out = bf16(y + f)
    return out[0], k[0], v[0]


def decode_step(x, pos, caches, layers_w, cfg):
    """The new token through every layer; caches is a list of [K, V] per layer,
    each extended in place (a new array) by the token's K and V."""
    for li, w in enumerate(layers_w):
        x, k, v = decode_layer(x, pos, caches[li][0], caches[li][1], w, cfg)
        caches[li][0] = np.concatenate([caches[li][0], k[None]], axis=0)
        caches[li][1] = np.concatenate([caches[li][1], v[None]], axis=0)
    return x
