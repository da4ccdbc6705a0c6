"""Seeded synthetic inputs for the SPTS prefill workloads.

This module is shared by the tests, the benchmark and the smoke check.  It
draws inputs only; it holds none of the method's arithmetic (no score,
selection, attention, proxy or feed-forward computation).  Random numbers
come from numpy's default_rng(seed) in the fixed draw order documented on
each generator; bfloat16 rounding is torch's round-to-nearest-even cast.

The workloads stand in for the pages' LongBench runs on LLaMA-3.1-8B-Instruct
([SPTS] Tables 1, 4, 5): model shapes d=4096, Hq=32, Hkv=8, d_head=128,
SwiGLU 14336, at 8K/32K/128K tokens, with random weights N(0, 0.02^2) and
inputs N(0, 1).  No benchmark items or trained weights are used.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

LLAMA = dict(d=4096, Hq=32, Hkv=8, dh=128, f=14336)


@dataclass
class LayerShape:
    n: int
    d: int = 4096
    Hq: int = 32
    Hkv: int = 8
    dh: int = 128
    f: int = 14336
    r: int = 256
    P: int = 64


# The five workloads.  Sizes, ratios and seeds are those of the workload
# statement; where it is silent (probe count of the 32K layers, per-layer keep
# ratio inside MSDP stages) the values below are this build's reading.
CONFIGS = {
    "pap_tiny_fp32": dict(n=256, Hq=4, Hkv=4, dh=64, P=16, k=64, seed=0),
    "attn_layer_8k": dict(shape=LayerShape(n=8192, P=64), keep_attn=0.5, needles=64, seed=0),
    "layer_32k": dict(shape=LayerShape(n=32768, P=64), keep_attn=0.35, keep_ffn=0.35,
                      w_fuse=(0.5, 0.5), seed=0),
    "msdp_stack_32k": dict(shape=LayerShape(n=32768, P=64), layers=8, stage_ends=(1, 3, 5, 7),
                           budget_ratios=(0.6, 0.45, 0.35, 0.25), keep_attn=0.35,
                           keep_ffn=0.35, w_fuse=(0.5, 0.5), eps=1e-5, theta=500000.0, seed=0),
    "long_layer_128k": dict(shape=LayerShape(n=131072, P=128), keep_attn=0.25, keep_ffn=0.25,
                            w_fuse=(0.5, 0.5), centroids=256, sigma=0.3, needles=512,
                            prefix=16384, seed=0),
}


def to_bf16(a) -> torch.Tensor:
    """float array -> torch bfloat16 CPU tensor (torch's RNE cast)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """torch tensor (bf16 / fp32 / int) -> float64 numpy array, exactly."""
    return t.detach().cpu().to(torch.float64).numpy()


def _normal(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# ------------------------------------------------------------------ tiny PAP

def make_pap_tiny(n=256, Hq=4, Hkv=4, dh=64, seed=0):
    """Q, K, V [n, H, dh] float32, i.i.d. N(0,1)/sqrt(dh); drawn Q, K, V."""
    rng = np.random.default_rng(seed)
    s = 1.0 / np.sqrt(dh)
    q = _normal(rng, (n, Hq, dh), s)
    k = _normal(rng, (n, Hkv, dh), s)
    v = _normal(rng, (n, Hkv, dh), s)
    return dict(q=torch.from_numpy(q), k=torch.from_numpy(k), v=torch.from_numpy(v))


# ------------------------------------------------------------- proxy factors

def proxy_factors(m: np.ndarray, r: int):
    """Rank-r truncated SVD of M = A S B^T, split as U = A_r S_r, V = B_r^T.

    Returns float64 (u_t = U^T [r, d], v_t = V^T [d, r]).  Each left singular
    vector's largest-magnitude entry is made positive (sign convention).  For
    large d the top-r pairs come from a partial symmetric eigensolve of M M^T.
    """
    import scipy.linalg as sl
    m = np.asarray(m, dtype=np.float64)
    d = m.shape[0]
    if d <= 1024 or r == d:
        a, s, bt = np.linalg.svd(m)
        a, s, b = a[:, :r], s[:r], bt[:r].T
    else:
        w, a = sl.eigh(m @ m.T, subset_by_index=[d - r, d - 1], driver="evr")
        order = np.argsort(w)[::-1]
        w, a = w[order], a[:, order]
        s = np.sqrt(np.maximum(w, 0.0))
        b = (m.T @ a) / s[None, :]
    flip = np.sign(a[np.argmax(np.abs(a), axis=0), np.arange(a.shape[1])])
    a, b = a * flip, b * flip
    u_t = (a * s[None, :]).T          # [r, d]
    v_t = b                           # [d, r]
    return u_t, v_t


def structured_proxy(wg, wu, wd, d_low: int, r: int, seed: int = 0):
    """Factors of a structured proxy ([SPTS] Table A's form) built from one
    layer's own feed-forward weights -- a synthetic stand-in for the pages'
    channels chosen by saliency on calibration data.

    Draws d_low of the f hidden channels (sorted, without replacement, from
    default_rng(seed)); restricts gate, up and down to them; truncates each
    restricted map to rank r by SVD (largest-magnitude entry of each left
    singular vector made positive).  Returns bf16 tensors in nn.Linear
    layout: a_g_t, a_u_t [r, d]; b_g_t, b_u_t [d_low, r]; c_t [r, d_low];
    d_t [d, r]; plus the channel indices.
    """
    rng = np.random.default_rng(seed)
    wg64, wu64, wd64 = as_f64(wg), as_f64(wu), as_f64(wd)
    ch = np.sort(rng.choice(wg64.shape[0], d_low, replace=False))

    def factor(mp):
        # mp: the [in, out] map x -> x @ mp; returns W1 [r, in], W2 [out, r]
        p, s, qt = np.linalg.svd(mp, full_matrices=False)
        p, s, q = p[:, :r], s[:r], qt[:r].T
        flip = np.sign(p[np.argmax(np.abs(p), axis=0), np.arange(r)])
        return (p * (s * flip)[None, :]).T, q * flip[None, :]

    a_g_t, b_g_t = factor(wg64[ch].T)
    a_u_t, b_u_t = factor(wu64[ch].T)
    c_t, d_t = factor(wd64[:, ch].T)
    return dict(a_g_t=to_bf16(a_g_t), b_g_t=to_bf16(b_g_t), a_u_t=to_bf16(a_u_t), b_u_t=to_bf16(b_u_t),
                c_t=to_bf16(c_t), d_t=to_bf16(d_t), channels=ch)


# ------------------------------------------------------------ layer weights

def _draw_layer_weights(rng, sh: LayerShape, with_ffn: bool, with_wk: bool = True,
                        w_std: float = 0.02):
    """Draw order: Wq, Wk, Wv, Wo, then (FFN) Wg, Wu, Wd, M."""
    w = {}
    w["wq"] = _normal(rng, (sh.Hq * sh.dh, sh.d), w_std)
    if with_wk:
        w["wk"] = _normal(rng, (sh.Hkv * sh.dh, sh.d), w_std)
    w["wv"] = _normal(rng, (sh.Hkv * sh.dh, sh.d), w_std)
    w["wo"] = _normal(rng, (sh.d, sh.Hq * sh.dh), w_std)
    if with_ffn:
        w["wg"] = _normal(rng, (sh.f, sh.d), w_std)
        w["wu"] = _normal(rng, (sh.f, sh.d), w_std)
        w["wd"] = _normal(rng, (sh.d, sh.f), w_std)
        m = _normal(rng, (sh.d, sh.d), w_std).astype(np.float64)
        u_t, v_t = proxy_factors(m, sh.r)
        w["u_t"], w["v_t"] = u_t, v_t
    return {k: to_bf16(v) for k, v in w.items()}


def _probe_directions(x_bf16: torch.Tensor, wq_bf16: torch.Tensor, sh: LayerShape):
    """Per probe row and KV head, the sum of that group's probe queries
    (float64, from the bf16 inputs); used only to aim planted needle keys."""
    xp = as_f64(x_bf16[-sh.P:])
    wq = as_f64(wq_bf16)
    q = (xp @ wq.T).reshape(sh.P, sh.Hq, sh.dh)
    g = sh.Hq // sh.Hkv
    return q.reshape(sh.P, sh.Hkv, g, sh.dh).sum(axis=2)          # [P, Hkv, dh]


def _needle_targets(u, rms_norm, scale=4.0):
    """Key rows aimed along u with norm scale * rms_norm (per KV head)."""
    nrm = np.linalg.norm(u, axis=-1, keepdims=True)
    return scale * rms_norm[None, :, None] * u / nrm


def make_layer(sh: LayerShape, seed=0, with_ffn=True, needles=0, x_std=1.0,
               clustered_keys: Optional[Tuple[int, float]] = None):
    """Inputs of one bare SPTS layer.

    Draw order: X [n, d] ~ N(0, x_std^2); layer weights (see
    _draw_layer_weights; Wk is skipped when keys are sampled); then, for
    clustered keys, per KV head the centroids [C, dh] ~ N(0, 1), the
    assignments (uniform) and the noise N(0, sigma^2); then the needle
    positions (uniform without replacement from [0, n - P)).

    Needles (this build's reading of "keys aligned with the probe queries at
    scale 4x"): needle j is aimed at probe p = j mod P; for each KV head g its
    key is 4 * rho_g * u/|u|, with u the sum of the group's probe queries and
    rho_g the RMS norm of that head's ordinary keys.  With projected keys the
    needle's input row X[j] is replaced by the minimum-norm row whose key
    projection equals that target; with sampled keys the key row itself is
    replaced.
    """
    rng = np.random.default_rng(seed)
    x = to_bf16(_normal(rng, (sh.n, sh.d), x_std))
    w = _draw_layer_weights(rng, sh, with_ffn, with_wk=clustered_keys is None)
    out = dict(x=x, **w)
    k_sampled = None
    if clustered_keys is not None:
        n_cent, sigma = clustered_keys
        k_sampled = np.empty((sh.n, sh.Hkv, sh.dh), dtype=np.float32)
        for g in range(sh.Hkv):
            cent = _normal(rng, (n_cent, sh.dh), 1.0)
            assign = rng.integers(0, n_cent, size=sh.n)
            noise = _normal(rng, (sh.n, sh.dh), sigma)
            k_sampled[:, g, :] = cent[assign] + noise
    pos = None
    if needles:
        pos = np.sort(rng.choice(sh.n - sh.P, size=needles, replace=False))
        u = _probe_directions(x, w["wq"], sh)                       # [P, Hkv, dh]
        if k_sampled is not None:
            rho = np.sqrt((k_sampled.astype(np.float64) ** 2).sum(-1).mean(0))   # [Hkv]
            tgt = _needle_targets(u[np.arange(needles) % sh.P], rho)
            k_sampled[pos] = tgt.astype(np.float32)
        else:
            wk = as_f64(w["wk"])                                     # [Hkv*dh, d]
            sample = as_f64(x[: min(sh.n, 1024)])
            ks = (sample @ wk.T).reshape(-1, sh.Hkv, sh.dh)
            rho = np.sqrt((ks ** 2).sum(-1).mean(0))                # [Hkv]
            tgt = _needle_targets(u[np.arange(needles) % sh.P], rho).reshape(needles, -1)
            # minimum-norm preimage: x = Wk^T (Wk Wk^T)^-1 t
            coef = np.linalg.solve(wk @ wk.T, tgt.T)                 # [Hkv*dh, needles]
            xn = (wk.T @ coef).T                                     # [needles, d]
            xf = x.to(torch.float32)
            xf[torch.from_numpy(pos)] = torch.from_numpy(xn.astype(np.float32))
            x = xf.to(torch.bfloat16)
            out["x"] = x
        out["needle_pos"] = torch.from_numpy(pos.astype(np.int64))
    if k_sampled is not None:
        out["k"] = to_bf16(k_sampled)
    return out


def make_stack(sh: LayerShape, layers: int, seed=0, x_std=1.0):
    """Inputs of an MSDP stack: X [N, d] ~ N(0,1), then each layer's weights
    in layer order (each drawn as in _draw_layer_weights, with its own M)."""
    rng = np.random.default_rng(seed)
    x = to_bf16(_normal(rng, (sh.n, sh.d), x_std))
    ws = [_draw_layer_weights(rng, sh, with_ffn=True) for _ in range(layers)]
    return dict(x=x, layers=ws)


def randn(shape, seed=0, std=1.0, bf16=True):
    """One tensor of i.i.d. N(0, std^2) draws (bf16 by default, else fp32)."""
    x = _normal(np.random.default_rng(seed), tuple(shape), std)
    return to_bf16(x) if bf16 else torch.from_numpy(x)


def clustered_keys(n, Hkv, dh, n_centroids=256, sigma=0.3, seed=0):
    """Keys [n, Hkv, dh] (bf16): per KV head, n_centroids centroids ~ N(0, I)
    and each key = a uniformly drawn centroid + N(0, sigma^2 I).
    Draw order per head: centroids, assignments, noise."""
    rng = np.random.default_rng(seed)
    k = np.empty((n, Hkv, dh), dtype=np.float32)
    for g in range(Hkv):
        cent = _normal(rng, (n_centroids, dh), 1.0)
        assign = rng.integers(0, n_centroids, size=n)
        k[:, g, :] = cent[assign] + _normal(rng, (n, dh), sigma)
    return to_bf16(k)


def sorted_rows(n, k, n_forced, seed=0):
    """k ascending distinct rows of [0, n) that include the last n_forced
    (a stand-in selection for per-op tests); int32 tensor."""
    rng = np.random.default_rng(seed)
    free = rng.choice(n - n_forced, size=k - n_forced, replace=False)
    rows = np.sort(np.concatenate([free, np.arange(n - n_forced, n)]))
    return torch.from_numpy(rows.astype(np.int32))


def make_scores(n, seed=0, ties=0, dist="exp"):
    """Synthetic non-negative fp32 score vectors for selection tests.

    dist "exp": Exp(1) draws; "few": values from a small set of 8 (many ties);
    "few3": 3 values; "band": 70 % of the rows in [1, 1 + 2^-20) (distinct
    values packed into a narrow range), the rest in [2, 4).
    `ties` extra rows copy a random earlier row's value.
    """
    rng = np.random.default_rng(seed)
    if dist == "few":
        s = rng.integers(0, 8, size=n).astype(np.float32) / np.float32(4)
    elif dist == "few3":
        s = rng.integers(0, 3, size=n).astype(np.float32)
    elif dist == "band":
        dense = rng.random(size=n) < 0.7
        s = np.where(dense, 1.0 + rng.random(size=n) * 2.0 ** -20, 2.0 + 2.0 * rng.random(size=n)).astype(np.float32)
    else:
        s = rng.exponential(size=n).astype(np.float32)
    if ties and n > 1:
        dst = rng.integers(1, n, size=ties)
        src = (rng.random(size=ties) * dst).astype(np.int64)
        s[dst] = s[src]
    return torch.from_numpy(s)
