"""Reduced attention over the selected queries -- test infrastructure only.

[SPTS] Fig. 2(a): the selected tokens take part in a reduced attention
computation.  This build's reading: each selected row i (an index into the
current candidate list) computes ordinary causal softmax attention against
the keys and values of ALL current candidate rows j <= i; skipped rows
compute nothing (their residual is left unchanged, [SPTS] Fig. 2 top).

  o_{i,h} = sum_{j <= i} softmax_j(tau * q_{i,h} . k_{j,g(h)}) v_{j,g(h)},
  g(h) = floor(h / (Hq/Hkv)).

With every row selected this is exactly dense causal attention.
"""

import numpy as np


def reduced_attention(q_sel, idx, k, v, scale, row_chunk=256):
    """q_sel [kq,Hq,dh], idx [kq] (row of each query), k/v [n,Hkv,dh] -> o [kq,Hq,dh]."""
    q_sel = np.asarray(q_sel, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    kq, Hq, dh = q_sel.shape
    n, Hkv, _ = k.shape
    if Hq % Hkv or idx.shape != (kq,) or (kq and (idx.min() < 0 or idx.max() >= n)):
        raise ValueError("reduced_attention: bad shapes or indices")
    group = Hq // Hkv
    o = np.zeros((kq, Hq, dh), dtype=np.float64)
    cols = np.arange(n)
    for c0 in range(0, kq, row_chunk):
        rows = idx[c0:c0 + row_chunk]
        hi = int(rows.max()) + 1
        causal = cols[None, :hi] <= rows[:, None]
        for h in range(Hq):
            g = h // group
            logits = scale * (q_sel[c0:c0 + row_chunk, h, :] @ k[:hi, g, :].T)
            logits = np.where(causal, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            a = e / e.sum(axis=1, keepdims=True)
            o[c0:c0 + row_chunk, h, :] = a @ v[:hi, g, :]
    return o
