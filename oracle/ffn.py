"""Reduced SwiGLU feed-forward -- test infrastructure only.

[SPTS] Fig. 2(b): the tokens that LTP selects go through a reduced
feed-forward; the others skip it.  The workload's FFN is the LLaMA SwiGLU
block, 4096 -> 14336 -> 4096:

    H_i = silu(z_i Wg^T) * (z_i Wu^T),   silu(x) = x * sigmoid(x),
    y_i = H_i Wd^T.

Storage points (as on the GPU): the gate and up products are fp32
accumulators, silu and the product are evaluated on those, H is stored as
bfloat16, and y is stored as bfloat16.
"""

import numpy as np

from .numerics import bf16, f32


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu_rows(z_sel, w_gate, w_up, w_down):
    """z_sel [k,d], w_gate/w_up [f,d], w_down [d,f] -> (H [k,f], y [k,d]) float64."""
    z_sel = np.asarray(z_sel, dtype=np.float64)
    g = f32(z_sel @ np.asarray(w_gate, dtype=np.float64).T)
    u = f32(z_sel @ np.asarray(w_up, dtype=np.float64).T)
    h = bf16(silu(g) * u)
    y = bf16(h @ np.asarray(w_down, dtype=np.float64).T)
    return h, y
