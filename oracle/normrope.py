"""RMSNorm and rotary position embedding -- test infrastructure only.

The SPTS pages name neither; the 8-layer LLaMA-3.1-8B-shaped workload does
(RMSNorm eps 1e-5, RoPE theta 5e5).  Readings:

  * RMSNorm with unit gain: x / sqrt(mean(x^2) + eps);
  * RoPE in the half-split ("rotate half") form: for head dimension dh and
    i < dh/2, the pair (x_i, x_{i+dh/2}) is rotated by the angle
    pos * theta^(-2i/dh), where pos is the token's ORIGINAL position in the
    sequence (so a token keeps its position after pruning).  No long-context
    frequency rescaling.
"""

import numpy as np


def rmsnorm(x, eps=1e-5):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, pos, theta):
    """x [rows, H, dh] float64, pos [rows] int -> rotated copy (float64)."""
    x = np.asarray(x, dtype=np.float64)
    rows, H, dh = x.shape
    half = dh // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / dh)                      # [half]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
