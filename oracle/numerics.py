"""bfloat16 storage points for the oracle -- test infrastructure only.

The pages fix no precision.  The GPU path accumulates in fp32 and stores
activations as bfloat16; the oracle mirrors only those storage points:
a float64 value is first rounded to fp32 (round-to-nearest-even, by numpy's
cast), then to bfloat16 (round-to-nearest-even, by integer arithmetic on the
fp32 bit pattern).  bfloat16 tensors are held as uint16 bit patterns.
"""

import numpy as np


def f32(x):
    """Round to fp32 (RNE) and return as float64 for further fp64 arithmetic."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_bf16_bits(x):
    """float -> bfloat16 bit pattern (uint16), via fp32, ties to even.

    NaN maps to the canonical quiet NaN 0x7FC0; infinities are preserved.
    """
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    bits = r.astype(np.uint16)
    bits = np.where(np.isnan(x32), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def from_bf16_bits(bits):
    """bfloat16 bit pattern (uint16) -> float64 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    u = b.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16(x):
    """Round a float64 array to the nearest bfloat16 value (through fp32)."""
    return from_bf16_bits(to_bf16_bits(x))


def keep_count(ratio, n):
    """Number of rows kept for a keep ratio applied to n current rows.

    The pages give ratios and budgets, not a rounding rule; this build rounds
    half up: floor(ratio * n + 0.5), computed in float64, capped to [0, n].
    """
    return int(min(n, max(0, np.floor(float(ratio) * float(n) + 0.5))))
