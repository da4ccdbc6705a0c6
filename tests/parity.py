"""Comparison rules shared by the GPU parity tests.

  * bf16 outputs:  max|got - ref| <= 2e-2 * max|ref| over the tensor;
  * fp32 outputs:  max|got - ref| <= 1e-4 * max|ref|;
  * index sets:    bit-exact, except where the oracle's score lies within
    1e-5 relative of the k-th boundary score (the "window rule": every
    chosen non-forced row scores >= t(1-1e-5), every unchosen one <= t(1+1e-5),
    t = the oracle's (k - n_forced)-th largest non-forced score).
"""

import numpy as np
import torch

BF16_REL = 2e-2
F32_REL = 1e-4
WINDOW_REL = 1e-5


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.detach().cpu().numpy().astype(np.float64)


def max_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def assert_close(got, ref, rel, what=""):
    e = max_rel_err(got, ref)
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), f"{what}: non-finite output"
    assert e <= rel, f"{what}: max|err|/max|ref| = {e:.3e} > {rel:.1e}"
    return e


def window_violations(oracle_scores, idx, k, n_forced, rel=WINDOW_REL):
    """Number of rows that break the window rule (0 = pass), plus checks of
    size, order and forcing."""
    s = np.asarray(oracle_scores, dtype=np.float64)
    n = s.shape[0]
    idx = np.asarray(idx, dtype=np.int64)
    if k >= n:
        return 0 if np.array_equal(idx, np.arange(n)) else n
    assert len(idx) == k, f"selected {len(idx)} rows, expected {k}"
    assert np.all(np.diff(idx) > 0), "indices not strictly ascending"
    forced = np.arange(n - n_forced, n)
    assert np.isin(forced, idx).all(), "a forced probe row is missing"
    free = np.arange(n - n_forced)
    if k == n_forced:
        return 0
    t = np.sort(s[free])[::-1][k - n_forced - 1]
    chosen = np.zeros(n, bool)
    chosen[idx] = True
    bad_in = free[chosen[free] & (s[free] < t * (1 - rel))]
    bad_out = free[~chosen[free] & (s[free] > t * (1 + rel))]
    return len(bad_in) + len(bad_out)


def agreeing_rows(final_pos, gpu_layers, ref_layers):
    """Original positions among final_pos whose every decision agreed in a
    free run: in each layer, membership in the candidate set, in the
    attention selection and in the FFN selection is the same on both sides.
    gpu_layers / ref_layers: per layer (pos, idx, idx_f) with pos the
    layer's candidates (original positions, after any pruning) and idx /
    idx_f indices into them (idx_f None for an attention-only layer)."""
    final_pos = np.asarray(final_pos, dtype=np.int64)
    ok = np.ones(len(final_pos), bool)

    def members(pos, rows):
        return np.isin(final_pos, np.asarray(pos, dtype=np.int64)[np.asarray(rows, dtype=np.int64)])

    for (gp, gi, gf), (rp, ri, rf) in zip(gpu_layers, ref_layers):
        ok &= np.isin(final_pos, gp) == np.isin(final_pos, rp)
        ok &= members(gp, gi) == members(rp, ri)
        if gf is not None:
            ok &= members(gp, gf) == members(rp, rf)
    return final_pos[ok]
