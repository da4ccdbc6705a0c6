"""Token selection and score fusion -- test infrastructure only.

[SPTS] abstract and Fig. 2(a)(b): the probed scores pick which tokens take
part in the reduced attention / reduced feed-forward; the rest are skipped.
The pages do not spell out the selection rule; this build takes top-k:

  * the last n_forced rows (the probe rows) are always kept -- [SPTS] Fig. 3(b)
    shows that the last token must still be computed -- and count toward k;
  * the other k - n_forced rows are the largest scores among the remaining
    rows, ties broken toward the lower row index;
  * the result is returned in ascending row order (causal order);
  * k >= n keeps every row.

Scores are ordered as IEEE values; NaN is treated as the smallest score and
-0.0 equals +0.0.

[SPTS] Table D compares ways to fuse the FFN probe with the attention score.
`fuse_maxnorm` is its "MaxNorm-Add": each score divided by its maximum over
the current candidates, then a weighted sum.  Because a fused score decides
an integer (which rows are kept), it is evaluated in float32 with a fixed
operation order, exactly as the kernel evaluates it:
    c = fl(fl(w_a * fl(s_a / max s_a)) + fl(w_b * fl(s_b / max s_b))),
with a term taken as 0 when its maximum is not positive.  The maxima run
over every row and skip NaN (a NaN score leaves the other rows' normalised
values as they are; its own fused value is NaN and ranks lowest); a score
with no number at all has no positive maximum, so its term is 0.

Table D's "Multiply" (the pages' default fusion, as C^FFN * S^MHA in Table 6)
is `fuse_multiply`: the product of the two scores, one float32 rounding.  A
positive factor on either score does not change the ranking, so no
normalisation is applied.  This build reads C^FFN as the LTP score itself.
"""

import numpy as np


def _sortable(s):
    s = np.asarray(s, dtype=np.float64).copy()
    s[np.isnan(s)] = -np.inf
    s[s == 0.0] = 0.0          # -0.0 -> +0.0
    return s


def select_topk(scores, k, n_forced):
    """Ascending indices of the kept rows (exactly min(k, n) of them)."""
    s = _sortable(scores)
    n = s.shape[0]
    if not (0 <= n_forced <= k) or n_forced > n:
        raise ValueError("select_topk: need 0 <= n_forced <= k and n_forced <= n")
    if k >= n:
        return np.arange(n, dtype=np.int64)
    free = np.arange(n - n_forced)
    # primary key: score descending; secondary: row index ascending
    order = np.lexsort((free, -s[free]))
    chosen = free[order[: k - n_forced]]
    forced = np.arange(n - n_forced, n)
    return np.sort(np.concatenate([chosen, forced])).astype(np.int64)


def fuse_maxnorm(s_a, s_b, w_a=0.5, w_b=0.5):
    """MaxNorm-Add fusion in float32, fixed operation order (see module doc)."""
    a = np.asarray(s_a, dtype=np.float32)
    b = np.asarray(s_b, dtype=np.float32)
    wa = np.float32(w_a)
    wb = np.float32(w_b)

    def term(w, x):
        finite = x[~np.isnan(x)]
        mx = np.float32(finite.max()) if finite.size else np.float32(0)
        if not (mx > 0):
            return np.zeros_like(x)
        q = (x / mx).astype(np.float32)
        return (w * q).astype(np.float32)

    return (term(wa, a) + term(wb, b)).astype(np.float32)


def fuse_multiply(s_a, s_b):
    """Multiply fusion in float32: c = fl(s_a * s_b)."""
    a = np.asarray(s_a, dtype=np.float32)
    b = np.asarray(s_b, dtype=np.float32)
    return (a * b).astype(np.float32)
