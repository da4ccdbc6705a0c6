"""Partial Attention Probing (PAP) token score -- test infrastructure only.

[SPTS] Fig. 2(a) caption and abstract: PAP picks informative tokens for the
attention block by computing a small fraction of the attention ahead of time
(a partial forward attention computation).  The pages print no formula; the
score computed here is the plainest one the rest supports:

  * the probe set F is the last P rows of the current candidate list
    ([SPTS] Table C varies this "query token length");
  * each probe row p attends causally (key j <= p) with the usual scaled
    softmax, scale tau = 1/sqrt(d_head), for every query head h, using the
    key head g(h) = floor(h / (Hq/Hkv)) (contiguous GQA groups);
  * the score of key token j is the post-softmax weight it receives, summed
    over all probe rows and all query heads:
        S_j = sum_h sum_{p in F, p >= j} softmax_j(tau * q_{p,h} . k_{j,g(h)}).

Since every softmax row sums to one, sum_j S_j = Hq * P exactly.
"""

import numpy as np


def pap_scores(q_probe, k, scale):
    """Probe score S over n candidate rows.

    q_probe : [P, Hq, dh] float64, queries of the last P candidate rows.
    k       : [n, Hkv, dh] float64, keys of all n candidate rows.
    scale   : softmax scale tau.
    returns : S [n] float64.
    """
    q_probe = np.asarray(q_probe, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    P, Hq, dh = q_probe.shape
    n, Hkv, dh2 = k.shape
    if dh != dh2 or Hq % Hkv != 0 or P > n:
        raise ValueError("pap_scores: bad shapes")
    group = Hq // Hkv
    probe_rows = np.arange(n - P, n)
    causal = np.arange(n)[None, :] <= probe_rows[:, None]          # [P, n]
    S = np.zeros(n, dtype=np.float64)
    for h in range(Hq):
        g = h // group
        logits = scale * (q_probe[:, h, :] @ k[:, g, :].T)            # [P, n]
        logits = np.where(causal, logits, -np.inf)
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        a = e / e.sum(axis=1, keepdims=True)
        S += a.sum(axis=0)
    return S
