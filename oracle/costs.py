"""Closed-form bookkeeping the pages print -- test infrastructure only.

[SPTS] Table 5: KV-cache size of the full model and of SPTS at 8K-32K tokens
on LLaMA-3.1-8B.  With MSDP a layer holds keys and values for its current
candidates only (Fig. A(c)), so the cache is the per-layer candidate count
times the K+V row size, summed over layers.  The page's "full cache" figures
(4.00 GB at 8K for 32 layers) count keys and values 4096 wide at 2 bytes, so
that is the row width used to reproduce them.

[SPTS] Table A: cost of one proxy projection per token, for D_low retained
channels of the 4096-wide model at rank r ("/" = not factored):
r * (4096 + D_low) multiply-accumulates when factored (4096 x r, then
r x D_low), and 4096 * D_low when not.
"""

from .layer import candidate_counts


def kv_cache_bytes(n, n_layers, points, kv_width=4096, bytes_per_elem=2):
    """K and V bytes over all layers for an n-token prompt."""
    counts = candidate_counts(n, n_layers, points)
    return sum(c * kv_width * 2 * bytes_per_elem for c in counts)


def proxy_macs(d_low, rank=None, d_model=4096):
    """Multiply-accumulates per token for one proxy projection."""
    if rank is None:
        return d_model * d_low
    return rank * (d_model + d_low)
