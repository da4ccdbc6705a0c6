"""The allocation-free top-k (spts_score_topk_noalloc) against the workspace
top-k (spts_score_topk) through the C ABI: bit-exact indices and fused
scores on two calls in a row, the second smaller, both past 32768 scores so
the keys go through the library's static scratch."""

import numpy as np
import pytest
import torch

import workloads as W
from free_token_skipping_amd import capi

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(n, k, nf, fused, seed):
    a = W.make_scores(n, seed=seed, ties=200).to(DEV)
    b = (W.make_scores(n, seed=seed + 1) * 1e-3).to(DEV) if fused else None
    ref_f = torch.empty(n, dtype=torch.float32, device=DEV) if fused else None
    ref = capi.spts_score_topk(a, k, nf, s_b=b, fused_out=ref_f)
    idx = torch.full((min(k, n),), -1, dtype=torch.int32, device=DEV)
    got_f = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV) if fused else None
    capi.spts_score_topk_noalloc(a, k, nf, idx, s_b=b, fused_out=got_f)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), ref.cpu()), (n, k, fused)
    if fused:
        assert torch.equal(got_f.cpu(), ref_f.cpu())


@pytest.mark.parametrize("fused", [False, True])
def test_noalloc_topk_matches_workspace_topk(fused):
    print(f"noalloc top-k, fused={fused}", flush=True)
    _case(131072, 32768, 128, fused, seed=11)       # first call: 131072 keys in the scratch
    _case(40000, 14000, 64, fused, seed=13)         # second, smaller: the scratch keeps older keys past 40000
    _case(20000, 7000, 64, fused, seed=15)          # keys in registers; no scratch use
