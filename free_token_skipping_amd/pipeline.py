"""One SPTS decoder layer and the Multi-Stage Delayed Pruning stack, as a
sequence of libspts calls on the current stream.

[SPTS] = "Probe and Skip: Self-Predictive Token Skipping for Efficient
Long-Context LLM Inference".  Fig. 2(a): PAP probe -> select -> reduced
attention, skipped tokens keep their residual; Fig. 2(b): LTP probe fused
with the attention score -> select -> reduced SwiGLU FFN; Fig. 2(c) and
Fig. A(c): the candidate set is fixed inside a stage and pruned at stage
boundaries.

This module only orders the calls and asks torch for buffers; every step
runs in the library's kernels.  With `fused=True` (default) the gather of
selected rows happens inside the projection GEMMs (gather on load) and the
residual adds inside the O / down projections (scatter-add on store); with
`fused=False` the standalone gather / scatter kernels do the same moves.

Sizes that the method leaves open follow the workload's reading: keep counts
are floor(ratio * n_current + 0.5); the last P candidates are the probes and
are forced into every selection and stage budget.
"""

import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import torch

from . import capi


def keep_count(ratio: float, n: int) -> int:
    """floor(ratio * n + 0.5), capped to [0, n]."""
    return int(min(n, max(0, math.floor(float(ratio) * float(n) + 0.5))))


@dataclass
class LayerConfig:
    Hq: int = 32
    Hkv: int = 8
    dh: int = 128
    P: int = 64
    keep_attn: float = 0.35
    keep_ffn: Optional[float] = 0.35      # None: attention-only layer
    w_fuse: Tuple[float, float] = (0.5, 0.5)
    prenorm: bool = False
    eps: float = 1e-5
    theta: Optional[float] = None         # None: no rotary embedding


def attention_block(x, pos, w: Dict[str, torch.Tensor], cfg: LayerConfig, rope_table=None,
                    k_given=None, prune_to=None, fused=True, trace=None):
    """x [n, d] bf16 residual (updated in place unless pruned), pos [n] int32.

    Returns (x_out, pos_out, S) where x_out/pos_out are the (possibly pruned)
    candidates and S their PAP score (float32)."""
    n, d = x.shape
    Hq, Hkv, dh, P = cfg.Hq, cfg.Hkv, cfg.dh, cfg.P
    rope = cfg.theta is not None
    xt = capi.spts_rmsnorm(x, cfg.eps) if cfg.prenorm else x
    # a1: K, V over all current candidates
    if k_given is None:
        K = (capi.spts_linear_rope(xt, w["wk"], pos, rope_table) if rope else capi.spts_linear(xt, w["wk"]))
        K = K.view(n, Hkv, dh)
    else:
        K = k_given
    V = capi.spts_linear(xt, w["wv"]).view(n, Hkv, dh)
    # a2: probe queries (last P rows)
    xp = xt[n - P:]
    Qp = (capi.spts_linear_rope(xp, w["wq"], pos[n - P:], rope_table) if rope else capi.spts_linear(xp, w["wq"]))
    # a3: PAP score
    S = capi.spts_probe_attention(Qp.view(P, Hq, dh), K)
    if trace is not None:
        trace.update(S_pre=S, K_pre=K, V_pre=V)
    # a14: MSDP boundary -- prune, then compact every per-candidate tensor
    if prune_to is not None and prune_to < n:
        keep, pos, x = capi.spts_msdp_stage(S, prune_to, P, pos, x)
        xt = capi.spts_gather(xt, keep) if cfg.prenorm else x
        K = capi.spts_gather(K, keep)
        V = capi.spts_gather(V, keep)
        S = capi.spts_gather(S, keep)
        n = prune_to
        if trace is not None:
            trace.update(keep=keep)
    # a4: select the attention rows
    k_a = keep_count(cfg.keep_attn, n)
    idx = capi.spts_score_topk(S, k_a, P)
    # a5 + a6: gather selected rows, Q projection
    if fused:
        Qs = (capi.spts_linear_rope(xt, w["wq"], pos, rope_table, a_rows=idx) if rope
              else capi.spts_linear(xt, w["wq"], a_rows=idx))
    else:
        xs = capi.spts_gather(xt, idx)
        Qs = (capi.spts_linear_rope(xs, w["wq"], capi.spts_gather(pos, idx), rope_table) if rope
              else capi.spts_linear(xs, w["wq"]))
    # a7: reduced attention over all candidates' K/V
    O = capi.spts_reduced_attention(Qs.view(k_a, Hq, dh), idx, K, V)
    # a8: O projection + residual add into the selected rows
    if fused:
        capi.spts_linear(O.view(k_a, Hq * dh), w["wo"], out=x, out_rows=idx, accumulate=True)
    else:
        delta = capi.spts_linear(O.view(k_a, Hq * dh), w["wo"])
        capi.spts_scatter(delta, idx, x, accumulate=True)
    if trace is not None:
        trace.update(S=S, idx=idx, K=K, V=V, Qp=Qp, Qs=Qs, O=O, pos=pos)
    return x, pos, S


def ffn_block(h, S, w, cfg: LayerConfig, fused=True, trace=None):
    """h [n, d] residual (updated in place), S [n] PAP score of this layer."""
    n, d = h.shape
    z = capi.spts_rmsnorm(h, cfg.eps) if cfg.prenorm else h
    # a9: LTP proxy score
    L = capi.spts_ltp_probe(z, w["u_t"], w["v_t"])
    # a10: fused score -> select the FFN rows
    k_f = keep_count(cfg.keep_ffn, n)
    fused_score = torch.empty(n, dtype=torch.float32, device=h.device) if trace is not None else None
    idx_f = capi.spts_score_topk(S, k_f, cfg.P, s_b=L, w_a=cfg.w_fuse[0], w_b=cfg.w_fuse[1], fused_out=fused_score)
    # a11 + a12 + a13: gather, reduced SwiGLU, residual add
    if fused:
        capi.spts_reduced_ffn(z, w["wg"], w["wu"], w["wd"], rows=idx_f, y=h, y_rows=idx_f, accumulate=True)
    else:
        zs = capi.spts_gather(z, idx_f)
        y = capi.spts_reduced_ffn(zs, w["wg"], w["wu"], w["wd"])
        capi.spts_scatter(y, idx_f, h, accumulate=True)
    if trace is not None:
        trace.update(L=L, fused=fused_score, idx_f=idx_f, z=z)
    return h


def spts_layer(x, pos, w, cfg: LayerConfig, rope_table=None, k_given=None, prune_to=None, fused=True,
               trace=None):
    """Attention block then (if cfg.keep_ffn is set) FFN block."""
    x, pos, S = attention_block(x, pos, w, cfg, rope_table, k_given, prune_to, fused, trace)
    if cfg.keep_ffn is not None:
        x = ffn_block(x, S, w, cfg, fused, trace)
    return x, pos


def prune_points(first_skip_layer, stage_end_layers, budgets, final_budget=None):
    """Layers where the candidate set is pruned, and the budget there."""
    starts = [first_skip_layer] + [e + 1 for e in stage_end_layers[:-1]]
    pts = dict(zip(starts, budgets))
    if final_budget is not None:
        pts[stage_end_layers[-1] + 1] = final_budget
    return pts


def msdp_stack(x0, layers, cfg: LayerConfig, points, fused=True, traces=None):
    """Run the stack on embeddings x0 [N, d] (not modified).  Returns the
    residual over the final candidates and their original positions."""
    N = x0.shape[0]
    x = x0.clone()
    pos = torch.arange(N, dtype=torch.int32, device=x0.device)
    table = capi.spts_rope_table(N, cfg.dh, cfg.theta, x0.device) if cfg.theta is not None else None
    for li, w in enumerate(layers):
        budget = points.get(li)
        prune = budget if budget is not None and budget < x.shape[0] else None
        tr = {} if traces is not None else None
        x, pos = spts_layer(x, pos, w, cfg, table, prune_to=prune, fused=fused, trace=tr)
        if traces is not None:
            traces.append(tr)
    return x, pos
