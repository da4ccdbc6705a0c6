"""One SPTS decoder layer and the Multi-Stage Delayed Pruning stack --
test infrastructure only.

[SPTS] Fig. 2: a skipping layer runs PAP selection and reduced attention in
its attention block (a), then LTP selection and the reduced feed-forward in
its FFN block (b); skipped tokens keep their residual unchanged (Fig. 2 top).
Fig. 2(c): MSDP splits the skipping layers into stages; the candidate token
set stays fixed inside a stage and is pruned at the stage boundary.
Fig. A(c): a skipped token is still a candidate (its keys and values are
recomputed in later layers of the stage) until a stage boundary prunes it.

Readings taken where the pages are silent (each also listed with the
workload recipe):
  * attention block first, then FFN; the FFN's fused score reuses the same
    layer's PAP score S;
  * the probe rows (last P candidates) are forced into every selection and
    every stage budget;
  * keep counts from ratios are floor(ratio * n_current + 0.5);
  * pruning happens at the first layer of each stage, ranked by that layer's
    PAP score over the outgoing candidate set; the layer then runs on the
    pruned set, with the score restricted to it;
  * bare layers (no norm, no RoPE) for the single-layer workloads; a
    pre-norm LLaMA block with RMSNorm and RoPE at original positions for the
    stack.

Storage points (bfloat16): Q, K, V after projection (and RoPE), the
attention output O, the O-projection delta, the residual after each add, the
FFN hidden H, the FFN output y, and the normalised input of each block.
Scores S and L are produced in float32.
"""

import numpy as np

from .numerics import bf16, f32, keep_count
from .pap import pap_scores
from .select import select_topk, fuse_maxnorm, fuse_multiply
from .attention import reduced_attention
from .ltp import ltp_scores, ltp_structured_scores
from .ffn import swiglu_rows
from .normrope import rmsnorm, rope


def project(x, w, heads, dh, pos=None, theta=None):
    """One head-shaped projection as the layer stores it: x W^T accumulated
    to fp32, rotated (RoPE at `pos`) when theta is given, rounded to bf16.
    x [rows, d], w [heads*dh, d] -> [rows, heads, dh] float64."""
    acc = f32(x @ np.asarray(w, dtype=np.float64).T)
    acc = acc.reshape(x.shape[0], heads, dh)
    if theta is not None:
        acc = rope(acc, pos, theta)
    return bf16(acc)


_proj = project


def attention_block(x, pos, w, cfg, k_given=None, prune_to=None):
    """SPTS attention block over the n current candidates.

    x [n,d] float64 (bf16 values), pos [n] original positions, w: dict with
    wq [Hq*dh,d], wk/wv [Hkv*dh,d], wo [d,Hq*dh].  cfg keys: Hq, Hkv, dh, P,
    keep_attn (ratio) or k_attn (count), prenorm, eps, theta (None = no RoPE).
    k_given: optional keys [n,Hkv,dh] used instead of the K projection.
    prune_to: optional MSDP budget; if set, the candidate set is pruned to it
    after the score is computed (first layer of a stage).

    Returns (y, state) where y is the new residual over the (possibly pruned)
    candidates and state holds S, idx, K, V, pos, keep (the prune result).
    """
    Hq, Hkv, dh, P = cfg["Hq"], cfg["Hkv"], cfg["dh"], cfg["P"]
    theta = cfg.get("theta")
    scale = 1.0 / np.sqrt(dh)
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    xt = bf16(rmsnorm(x, cfg.get("eps", 1e-5))) if cfg.get("prenorm") else x
    if k_given is None:
        K = _proj(xt, w["wk"], Hkv, dh, pos, theta)
    else:
        K = np.asarray(k_given, dtype=np.float64)
    V = _proj(xt, w["wv"], Hkv, dh)
    Qp = _proj(xt[-P:], w["wq"], Hq, dh, pos[-P:], theta)
    S = pap_scores(Qp, K, scale)
    S_full = S
    keep = None
    if prune_to is not None:
        keep = select_topk(f32(S), prune_to, P)
        x, xt, pos, K, V, S = x[keep], xt[keep], pos[keep], K[keep], V[keep], S[keep]
    n = x.shape[0]
    k_a = cfg["k_attn"] if "k_attn" in cfg else keep_count(cfg["keep_attn"], n)
    idx = select_topk(f32(S), k_a, P)
    Qs = _proj(xt[idx], w["wq"], Hq, dh, pos[idx], theta)
    O = bf16(reduced_attention(Qs, idx, K, V, scale))
    delta = bf16(O.reshape(len(idx), Hq * dh) @ np.asarray(w["wo"], dtype=np.float64).T)
    y = x.copy()
    y[idx] = bf16(x[idx] + delta)
    state = dict(S=S, S_full=S_full, idx=idx, K=K, V=V, Qp=Qp, Qs=Qs, O=O, pos=pos, keep=keep, xt=xt)
    return y, state


def ffn_block(h, S, w, cfg):
    """SPTS FFN block: LTP score, fusion with S (MaxNorm-Add or Multiply), reduced SwiGLU.

    h [n,d] residual, S [n] PAP score of this layer.  w: wg/wu [f,d], wd [d,f],
    u_t [r,d], v_t [d,r] (or, with proxy "structured", the factors a_g_t,
    b_g_t, a_u_t, b_u_t, c_t, d_t).  cfg keys: P, keep_ffn or k_ffn, fusion ("maxnorm_add",
    the default, with w_fuse (w_a, w_b); or "multiply", [SPTS] Table D), prenorm, eps.
    """
    P = cfg["P"]
    h = np.asarray(h, dtype=np.float64)
    z = bf16(rmsnorm(h, cfg.get("eps", 1e-5))) if cfg.get("prenorm") else h
    if cfg.get("proxy", "linear") == "structured":
        L = ltp_structured_scores(z, w["a_g_t"], w["b_g_t"], w["a_u_t"], w["b_u_t"], w["c_t"], w["d_t"])
    else:
        L = ltp_scores(z, w["u_t"], w["v_t"])
    if cfg.get("fusion", "maxnorm_add") == "multiply":
        fused = fuse_multiply(f32(S), f32(L))
    else:
        w_a, w_b = cfg.get("w_fuse", (0.5, 0.5))
        fused = fuse_maxnorm(f32(S), f32(L), w_a, w_b)
    n = h.shape[0]
    k_f = cfg["k_ffn"] if "k_ffn" in cfg else keep_count(cfg["keep_ffn"], n)
    idx_f = select_topk(fused, k_f, P)
    H, y = swiglu_rows(z[idx_f], w["wg"], w["wu"], w["wd"])
    out = h.copy()
    out[idx_f] = bf16(h[idx_f] + y)
    return out, dict(L=L, fused=fused, idx_f=idx_f, z=z, H=H, y=y)


def spts_layer(x, pos, w, cfg, k_given=None, prune_to=None):
    """Attention block then FFN block.  Returns (out, attn_state, ffn_state)."""
    y, st_a = attention_block(x, pos, w, cfg, k_given=k_given, prune_to=prune_to)
    out, st_f = ffn_block(y, st_a["S"], w, cfg)
    return out, st_a, st_f


# ---------------------------------------------------------------- MSDP stack

def prune_points(first_skip_layer, stage_end_layers, budgets, final_budget=None):
    """Layers at which the candidate set is pruned, and the budget there.

    [SPTS] Table B gives, per model, the first skipping layer, the last layer
    of each stage, each stage's active token budget and the tokens left after
    the last stage.  Stage s starts one layer after stage s-1 ends (the first
    stage starts at the first skipping layer); the layers after the last
    stage keep `final_budget` tokens.
    """
    starts = [first_skip_layer] + [e + 1 for e in stage_end_layers[:-1]]
    pts = {s: b for s, b in zip(starts, budgets)}
    if final_budget is not None:
        pts[stage_end_layers[-1] + 1] = final_budget
    return pts


def candidate_counts(n, n_layers, points):
    """Candidates held by each layer: the count only shrinks, at prune points."""
    counts, c = [], n
    for layer in range(n_layers):
        if layer in points:
            c = min(c, points[layer])
        counts.append(c)
    return counts


def msdp_stack(x0, layers_w, cfg, points):
    """Run an SPTS stack with Multi-Stage Delayed Pruning.

    x0 [N,d] embeddings (bf16 values); layers_w: list of per-layer weight
    dicts; points: {layer: budget} from `prune_points`.  Returns (x, pos,
    history) with x the residual over the final candidates, pos their
    original positions and history a per-layer list of states.
    """
    x = np.asarray(x0, dtype=np.float64)
    pos = np.arange(x.shape[0], dtype=np.int64)
    history = []
    for layer, w in enumerate(layers_w):
        budget = points.get(layer)
        prune_to = None if budget is None or budget >= x.shape[0] else budget
        x_in_pos = pos
        x, st_a, st_f = spts_layer(x, pos, w, cfg, prune_to=prune_to)
        pos = st_a["pos"]
        history.append(dict(layer=layer, pos_in=x_in_pos, pos=pos, attn=st_a, ffn=st_f))
    return x, pos, history
