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


class _NoTimer:
    def __call__(self, name, work=None):
        return self

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


NO_TIMER = _NoTimer()


class CallTimer:
    """Records a start/end HIP event pair on the current stream around each
    named library call (the stream the call's kernels run on), with an
    optional algorithmic work figure for the call.  only: if given, the set of
    call names that get events; other calls run unbracketed."""

    def __init__(self, only=None):
        self.records = []
        self._cur = None
        self._only = only

    def __call__(self, name, work=None):
        self._cur = (name, work)
        return self

    def __enter__(self):
        self._start = None
        if self._only is None or self._cur[0] in self._only:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record()
            self._start = e0
        return self

    def __exit__(self, *exc):
        if self._start is None:
            return False
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        name, work = self._cur
        self.records.append((name, work, self._start, e1))
        return False

    def summary(self):
        """{name: (calls, total_ms, total_work)} after a synchronize."""
        out = {}
        for name, work, a, b in self.records:
            if callable(work):
                work = work()
            c, t, w = out.get(name, (0, 0.0, 0.0))
            out[name] = (c + 1, t + a.elapsed_time(b), w + (work or 0.0))
        return out


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
    fusion: str = "maxnorm_add"           # FFN score fusion: "maxnorm_add" or "multiply"
    proxy: str = "linear"                 # LTP proxy: "linear" (u_t, v_t) or "structured" (proxy_packed)
    ltp_form: str = "gram"                # linear proxy score: "gram" (sqrt(t G t^T)) or "direct" (||t V||)
    prenorm: bool = False
    eps: float = 1e-5
    theta: Optional[float] = None         # None: no rotary embedding


def ltp_gram(w, key="v_t"):
    """Gram operand of the proxy's last factor w[key] (spts_ltp_gram): v_t of
    the linear proxy, d_t of the packed structured one.  Prepared on first use
    and kept in w; prepared again when the factor is replaced or written in
    place (its version counter moves)."""
    v = w[key]
    stamp = (v.data_ptr(), v._version, tuple(v.shape))
    cached = w.get("_gram_" + key)
    if cached is None or cached[0] != stamp:
        cached = (stamp, capi.spts_ltp_gram(v))
        w["_gram_" + key] = cached
    return cached[1]


def _attn_flops(idx, Hq, dh):
    """Algorithmic reduced-attention FLOPs: 4*Hq*dh per (query, visible key)."""
    return lambda: 4.0 * Hq * dh * float((idx.to(torch.float64) + 1).sum().item())


def attention_block(x, pos, w: Dict[str, torch.Tensor], cfg: LayerConfig, rope_table=None,
                    k_given=None, prune_to=None, fused=True, trace=None, tm=NO_TIMER, kv_out=None):
    """x [n, d] bf16 residual (updated in place unless pruned), pos [n] int32.

    Returns (x_out, pos_out, S) where x_out/pos_out are the (possibly pruned)
    candidates and S their PAP score (float32).  `tm` (a CallTimer) brackets
    each library call with events; work figures are algorithmic FLOPs or bytes."""
    n, d = x.shape
    Hq, Hkv, dh, P = cfg.Hq, cfg.Hkv, cfg.dh, cfg.P
    rope = cfg.theta is not None
    if cfg.prenorm:
        with tm("rmsnorm", 4.0 * n * d):
            xt = capi.spts_rmsnorm(x, cfg.eps)
    else:
        xt = x
    # a1: K, V over all current candidates (+ RoPE on K).  At an MSDP boundary
    # (fused path) only K is needed for every candidate -- the probe scores
    # them all -- so V is projected after the pruning, for the kept rows only
    v_late = fused and k_given is None and prune_to is not None and prune_to < n
    V = None
    if k_given is None and fused and not v_late:
        with tm("kv_proj", 4.0 * n * d * Hkv * dh):
            K, V = capi.spts_linear_kv(xt, w["wk"], w["wv"], pos if rope else None, rope_table if rope else None)
        K, V = K.view(n, Hkv, dh), V.view(n, Hkv, dh)
    else:
        if k_given is None:
            with tm("k_proj", 2.0 * n * d * Hkv * dh):
                K = (capi.spts_linear_rope(xt, w["wk"], pos, rope_table) if rope
                     else capi.spts_linear(xt, w["wk"]))
            K = K.view(n, Hkv, dh)
        else:
            K = k_given
        if not v_late:
            with tm("v_proj", 2.0 * n * d * Hkv * dh):
                V = capi.spts_linear(xt, w["wv"]).view(n, Hkv, dh)
    # a2: probe queries (last P rows)
    xp = xt[n - P:]
    with tm("probe_q_proj", 2.0 * P * d * Hq * dh):
        Qp = (capi.spts_linear_rope(xp, w["wq"], pos[n - P:], rope_table) if rope
              else capi.spts_linear(xp, w["wq"]))
    # a3: PAP score
    with tm("pap_probe", 2.0 * Hq * dh * P * n):
        S = capi.spts_probe_attention(Qp.view(P, Hq, dh), K)
    if trace is not None:
        trace.update(S_pre=S, K_pre=K, V_pre=V, xt=xt if cfg.prenorm else None)
    # a14: MSDP boundary -- prune, then compact every per-candidate tensor
    xt_rows, xt_pos = None, pos             # rows of xt (and their positions) behind candidate i
    if prune_to is not None and prune_to < n:
        with tm("msdp_stage", 4.0 * n + 4.0 * prune_to + 2.0 * prune_to * (4 + 2 * d)):
            keep, pos, x = capi.spts_msdp_stage(S, prune_to, P, pos, x)
        # fused: the normalised rows stay where they are; the Q projection
        # gathers them through keep
        copy_xt = cfg.prenorm and not fused
        with tm("msdp_compact", 2.0 * prune_to * (2 * Hkv * dh * 2 + 4 + (2 * d if copy_xt else 0))):
            if not cfg.prenorm:
                xt, xt_pos = x, pos
            elif copy_xt:
                xt, xt_pos = capi.spts_gather(xt, keep), pos
            else:
                xt_rows = keep
            K = capi.spts_gather(K, keep)
            if V is not None:
                V = capi.spts_gather(V, keep)
            S = capi.spts_gather(S, keep)
        n = prune_to
        if trace is not None:
            trace.update(keep=keep)
    if V is None:
        # V of the kept candidates, their normalised rows gathered on load
        with tm("v_proj", 2.0 * n * d * Hkv * dh):
            V = (capi.spts_linear(xt, w["wv"], a_rows=xt_rows) if xt_rows is not None
                 else capi.spts_linear(xt, w["wv"])).view(n, Hkv, dh)
    if kv_out is not None:
        kv_out.append((K, V))             # this layer's cache: its candidates' keys and values
    # a4: select the attention rows
    k_a = keep_count(cfg.keep_attn, n)
    with tm("select_attn", 4.0 * n + 4.0 * k_a):
        idx = capi.spts_score_topk(S, k_a, P)
    # a5 + a6: gather selected rows, Q projection
    if fused:
        with tm("q_proj", 2.0 * k_a * d * Hq * dh):
            rows = idx if xt_rows is None else capi.spts_gather(xt_rows, idx)
            Qs = (capi.spts_linear_rope(xt, w["wq"], xt_pos, rope_table, a_rows=rows) if rope
                  else capi.spts_linear(xt, w["wq"], a_rows=rows))
    else:
        with tm("gather_x", 4.0 * k_a * d):
            xs = capi.spts_gather(xt, idx)
        with tm("q_proj", 2.0 * k_a * d * Hq * dh):
            Qs = (capi.spts_linear_rope(xs, w["wq"], capi.spts_gather(pos, idx), rope_table) if rope
                  else capi.spts_linear(xs, w["wq"]))
    # a7: reduced attention over all candidates' K/V
    with tm("reduced_attention", _attn_flops(idx, Hq, dh)):
        O = capi.spts_reduced_attention(Qs.view(k_a, Hq, dh), idx, K, V)
    # a8: O projection + residual add into the selected rows
    if fused:
        with tm("o_proj_add", 2.0 * k_a * Hq * dh * d):
            capi.spts_linear(O.view(k_a, Hq * dh), w["wo"], out=x, out_rows=idx, accumulate=True)
    else:
        with tm("o_proj", 2.0 * k_a * Hq * dh * d):
            delta = capi.spts_linear(O.view(k_a, Hq * dh), w["wo"])
        with tm("scatter_add_x", 6.0 * k_a * d):
            capi.spts_scatter(delta, idx, x, accumulate=True)
    if trace is not None:
        trace.update(S=S, idx=idx, K=K, V=V, Qp=Qp, Qs=Qs, O=O, pos=pos)
    return x, pos, S


def ffn_block(h, S, w, cfg: LayerConfig, fused=True, trace=None, tm=NO_TIMER):
    """h [n, d] residual (updated in place), S [n] PAP score of this layer."""
    n, d = h.shape
    f = w["wg"].shape[0]
    if cfg.prenorm:
        with tm("rmsnorm", 4.0 * n * d):
            z = capi.spts_rmsnorm(h, cfg.eps)
    else:
        z = h
    # a9: LTP proxy score
    if cfg.proxy == "structured":
        pk = w["proxy_packed"]
        r, d_low = pk["c_t"].shape
        if cfg.ltp_form == "gram":
            gram = ltp_gram(pk, "d_t")      # offline: once per proxy
            with tm("ltp_probe", 2.0 * n * r * (2 * d + 3 * d_low + r)):
                L = capi.spts_ltp_probe_structured(z, pk, gram=gram)
        else:
            with tm("ltp_probe", 2.0 * n * 3 * r * (d + d_low)):
                L = capi.spts_ltp_probe_structured(z, pk)
    elif cfg.ltp_form == "gram":
        r = w["u_t"].shape[0]
        gram = ltp_gram(w)                  # offline: once per proxy
        with tm("ltp_probe", 2.0 * n * r * (d + r)):
            L = capi.spts_ltp_probe_gram(z, w["u_t"], gram)
    else:
        r = w["u_t"].shape[0]
        with tm("ltp_probe", 4.0 * n * d * r):
            L = capi.spts_ltp_probe(z, w["u_t"], w["v_t"])
    # a10: fused score -> select the FFN rows
    k_f = keep_count(cfg.keep_ffn, n)
    fused_score = torch.empty(n, dtype=torch.float32, device=h.device) if trace is not None else None
    with tm("select_ffn", 8.0 * n + 4.0 * k_f):
        if cfg.fusion == "multiply":
            idx_f = capi.spts_score_topk_multiply(S, L, k_f, cfg.P, fused_out=fused_score)
        else:
            idx_f = capi.spts_score_topk(S, k_f, cfg.P, s_b=L, w_a=cfg.w_fuse[0], w_b=cfg.w_fuse[1],
                                         fused_out=fused_score)
    # a11 + a12 + a13: gather, reduced SwiGLU, residual add
    if fused:
        # the two GEMMs of spts_reduced_ffn as separate calls, so each is timed
        with tm("ffn_gate_up", 4.0 * k_f * d * f):
            H = capi.spts_linear_swiglu(z, w["wg"], w["wu"], a_rows=idx_f)
        with tm("ffn_down_add", 2.0 * k_f * d * f):
            capi.spts_linear(H, w["wd"], out=h, out_rows=idx_f, accumulate=True)
    else:
        with tm("gather_z", 4.0 * k_f * d):
            zs = capi.spts_gather(z, idx_f)
        with tm("reduced_ffn", 6.0 * k_f * d * f):
            y = capi.spts_reduced_ffn(zs, w["wg"], w["wu"], w["wd"])
        with tm("scatter_add_h", 6.0 * k_f * d):
            capi.spts_scatter(y, idx_f, h, accumulate=True)
    if trace is not None:
        trace.update(L=L, fused=fused_score, idx_f=idx_f, z=z)
    return h


def spts_layer(x, pos, w, cfg: LayerConfig, rope_table=None, k_given=None, prune_to=None, fused=True,
               trace=None, tm=NO_TIMER, kv_out=None):
    """Attention block then (if cfg.keep_ffn is set) FFN block.  A trace
    dict, if given, also receives copies of the layer's input (x_in, pos_in),
    of the residual between the blocks (x_mid) and of its output (x_out)."""
    if trace is not None:
        trace.update(x_in=x.clone(), pos_in=pos.clone())
    x, pos, S = attention_block(x, pos, w, cfg, rope_table, k_given, prune_to, fused, trace, tm, kv_out)
    if cfg.keep_ffn is not None:
        if trace is not None:
            trace["x_mid"] = x.clone()
        x = ffn_block(x, S, w, cfg, fused, trace, tm)
    if trace is not None:
        trace["x_out"] = x.clone()
    return x, pos


def prune_points(first_skip_layer, stage_end_layers, budgets, final_budget=None):
    """Layers where the candidate set is pruned, and the budget there."""
    starts = [first_skip_layer] + [e + 1 for e in stage_end_layers[:-1]]
    pts = dict(zip(starts, budgets))
    if final_budget is not None:
        pts[stage_end_layers[-1] + 1] = final_budget
    return pts


def dense_layer(x, pos, w, cfg: LayerConfig, rope_table=None, tm=NO_TIMER, kv_out=None, trace=None):
    """The same decoder layer with every row computed: no probes, no
    selection.  This is the dense-prefill baseline that SPTS is compared
    against ([SPTS] Table 4 compares TTFT against the full model).  x [n, d]
    bf16 is updated in place; every row is a query, so the attention call is
    plain causal attention."""
    n, d = x.shape
    Hq, Hkv, dh = cfg.Hq, cfg.Hkv, cfg.dh
    rope = cfg.theta is not None
    if trace is not None:
        trace.update(x_in=x.clone(), pos_in=pos.clone(), dense=True)
    if cfg.prenorm:
        with tm("rmsnorm", 4.0 * n * d):
            xt = capi.spts_rmsnorm(x, cfg.eps)
    else:
        xt = x
    with tm("kv_proj", 4.0 * n * d * Hkv * dh):
        K, V = capi.spts_linear_kv(xt, w["wk"], w["wv"], pos if rope else None, rope_table if rope else None)
    with tm("q_proj", 2.0 * n * d * Hq * dh):
        Q = (capi.spts_linear_rope(xt, w["wq"], pos, rope_table) if rope else capi.spts_linear(xt, w["wq"]))
    if kv_out is not None:
        kv_out.append((K.view(n, Hkv, dh), V.view(n, Hkv, dh)))
    idx = torch.arange(n, dtype=torch.int32, device=x.device)
    with tm("attention", _attn_flops(idx, Hq, dh)):
        O = capi.spts_reduced_attention(Q.view(n, Hq, dh), idx, K.view(n, Hkv, dh), V.view(n, Hkv, dh))
    with tm("o_proj_add", 2.0 * n * Hq * dh * d):
        capi.spts_linear(O.view(n, Hq * dh), w["wo"], out=x, accumulate=True)
    if cfg.keep_ffn is not None:
        f = w["wg"].shape[0]
        if cfg.prenorm:
            with tm("rmsnorm", 4.0 * n * d):
                z = capi.spts_rmsnorm(x, cfg.eps)
        else:
            z = x
        with tm("ffn_gate_up", 4.0 * n * d * f):
            H = capi.spts_linear_swiglu(z, w["wg"], w["wu"])
        with tm("ffn_down_add", 2.0 * n * d * f):
            capi.spts_linear(H, w["wd"], out=x, accumulate=True)
    if trace is not None:
        trace["x_out"] = x.clone()
    return x


def prefill_schedule(x0, layers, cfg: LayerConfig, n_layers, first_skip_layer, points, dense=False,
                     tm=NO_TIMER, kv_out=None, traces=None):
    """Prefill of an n_layers model: layers before first_skip_layer are dense,
    the rest are SPTS layers pruned at `points` ([SPTS] Table B gives such a
    schedule per model).  dense=True runs every layer dense (the full-model
    baseline).  Layer li uses weights layers[li % len(layers)].  Returns the
    residual over the final candidates and their original positions.
    traces: if a list, receives one trace dict per layer."""
    N = x0.shape[0]
    x = x0.clone()
    pos = torch.arange(N, dtype=torch.int32, device=x0.device)
    table = capi.spts_rope_table(N, cfg.dh, cfg.theta, x0.device) if cfg.theta is not None else None
    for li in range(n_layers):
        w = layers[li % len(layers)]
        tr = {} if traces is not None else None
        if dense or li < first_skip_layer:
            x = dense_layer(x, pos, w, cfg, table, tm=tm, kv_out=kv_out, trace=tr)
        else:
            budget = points.get(li)
            prune = budget if budget is not None and budget < x.shape[0] else None
            x, pos = spts_layer(x, pos, w, cfg, table, prune_to=prune, tm=tm, kv_out=kv_out, trace=tr)
        if traces is not None:
            traces.append(tr)
    return x, pos


# ------------------------------------------------------------------- decode

class DecodeCaches:
    """Per-layer K/V caches for the decode phase: [capacity, Hkv, dh] bf16
    each, the first `lengths[l]` rows filled.  A prefill's (K, V) per layer
    (its candidates; [SPTS] Table 5) is copied in once, with room for
    `extra` generated tokens."""

    def __init__(self, kvs, extra):
        self.k, self.v, self.lengths = [], [], []
        for K, V in kvs:
            n = K.shape[0]
            kc = torch.empty((n + extra,) + tuple(K.shape[1:]), dtype=K.dtype, device=K.device)
            vc = torch.empty_like(kc)
            kc[:n].copy_(K)
            vc[:n].copy_(V)
            self.k.append(kc)
            self.v.append(vc)
            self.lengths.append(n)

    def nbytes(self):
        return sum(2 * l * k[0].numel() * k.element_size() for l, k in zip(self.lengths, self.k))

    def layer_table(self, layers):
        """The native step's per-layer pointer table, built once per list of
        weight dicts (keyed by the dicts' identities): replace a weight by
        passing a new dict, not by assigning into one already used here."""
        key = tuple(id(w) for w in layers)
        if getattr(self, "_table_key", None) != key:
            self._table = capi.decode_layer_table(layers, self.k, self.v)
            self._table_key = key
        return self._table


def decode_step(x, pos, layers, caches: DecodeCaches, cfg: LayerConfig, rope_table, tm=NO_TIMER):
    """One new token (residual row x [d] bf16, updated in place) at original
    position pos through every layer; layer l's K/V row is written into its
    cache and its query attends to every cached row.  Layer l uses weights
    layers[l % len(layers)]."""
    Hq, Hkv, dh = cfg.Hq, cfg.Hkv, cfg.dh
    d = x.shape[0]
    rope = cfg.theta is not None
    for li in range(len(caches.k)):
        w = layers[li % len(layers)]
        L = caches.lengths[li]
        xt = capi.spts_rmsnorm(x.view(1, d), cfg.eps).view(d) if cfg.prenorm else x
        with tm("dec_qkv", 2.0 * d * (Hq + 2 * Hkv) * dh):        # weight bytes read
            if rope:
                q = capi.spts_decode_linear_rope(xt, w["wq"], pos, rope_table)
                capi.spts_decode_linear_rope(xt, w["wk"], pos, rope_table, out=caches.k[li][L].view(-1))
            else:
                q = capi.spts_decode_linear(xt, w["wq"])
                capi.spts_decode_linear(xt, w["wk"], out=caches.k[li][L].view(-1))
            capi.spts_decode_linear(xt, w["wv"], out=caches.v[li][L].view(-1))
        caches.lengths[li] = L + 1
        with tm("dec_attention", 2.0 * 2 * (L + 1) * Hkv * dh):   # cache bytes read (K and V)
            o = capi.spts_decode_attention(q.view(Hq, dh), caches.k[li], caches.v[li], L + 1)
        with tm("dec_o_proj", 2.0 * Hq * dh * d):
            capi.spts_decode_linear(o.view(-1), w["wo"], out=x, accumulate=True)
        z = capi.spts_rmsnorm(x.view(1, d), cfg.eps).view(d) if cfg.prenorm else x
        f = w["wg"].shape[0]
        with tm("dec_ffn", 2.0 * 3 * d * f):
            h = capi.spts_decode_swiglu(z, w["wg"], w["wu"])
            capi.spts_decode_linear(h, w["wd"], out=x, accumulate=True)
    return x


def decode_step_native(x, pos, layers, caches: DecodeCaches, cfg: LayerConfig, rope_table):
    """decode_step as one library call (spts_decode_step): the same layer
    arithmetic, with the norms fused into the projections and the three
    projections of a layer in one launch."""
    f = layers[0]["wg"].shape[0]
    return capi.spts_decode_step(x, pos, caches.layer_table(layers), caches.lengths, cfg.Hq, cfg.Hkv, cfg.dh, f,
                                 cfg.eps, cfg.prenorm, rope_table if cfg.theta is not None else None)


def msdp_stack(x0, layers, cfg: LayerConfig, points, fused=True, traces=None, tm=NO_TIMER):
    """Run the stack on embeddings x0 [N, d] (not modified).  Returns the
    residual over the final candidates and their original positions."""
    N = x0.shape[0]
    # Layer 0 only reads the residual until its MSDP boundary, and the
    # boundary gathers the kept rows into a new tensor; so when layer 0 prunes,
    # x0 itself can be its input.  Otherwise the stack writes into a copy.
    first = points.get(0)
    copy_x0 = first is None or first >= N
    with tm("stack_setup", 4.0 * x0.numel() if copy_x0 else 4.0 * N):
        x = x0.clone() if copy_x0 else x0
        pos = torch.arange(N, dtype=torch.int32, device=x0.device)
        table = capi.spts_rope_table(N, cfg.dh, cfg.theta, x0.device) if cfg.theta is not None else None
    for li, w in enumerate(layers):
        budget = points.get(li)
        prune = budget if budget is not None and budget < x.shape[0] else None
        tr = {} if traces is not None else None
        x, pos = spts_layer(x, pos, w, cfg, table, prune_to=prune, fused=fused, trace=tr, tm=tm)
        if traces is not None:
            traces.append(tr)
    return x, pos
