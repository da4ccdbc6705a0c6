"""Teacher-forced parity of one layer of the HIP path against the oracle.

Each step of the layer is checked on the GPU's own inputs to that step (the
trace a pipeline call records): the oracle recomputes the step from them and
the GPU's output must meet the bar.  This removes the drift of a free run
(an fp32 accumulation order that flips one bf16 rounding in a thousand), so
every selection is held to the 1e-5 window and every output to the bf16 bar
by its maximum error, at full size:

  step                        oracle input (from the GPU trace)     bar
  pre-norm xt                 x_in                                  bf16, every row
  K, V, probe Q               xt                                    bf16, sampled rows / all probes
  PAP score S                 probe Q, K                            fp32 (1e-4), score mass Hq*P
  MSDP keep                   S                                     1e-5 window; K, V, S, pos compacted exactly
  attention selection idx     S over the kept candidates            1e-5 window
  Q of selected rows          xt                                    bf16, sampled rows
  reduced attention O         Q of those rows, K, V                 bf16, sampled rows
  residual after attention    x_in, O                               bf16, sampled rows; the rest bit-identical
  FFN pre-norm z              residual after attention              bf16, every row
  LTP score L                 z                                     fp32 (1e-4), 2e-5 per row
  fused score                 the GPU's S and L                     bit-exact (same fp32 operations)
  FFN selection idx_f         oracle S and L, fused in fp32, and    1e-5 window
                              fused by the float64 definition
  layer output                z, residual after attention           bf16, sampled rows; the rest bit-identical

"Sampled rows" are at least 64 rows per check, including the first and last
selected rows.
"""

import numpy as np

from oracle import layer as olayer, numerics, pap, select, attention, ltp, ffn, normrope
from parity import np64, max_rel_err, window_violations, BF16_REL, F32_REL

import workloads as W


STRUCTURED_KEYS = ("a_g_t", "b_g_t", "a_u_t", "b_u_t", "c_t", "d_t")


def _rows_bar(got, ref, what, rel=BF16_REL):
    """bf16 bar row by row: every row's max error within rel of that row's
    max reference magnitude, and the whole set within rel of its max."""
    got = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    scale = np.abs(ref).max(axis=1)
    scale[scale == 0] = 1.0
    per_row = np.abs(got - ref).max(axis=1) / scale
    worst = float(per_row.max()) if len(per_row) else 0.0
    assert worst <= rel, f"{what}: worst row max|err|/max|ref| = {worst:.3e} > {rel:.1e}"
    return worst


def _sample(n, count, rng, must=()):
    count = min(n, count)
    pick = set(rng.choice(n, count, replace=False).tolist()) | {int(m) for m in must if 0 <= m < n}
    return np.array(sorted(pick), dtype=np.int64)


def check_layer(tr, w, cfg, prune_to=None, n_sample=64, seed=0, log=print, k_given=False):
    """Teacher-forced checks of one SPTS layer.

    tr: trace dict of a pipeline.spts_layer call (GPU tensors).  w: the
    layer's bf16 weights (CPU tensors).  cfg: dict with Hq, Hkv, dh, P,
    keep_attn, keep_ffn (None: attention only), prenorm, eps, theta, w_fuse,
    fusion.  prune_to: the MSDP budget of this layer (None: no boundary).
    k_given: the keys were an input (no K projection to check).
    Returns a dict of the worst errors seen, for the log."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, dh, P = cfg["Hq"], cfg["Hkv"], cfg["dh"], cfg["P"]
    theta = cfg.get("theta")
    prenorm = cfg.get("prenorm", False)
    eps = cfg.get("eps", 1e-5)
    scale = dh ** -0.5
    w64 = {k: W.as_f64(v) for k, v in w.items() if k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd", "u_t", "v_t")
           + STRUCTURED_KEYS}
    out = {}

    x_in = np64(tr["x_in"])
    pos_in = tr["pos_in"].cpu().numpy().astype(np.int64)
    n_in = x_in.shape[0]

    # ---- pre-norm
    if prenorm:
        xt = np64(tr["xt"])
        out["xt"] = _rows_bar(xt, numerics.bf16(normrope.rmsnorm(x_in, eps)), "pre-norm xt")
    else:
        xt = x_in

    # ---- K, V, probe queries from the GPU's xt
    K_pre = np64(tr["K_pre"]).reshape(n_in, Hkv, dh)
    # at an MSDP boundary the pipeline projects V only for the kept rows,
    # after the pruning (V_pre is then None and V is checked below)
    V_pre = np64(tr["V_pre"]).reshape(n_in, Hkv, dh) if tr["V_pre"] is not None else None
    rows = _sample(n_in, n_sample, rng, must=(0, n_in - 1))
    if not k_given:
        out["K"] = _rows_bar(K_pre[rows], olayer.project(xt[rows], w64["wk"], Hkv, dh, pos_in[rows], theta), "K")
    if V_pre is not None:
        out["V"] = _rows_bar(V_pre[rows], olayer.project(xt[rows], w64["wv"], Hkv, dh), "V")
    Qp = np64(tr["Qp"]).reshape(P, Hq, dh)
    out["Qp"] = _rows_bar(Qp, olayer.project(xt[-P:], w64["wq"], Hq, dh, pos_in[-P:], theta), "probe Q")

    # ---- PAP score on the GPU's probe queries and keys
    S_ref = pap.pap_scores(Qp, K_pre, scale)
    S_pre = np64(tr["S_pre"])
    out["S"] = max_rel_err(S_pre, S_ref)
    assert out["S"] <= F32_REL, f"PAP score: {out['S']:.3e}"
    assert abs(S_pre.sum() - Hq * P) <= 1e-4 * Hq * P, "PAP score mass"
    log(f"  S vs oracle on the GPU's Q, K: {out['S']:.2e}")

    # ---- MSDP boundary
    if prune_to is not None and prune_to < n_in:
        keep = tr["keep"].cpu().numpy().astype(np.int64)
        assert window_violations(S_ref, keep, prune_to, P) == 0, "MSDP keep outside the 1e-5 window"
        cand = keep
        assert np.array_equal(tr["pos"].cpu().numpy(), pos_in[keep]), "positions after the boundary"
        assert np.array_equal(np64(tr["K"]).reshape(-1, Hkv, dh), K_pre[keep]), "K compaction"
        if V_pre is not None:
            assert np.array_equal(np64(tr["V"]).reshape(-1, Hkv, dh), V_pre[keep]), "V compaction"
        assert np.array_equal(np64(tr["S"]), S_pre[keep]), "S compaction"
    else:
        cand = np.arange(n_in)
    n = len(cand)
    K = K_pre[cand]
    if V_pre is not None:
        V = V_pre[cand]
    else:
        # V of the kept rows, projected after the boundary from the same xt rows
        V = np64(tr["V"]).reshape(n, Hkv, dh)
        vr = _sample(n, n_sample, rng, must=(0, n - 1))
        out["V"] = _rows_bar(V[vr], olayer.project(xt[cand[vr]], w64["wv"], Hkv, dh), "V (kept rows)")
    S_c = S_ref[cand]
    pos = pos_in[cand]

    # ---- attention selection and the reduced attention
    k_a = numerics.keep_count(cfg["keep_attn"], n)
    idx = tr["idx"].cpu().numpy().astype(np.int64)
    assert window_violations(S_c, idx, k_a, P) == 0, "attention selection outside the 1e-5 window"
    sel = _sample(len(idx), n_sample, rng, must=(0, len(idx) - 1))
    qi = idx[sel]
    Qs = np64(tr["Qs"]).reshape(len(idx), Hq, dh)
    out["Qs"] = _rows_bar(Qs[sel], olayer.project(xt[cand[qi]], w64["wq"], Hq, dh, pos[qi], theta), "selected Q")
    O = np64(tr["O"]).reshape(len(idx), Hq, dh)
    O_ref = numerics.bf16(attention.reduced_attention(Qs[sel], qi, K, V, scale))
    out["O"] = _rows_bar(O[sel], O_ref, "reduced attention")
    log(f"  attention: Qs {out['Qs']:.2e}, O {out['O']:.2e} on {len(sel)} rows")

    # ---- residual after the attention block
    x_c = x_in[cand]
    x_mid = np64(tr["x_mid"]) if cfg.get("keep_ffn") is not None else np64(tr["x_out"])
    delta = numerics.bf16(O[sel].reshape(len(sel), Hq * dh) @ w64["wo"].T)
    out["x_mid"] = _rows_bar(x_mid[qi], numerics.bf16(x_c[qi] + delta), "residual after attention")
    skipped = np.ones(n, bool)
    skipped[idx] = False
    assert np.array_equal(x_mid[skipped], x_c[skipped]), "rows skipped by attention changed"
    if cfg.get("keep_ffn") is None:
        return out

    # ---- FFN block
    if prenorm:
        z = np64(tr["z"])
        out["z"] = _rows_bar(z, numerics.bf16(normrope.rmsnorm(x_mid, eps)), "FFN pre-norm z")
    else:
        z = x_mid
    L = np64(tr["L"])
    if cfg.get("proxy", "linear") == "structured":
        L_ref = ltp.ltp_structured_scores(z, *[w64[k] for k in STRUCTURED_KEYS])
        row_bar = 5e-5                  # three hi/lo stages of ~16 bits each
    else:
        L_ref = ltp.ltp_scores(z, w64["u_t"], w64["v_t"])
        row_bar = 2e-5
    out["L"] = max_rel_err(L, L_ref)
    assert out["L"] <= F32_REL, f"LTP score: {out['L']:.3e}"
    out["L_row"] = float((np.abs(L - L_ref) / L_ref).max())
    assert out["L_row"] < row_bar, f"LTP score per row: {out['L_row']:.3e}"
    # the GPU's fused score from its own S and L: same fp32 operations
    S_g = np.asarray(tr["S"].cpu().numpy(), dtype=np.float32)
    L_g = np.asarray(tr["L"].cpu().numpy(), dtype=np.float32)
    if cfg.get("fusion", "maxnorm_add") == "multiply":
        fused_g = select.fuse_multiply(S_g, L_g)
        fused_ref = select.fuse_multiply(numerics.f32(S_c), numerics.f32(L_ref))
    else:
        wa, wb = cfg.get("w_fuse", (0.5, 0.5))
        fused_g = select.fuse_maxnorm(S_g, L_g, wa, wb)
        fused_ref = select.fuse_maxnorm(numerics.f32(S_c), numerics.f32(L_ref), wa, wb)
    if tr.get("fused") is not None:
        assert np.array_equal(tr["fused"].cpu().numpy(), fused_g), "fused score"
    k_f = numerics.keep_count(cfg["keep_ffn"], n)
    idx_f = tr["idx_f"].cpu().numpy().astype(np.int64)
    assert window_violations(fused_ref.astype(np.float64), idx_f, k_f, P) == 0, \
        "FFN selection outside the 1e-5 window"
    # and against the fusion's plain float64 definition on the oracle's scores,
    # which does not depend on any fp32 operation order
    S64, L64 = np.asarray(S_c, dtype=np.float64), np.asarray(L_ref, dtype=np.float64)
    if cfg.get("fusion", "maxnorm_add") == "multiply":
        fused64 = S64 * L64
    else:
        fused64 = wa * S64 / S64.max() + wb * L64 / L64.max()
    assert window_violations(fused64, idx_f, k_f, P) == 0, "FFN selection outside the 1e-5 window (float64 fusion)"
    fsel = _sample(len(idx_f), n_sample, rng, must=(0, len(idx_f) - 1))
    fi = idx_f[fsel]
    _, y = ffn.swiglu_rows(z[fi], w64["wg"], w64["wu"], w64["wd"])
    x_out = np64(tr["x_out"])
    out["x_out"] = _rows_bar(x_out[fi], numerics.bf16(x_mid[fi] + y), "layer output (FFN rows)")
    fskip = np.ones(n, bool)
    fskip[idx_f] = False
    assert np.array_equal(x_out[fskip], x_mid[fskip]), "rows skipped by the FFN changed"
    log(f"  FFN: L {out['L']:.2e} (row {out['L_row']:.2e}), output {out['x_out']:.2e} on {len(fsel)} rows")
    return out


def check_dense_layer(tr, w, cfg, n_sample=64, seed=0, log=print):
    """Teacher-forced check of a dense layer (every row computed) on sampled
    output rows: the oracle's keep-all layer on the GPU's layer input, with
    every K/V row projected by the oracle (causal attention needs them all)."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, dh = cfg["Hq"], cfg["Hkv"], cfg["dh"]
    theta = cfg.get("theta")
    eps = cfg.get("eps", 1e-5)
    scale = dh ** -0.5
    w64 = {k: W.as_f64(v) for k, v in w.items() if k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}
    x_in = np64(tr["x_in"])
    pos = tr["pos_in"].cpu().numpy().astype(np.int64)
    n = x_in.shape[0]
    xt = numerics.bf16(normrope.rmsnorm(x_in, eps)) if cfg.get("prenorm") else x_in
    K = olayer.project(xt, w64["wk"], Hkv, dh, pos, theta)
    V = olayer.project(xt, w64["wv"], Hkv, dh)
    rows = _sample(n, n_sample, rng, must=(0, n - 1))
    Q = olayer.project(xt[rows], w64["wq"], Hq, dh, pos[rows], theta)
    O = numerics.bf16(attention.reduced_attention(Q, rows, K, V, scale))
    x_mid = numerics.bf16(x_in[rows] + numerics.bf16(O.reshape(len(rows), -1) @ w64["wo"].T))
    z = numerics.bf16(normrope.rmsnorm(x_mid, eps)) if cfg.get("prenorm") else x_mid
    _, y = ffn.swiglu_rows(z, w64["wg"], w64["wu"], w64["wd"])
    ref = numerics.bf16(x_mid + y)
    err = _rows_bar(np64(tr["x_out"])[rows], ref, "dense layer output")
    log(f"  dense layer output {err:.2e} on {len(rows)} rows")
    return err
