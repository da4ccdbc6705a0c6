"""Low-rank Transformation Probing (LTP) score -- test infrastructure only.

[SPTS] abstract and Fig. 2(b): LTP builds an offline low-rank proxy network
that predicts how the feed-forward block would transform each token, and
uses that predicted transformation to decide which tokens go through the
reduced feed-forward.  The page does not print the proxy's form for the hot
path; this build's reading is a rank-r linear proxy

    dX_hat_n = (z_n U) V,   U: d x r,   V: r x d,
    L_n = || dX_hat_n ||_2,

with U, V given in nn.Linear layout (u_t = U^T [r, d], v_t = V^T [d, r]).
The intermediate T = z U is not a storage point: it is kept at full
precision (a bfloat16 rounding there would move L by about 1e-5 relative).

[SPTS] Table A describes a structured proxy (D_low channels of the FFN, each
projection factored at rank r); `structured_proxy_delta` restates that form:
at full rank and all channels it is the SwiGLU block itself.
"""

import numpy as np


def ltp_scores(z, u_t, v_t):
    """z [n,d], u_t [r,d], v_t [d,r] -> L [n] = ||(z U) V||_2 per row (float64)."""
    z = np.asarray(z, dtype=np.float64)
    u_t = np.asarray(u_t, dtype=np.float64)
    v_t = np.asarray(v_t, dtype=np.float64)
    t = z @ u_t.T            # [n, r]
    dx = t @ v_t.T           # [n, d]
    return np.sqrt(np.einsum("nd,nd->n", dx, dx))


def structured_proxy_delta(z, gate_f, up_f, down_f, channels):
    """Table A's proxy form: FFN restricted to `channels` of the hidden dim,
    each projection given as a list of factors whose product is the weight.

    gate_f, up_f: lists of matrices whose product (left to right) is the
    [d, D_low] map z -> hidden (restricted channels); down_f: same for the
    [D_low, d] map back.  Returns the predicted delta [n, d].
    """
    z = np.asarray(z, dtype=np.float64)

    def apply(x, factors):
        for f in factors:
            x = x @ np.asarray(f, dtype=np.float64)
        return x

    g = apply(z, gate_f)
    u = apply(z, up_f)
    h = (g / (1.0 + np.exp(-g))) * u
    return apply(h, down_f)


def ltp_structured_scores(z, a_g_t, b_g_t, a_u_t, b_u_t, c_t, d_t):
    """Score of the structured proxy: L_n = ||dX_hat_n||_2 with dX_hat from
    `structured_proxy_delta`, every projection given as two nn.Linear-layout
    factors (gate: a_g_t [r, d] then b_g_t [D_low, r]; up likewise; down:
    c_t [r, D_low] then d_t [d, r])."""
    t = lambda w: np.asarray(w, dtype=np.float64).T
    dx = structured_proxy_delta(z, [t(a_g_t), t(b_g_t)], [t(a_u_t), t(b_u_t)], [t(c_t), t(d_t)], None)
    return np.sqrt(np.einsum("nd,nd->n", dx, dx))
