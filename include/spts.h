/*
 * spts.h -- C ABI of the SPTS prefill hot path on AMD Instinct MI355X (gfx950).
 *
 * Method: "Probe and Skip: Self-Predictive Token Skipping for Efficient
 * Long-Context LLM Inference" (Wu, Wang, Jin, Chen, Wang), cited as [SPTS].
 * Partial Attention Probing (PAP) scores tokens for the attention block,
 * Low-rank Transformation Probing (LTP) scores them for the FFN block, the
 * selected tokens run a reduced attention / reduced SwiGLU, skipped tokens
 * keep their residual, and Multi-Stage Delayed Pruning (MSDP) shrinks the
 * candidate set at stage boundaries ([SPTS] abstract, Fig. 2).
 *
 * Conventions shared by every call
 *   - Tensors are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or retains them beyond the call's stream work.
 *   - Layouts are row-major and token-major.  Weights use the nn.Linear
 *     layout [out_features, in_features].  "bf16" is IEEE bfloat16 stored in
 *     16 bits; accumulation is fp32.
 *   - Index arrays are int32, strictly ascending, in [0, n), except where a
 *     call says otherwise.
 *   - Every compute call is asynchronous on the context's stream (a HIP
 *     stream borrowed from the caller, never destroyed here) and returns a
 *     status.  Arguments are validated on the host before anything is
 *     launched; a failing validation launches nothing.  A launch failure
 *     returns SPTS_ERR_HIP; faults inside kernels surface at the caller's
 *     next synchronisation or at spts_check().
 *   - Calls that need temporary device memory take it from the context's
 *     workspace (spts_set_workspace); the required size is given by the
 *     matching *_workspace() query, and a smaller workspace returns
 *     SPTS_ERR_NOMEM.  Each call uses the workspace from offset 0, so calls
 *     on one context must not run concurrently (one context per stream).
 *   - Pointers must be 16-byte aligned (SPTS_ERR_ALIGN otherwise).
 *   - No C++ exception crosses this interface.
 */
#ifndef SPTS_H
#define SPTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spts_status {
    SPTS_OK = 0,
    SPTS_ERR_INVALID = 1,      /* null pointer, bad context, bad enum      */
    SPTS_ERR_SHAPE = 2,        /* sizes inconsistent or out of range       */
    SPTS_ERR_DTYPE = 3,        /* dtype not accepted by this call          */
    SPTS_ERR_ALIGN = 4,        /* pointer not 16-byte aligned              */
    SPTS_ERR_NOMEM = 5,        /* workspace smaller than the call needs    */
    SPTS_ERR_HIP = 6,          /* HIP runtime reported an error            */
    SPTS_ERR_UNSUPPORTED = 7   /* valid, but outside what the kernels do   */
} spts_status;

typedef enum spts_dtype { SPTS_BF16 = 0, SPTS_F32 = 1, SPTS_I32 = 2 } spts_dtype;

typedef struct spts_ctx spts_ctx;

/* ------------------------------------------------------------- context */

/* Create a context bound to `hip_stream` (a hipStream_t; NULL = default
 * stream).  The stream is borrowed.  Returns SPTS_ERR_INVALID if ctx is NULL. */
spts_status spts_create(spts_ctx** ctx, void* hip_stream);
/* Destroy a context (does not synchronise or destroy the stream). */
spts_status spts_destroy(spts_ctx* ctx);
/* Rebind the context to another borrowed stream. */
spts_status spts_set_stream(spts_ctx* ctx, void* hip_stream);
/* Give the context `bytes` of caller-owned device memory for temporaries. */
spts_status spts_set_workspace(spts_ctx* ctx, void* dev_ptr, size_t bytes);
/* Text of the last error on this context ("" if none).  Owned by ctx. */
const char* spts_last_error(const spts_ctx* ctx);
/* Name of a status code, e.g. "SPTS_ERR_SHAPE". */
const char* spts_status_name(spts_status s);
/* Synchronise the context's stream and report any pending HIP error. */
spts_status spts_check(spts_ctx* ctx);

/* ------------------------------------------------------ workspace sizes */

size_t spts_probe_attention_workspace(int n, int P, int Hq);
size_t spts_score_topk_workspace(int n);
size_t spts_ltp_probe_workspace(int n, int d, int r);
size_t spts_ltp_structured_workspace(int n, int d, int r, int d_low);
size_t spts_ltp_gram_workspace(int n, int d, int r);
size_t spts_decode_attention_workspace(int L, int Hq);
size_t spts_decode_step_workspace(int max_len, int Hq, int f);
size_t spts_reduced_ffn_workspace(int k, int d, int f);
size_t spts_msdp_stage_workspace(int n_prev);
/* Workspace with which spts_linear / spts_linear_rope, spts_linear_kv and
 * spts_linear_swiglu split the inner dimension across workgroups; 0 when the
 * problem runs unsplit.  The split is either of every 256 x 256 output tile
 * (linear / rope only) or of the tiles of the last, partly filled round of
 * workgroups over the 256 CUs, so that round fills the chip.  The fp32
 * partial sums are added in a fixed order, so a given problem always gives
 * the same result; a smaller workspace makes the call run unsplit (same
 * result up to the order of the fp32 additions, possibly slower). */
size_t spts_linear_workspace(int m, int kdim, int n);
size_t spts_linear_kv_workspace(int m, int kdim, int nk, int nv);
size_t spts_linear_swiglu_workspace(int m, int kdim, int f);

/* ----------------------------------------------------------------- PAP */

/* Partial Attention Probing score ([SPTS] Fig. 2(a), abstract).
 * The probe rows are the last P of the n current candidate rows; probe p
 * (row n-P+p) attends keys 0..n-P+p with softmax(scale * q.k), query head h
 * using key head h / (Hq/Hkv).  Output, for every row j:
 *     scores[j] = sum over heads h and probes p of that softmax weight.
 *   q_probe [P, Hq, dh]   dtype
 *   k       [n, Hkv, dh]  dtype
 *   scores  [n]           float32, written
 * dtype SPTS_BF16: dh == 128, P % 32 == 0, (Hq/Hkv) % 4 == 0 (MFMA path).
 * dtype SPTS_F32 : dh <= 128, any P (plain fp32 path for small cases).
 * Workspace: spts_probe_attention_workspace(n, P, Hq). */
spts_status spts_probe_attention(spts_ctx* ctx, spts_dtype dtype, const void* q_probe,
                                 const void* k, int n, int P, int Hq, int Hkv, int dh,
                                 float scale, float* scores);

/* --------------------------------------------------------------- select */

/* Top-k token selection ([SPTS] Fig. 2(a)(b); fusion: Table D "MaxNorm-Add").
 * Ranking score: s_a if s_b == NULL, else the float32 value
 *     c = fl(fl(w_a*fl(s_a/max s_a)) + fl(w_b*fl(s_b/max s_b)))
 * (the maxima are taken over all n rows and ignore NaN; a term is 0 when
 * its max is not positive).  The last n_forced rows are
 * always kept and count toward k; the other k-n_forced rows are the largest
 * ranking scores among rows 0..n-n_forced-1, ties to the lower index; NaN
 * ranks lowest and -0 equals +0.  idx[0..min(k,n)-1] receives the kept rows
 * in ascending order.  fused_out [n] (optional) receives c.
 * Requires 0 <= n_forced <= k, n_forced <= n, n >= 1.
 * Workspace: spts_score_topk_workspace(n). */
spts_status spts_score_topk(spts_ctx* ctx, const float* s_a, const float* s_b, float w_a,
                            float w_b, int n, int k, int n_forced, int32_t* idx,
                            float* fused_out);

/* spts_score_topk without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, rules and results as
 * spts_score_topk; the context's workspace is not used.  A selection over
 * more than 32768 scores keeps its radix histograms and counters (about
 * 29 KiB) in a static device array of the library (4 MiB, one per GPU, held
 * until the process ends) instead of the workspace; nothing is allocated or
 * freed.  Every call
 * on one GPU shares that array, so calls that overlap on one GPU (on
 * different streams or host threads) race; calls in one stream's order do
 * not.  Requires n <= 1048576 (SPTS_ERR_UNSUPPORTED otherwise). */
spts_status spts_score_topk_noalloc(spts_ctx* ctx, const float* s_a, const float* s_b, float w_a,
                                    float w_b, int n, int k, int n_forced, int32_t* idx,
                                    float* fused_out);

/* spts_score_topk (one score, no fusion) on `batch` independent rows in one
 * launch, one workgroup per row: row b reads s + b * s_stride and writes
 * min(k, n) ascending indices to idx + b * idx_stride (same rule: last
 * n_forced rows forced, ties to the lower index).  Requires n <= 32768 (a
 * row's keys stay in registers; no workspace); strides in elements, at
 * least the row lengths (rows are read and written 4 bytes at a time, so
 * only s and idx themselves must be 16-byte aligned).  batch == 0 is a no-op. */
spts_status spts_score_topk_batched(spts_ctx* ctx, const float* s, int64_t s_stride, int batch, int n,
                                    int k, int n_forced, int32_t* idx, int64_t idx_stride);

/* As spts_score_topk with Table D's "Multiply" fusion, the pages' default
 * (the criterion C^FFN * S^MHA of [SPTS] Table 6): ranking score
 *     c = fl(s_a * s_b)   (one float32 product; s_b required),
 * same forcing, tie, NaN and order rules.  fused_out [n] (optional) receives c.
 * Workspace: spts_score_topk_workspace(n). */
spts_status spts_score_topk_multiply(spts_ctx* ctx, const float* s_a, const float* s_b, int n,
                                     int k, int n_forced, int32_t* idx, float* fused_out);

/* --------------------------------------------------------- gather/scatter */

/* dst[i, :] = src[idx[i], :] for i < k; rows of row_elems elements.
 * dtype BF16, F32 or I32.  src and dst must not overlap. */
spts_status spts_gather(spts_ctx* ctx, spts_dtype dtype, const void* src, const int32_t* idx,
                        int k, int row_elems, void* dst);

/* accumulate == 0:  dst[idx[i], :] = src[i, :]
 * accumulate == 1:  dst[idx[i], :] = dst[idx[i], :] + src[i, :]  (bf16: the
 *                   sum is formed in fp32 and rounded to bf16 once).
 * Rows of dst not named in idx are untouched -- the skipped tokens' residual
 * passes through unchanged ([SPTS] Fig. 2 top).  idx entries distinct. */
spts_status spts_scatter(spts_ctx* ctx, spts_dtype dtype, const void* src, const int32_t* idx,
                         int k, int row_elems, void* dst, int accumulate);

/* ----------------------------------------------------- reduced attention */

/* Reduced attention of the selected rows ([SPTS] Fig. 2(a)).  Query i sits
 * at candidate row idx[i] and attends, causally, rows 0..idx[i] of the keys
 * and values of ALL n current candidates:
 *     o_sel[i,h] = sum_{j<=idx[i]} softmax_j(scale*q_sel[i,h].k[j,g]) v[j,g],
 *     g = h / (Hq/Hkv).
 *   q_sel [kq, Hq, dh], k and v [n, Hkv, dh], o_sel [kq, Hq, dh]; all dtype.
 * idx may be in any order and may repeat rows: each query's causal range
 * comes from its own row (ascending idx, as selections produce, is fastest).
 * dtype SPTS_BF16: dh == 128, (Hq/Hkv) % 4 == 0, n*Hkv*dh < 2^31.
 * SPTS_F32: dh <= 128. */
spts_status spts_reduced_attention(spts_ctx* ctx, spts_dtype dtype, const void* q_sel,
                                   const int32_t* idx, const void* k, const void* v, int kq,
                                   int n, int Hq, int Hkv, int dh, float scale, void* o_sel);

/* ------------------------------------------------------------------ LTP */

/* Low-rank Transformation Probing score ([SPTS] Fig. 2(b), abstract):
 *     score[m] = || (z[m,:] U) V ||_2,   U = u_t^T (d x r), V = v_t^T (r x d)
 * with z U kept near fp32 precision (split into two bf16 terms).
 *   z [n, d] bf16, u_t [r, d] bf16, v_t [d, r] bf16, score [n] float32.
 * Requires d % 256 == 0, r % 256 == 0.  Workspace: spts_ltp_probe_workspace. */
spts_status spts_ltp_probe(spts_ctx* ctx, const void* z, const void* u_t, const void* v_t,
                           int n, int d, int r, float* score);

/* The same score through the Gram matrix of the proxy's second factor:
 *     score[m]^2 = t G t^T,   t = z[m,:] U (1 x r),   G = V V^T (r x r),
 * which equals ||t V||^2 exactly, so the (n x r) x (r x d) product becomes an
 * (n x r) x (r x r) one.  G depends only on the proxy, which the method builds
 * offline ([SPTS] abstract, Fig. 2(b)), so it is prepared once per proxy by
 * spts_ltp_gram and passed in here.  t is kept near fp32 precision (two bf16
 * terms); G as two bf16 terms (hi, lo); the product t G drops only the
 * lo(t) lo(G) term (~2^-18 relative).  For a positive semi-definite G that
 * rounds to a value just below 0 the score is 0.
 *   z [n, d] bf16, u_t [r, d] bf16, gram [r, 3r] bf16 from spts_ltp_gram,
 *   score [n] float32.
 * Requires d % 256 == 0, r % 256 == 0.  Workspace: spts_ltp_gram_workspace. */
spts_status spts_ltp_probe_gram(spts_ctx* ctx, const void* z, const void* u_t, const void* gram,
                                int n, int d, int r, float* score);

/* Offline preparation for spts_ltp_probe_gram: G = V V^T from v_t = V^T
 * [d, r] bf16, accumulated in fp64 (G is symmetric bit for bit), written to
 * gram [r, 3r] bf16 as rows [hi(G) | hi(G) | lo(G)], hi = bf16(G),
 * lo = bf16(G - hi).  The buffer belongs to the caller and stays valid while
 * v_t is unchanged.  Requires r % 256 == 0, d > 0.  No workspace. */
spts_status spts_ltp_gram(spts_ctx* ctx, const void* v_t, int d, int r, void* gram);

/* The structured proxy form of [SPTS] Table A: the feed-forward restricted to
 * d_low of its hidden channels, each projection factored at rank r
 * (r * (d + d_low) multiply-accumulates per projection and token):
 *     g = (z A_g) B_g,  u = (z A_u) B_u       (d -> r -> d_low)
 *     h = silu(g) * u
 *     score[m] = || (h C) D ||_2               (d_low -> r -> d)
 * The factors come packed in nn.Linear layout (blocks of r columns):
 *     a_gu_t [2r, d]     = [A_g^T ; A_u^T]
 *     b_gate [d_low, 4r] = [B_g^T | 0 | B_g^T | 0]
 *     b_up   [d_low, 4r] = [0 | B_u^T | 0 | B_u^T]
 *     c_t    [r, d_low]  = C^T,   d_t [d, r] = D^T
 * z A, h and h C are kept near fp32 precision (each split into two bf16 terms;
 * the zero blocks route the terms of the gate and up halves).
 *   z [n, d] bf16, score [n] float32.
 * Requires d, r, d_low multiples of 256.  Workspace: spts_ltp_structured_workspace. */
spts_status spts_ltp_probe_structured(spts_ctx* ctx, const void* z, const void* a_gu_t,
                                      const void* b_gate, const void* b_up, const void* c_t,
                                      const void* d_t, int n, int d, int r, int d_low,
                                      float* score);

/* The structured score with its last factor through D's Gram matrix:
 * score[m]^2 = u G u^T, u = h[m,:] C, G = D D^T, equal to ||u D||^2 (the
 * rounding as in spts_ltp_probe_gram).  gram [r, 3r] bf16 is spts_ltp_gram
 * of d_t, prepared once per proxy; the other arguments and the workspace
 * (spts_ltp_structured_workspace) are those of spts_ltp_probe_structured. */
spts_status spts_ltp_probe_structured_gram(spts_ctx* ctx, const void* z, const void* a_gu_t,
                                           const void* b_gate, const void* b_up, const void* c_t,
                                           const void* gram, int n, int d, int r, int d_low,
                                           float* score);

/* ------------------------------------------------------------- reduced FFN */

/* Reduced SwiGLU feed-forward ([SPTS] Fig. 2(b)) on k selected rows:
 *     H = bf16(silu(Z Wg^T) * (Z Wu^T)),  Y = bf16(H Wd^T)
 * where Z[i] = z[rows[i]] if rows != NULL (gather on load), else z[i].
 * Output row i goes to y[o(i)], o(i) = y_rows[i] if y_rows != NULL (scatter
 * on store), else i; accumulate == 1 stores bf16(y[o(i)] + Y[i]) (the
 * residual add of the selected tokens), accumulate == 0 stores Y[i].
 *   z [*, d] bf16, w_gate, w_up [f, d], w_down [d, f], y [*, d] bf16.
 * y must not alias the rows of z being read when y_rows == NULL.
 * Requires d % 256 == 0, f % 128 == 0, and each weight below 4 GiB.
 * Workspace: spts_reduced_ffn_workspace(k, d, f) bytes = H [k, f] bf16 plus
 * the fp32 pieces with which the two GEMMs split their last, partly filled
 * round of tiles along the inner dimension (as spts_linear_swiglu and
 * spts_linear do).  At least the H part (k*f*2 bytes rounded up to 256) is
 * required (SPTS_ERR_NOMEM otherwise); with less than the full size a GEMM
 * whose split does not fit runs unsplit (same result up to the order of
 * the fp32 additions). */
spts_status spts_reduced_ffn(spts_ctx* ctx, const void* z, const int32_t* rows, const void* w_gate,
                             const void* w_up, const void* w_down, int k, int d, int f, void* y,
                             const int32_t* y_rows, int accumulate);

/* ------------------------------------------------------------------- MSDP */

/* Stage-boundary pruning ([SPTS] Fig. 2(c), Fig. A(c)): keep the `budget`
 * candidates of the n_prev current ones ranked by `scores` (last n_forced
 * forced, same rule as spts_score_topk), write
 *     keep[0..budget-1]  ascending indices into the previous candidate list,
 *     pos_new[i] = pos_prev[keep[i]],
 *     x_new[i,:] = x_prev[keep[i],:]   (bf16 rows of d, if x_prev != NULL).
 * Workspace: spts_msdp_stage_workspace(n_prev). */
spts_status spts_msdp_stage(spts_ctx* ctx, const float* scores, int n_prev, int budget,
                            int n_forced, const int32_t* pos_prev, int32_t* keep,
                            int32_t* pos_new, const void* x_prev, void* x_new, int d);

/* ------------------------------------- projections and layer glue (bf16) */

/* out = A W^T on bf16 MFMA, fp32 accumulate, bf16 result.
 *   A row i = a[a_rows[i]] if a_rows != NULL (gather on load), else a[i]; A is
 *   [m, kdim], W is [n, kdim].
 *   accumulate == 0: out[o(i), :] = bf16(A W^T)[i]
 *   accumulate == 1: out[o(i), :] = bf16(out[o(i), :] + bf16(A W^T)[i])
 *   with o(i) = out_rows[i] if out_rows != NULL (scatter on store), else i.
 * Requires kdim % 64 == 0, n % 256 == 0, and W below 4 GiB (n*kdim*2 < 2^32;
 * the same bound holds for every weight of the calls below, else
 * SPTS_ERR_UNSUPPORTED).  A (gathered or not) may span any size.  These
 * projections are needed because every step of the path runs in this library.
 * Workspace (optional): spts_linear_workspace (spts_linear_rope too). */
spts_status spts_linear(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m, int kdim,
                        const void* w, int n, void* out, const int32_t* out_rows, int accumulate);

/* As spts_linear (accumulate 0, no out_rows) with rotary embedding applied to
 * the fp32 result before rounding: heads of 128 columns, pair (c, c+64) of a
 * head rotated by table[p, c] = (cos, sin) of p * theta^(-2c/128), where p =
 * pos[a_rows ? a_rows[i] : i].  table from spts_rope_table. */
spts_status spts_linear_rope(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m,
                             int kdim, const void* w, int n, void* out, const int32_t* pos,
                             const float* table);

/* Keys and values of the same rows in one launch -- every current candidate
 * keeps its K and V for the reduced attention ([SPTS] Fig. 2(a)):
 *     k_out[i, :] = bf16(RoPE(A Wk^T))[i]   (no rotation if table == NULL)
 *     v_out[i, :] = bf16(A Wv^T)[i],         A row i = a[a_rows ? a_rows[i] : i]
 *   a [*, kdim] bf16; wk [nk, kdim], wv [nv, kdim] bf16; k_out [m, nk],
 *   v_out [m, nv] bf16.  RoPE as in spts_linear_rope (pos, table required
 *   together).  Results agree with spts_linear_rope / spts_linear on the same
 *   inputs up to the order of the fp32 additions; one launch fills the GPU
 *   better than two thin ones.
 * Requires kdim % 64 == 0, nk % 256 == 0, nv % 256 == 0.
 * Workspace (optional): spts_linear_kv_workspace. */
spts_status spts_linear_kv(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m, int kdim,
                           const void* wk, int nk, const void* wv, int nv, void* k_out,
                           void* v_out, const int32_t* pos, const float* table);

/* The first half of the reduced FFN as its own call:
 *     h_out[i, :] = bf16(silu(A Wg^T) * (A Wu^T))[i],  A row i = a[a_rows ? a_rows[i] : i]
 *   a [*, kdim] bf16, w_gate, w_up [f, kdim] bf16, h_out [m, f] bf16.
 * Requires kdim % 64 == 0, f % 128 == 0.  ([SPTS] Fig. 2(b), reduced feed-forward.)
 * Workspace (optional): spts_linear_swiglu_workspace. */
spts_status spts_linear_swiglu(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m, int kdim,
                               const void* w_gate, const void* w_up, int f, void* h_out);

/* ------------------------------------------------------------------ decode */

/* Decode phase: one new token per step through every layer.  With MSDP each
 * layer keeps the K/V of its candidates only ([SPTS] Table 5, Fig. A(c)), so
 * the new token attends to that layer's cache.  One token row x [kdim] bf16.
 * Projections (HBM-bound matrix-vector products, fp32 accumulate):
 *   spts_decode_linear:      out[c] = bf16(x . w[c,:]); accumulate == 1:
 *                            out[c] = bf16(out[c] + bf16(x . w[c,:]))  (residual add)
 *   spts_decode_linear_rope: as store, then RoPE at position pos on 128-wide
 *                            heads (pairs c, c+64); table from spts_rope_table
 *                            must hold row pos (the caller sizes it to the
 *                            prompt plus every generated token)
 *   spts_decode_swiglu:      h[c] = bf16(silu(x . w_gate[c,:]) * (x . w_up[c,:]))
 *   w [n, kdim] bf16; out [n] bf16.  Requires kdim % 512 == 0, kdim <= 16384;
 *   x and w 16-byte aligned.  Errors: SPTS_ERR_INVALID (null pointer, bad
 *   flag), SPTS_ERR_SHAPE, SPTS_ERR_UNSUPPORTED, SPTS_ERR_ALIGN. */
spts_status spts_decode_linear(spts_ctx* ctx, const void* x, const void* w, int kdim, int n, void* out,
                               int accumulate);
spts_status spts_decode_linear_rope(spts_ctx* ctx, const void* x, const void* w, int kdim, int n,
                                    void* out, int pos, const float* table);
spts_status spts_decode_swiglu(spts_ctx* ctx, const void* x, const void* w_gate, const void* w_up,
                               int kdim, int f, void* h_out);
/* One query row against a layer's cache, every cached row visible:
 *   o[h] = sum_j softmax_j(scale * q[h] . k_cache[j, g]) v_cache[j, g],  g = h / (Hq/Hkv),
 *   j < L.  q [Hq, 128], k_cache, v_cache [>= L, Hkv, 128], o [Hq, 128], bf16.
 * Split over chunks of keys (a multiple of 64, sized for about 512
 * workgroups); a second launch merges the chunk partials in chunk order.
 * Requires dh == 128, Hq/Hkv == 4.  Workspace:
 * spts_decode_attention_workspace(L, Hq). */
spts_status spts_decode_attention(spts_ctx* ctx, const void* q, const void* k_cache,
                                  const void* v_cache, int L, int Hq, int Hkv, int dh, float scale,
                                  void* o);

/* One layer's weights and cache for spts_decode_step (device pointers, bf16,
 * 16-byte aligned, owned by the caller): wq [Hq*dh, d], wk, wv [Hkv*dh, d],
 * wo [d, Hq*dh], w_gate, w_up [f, d], w_down [d, f]; k_cache, v_cache
 * [cap, Hkv, dh] rows of this layer's cache. */
typedef struct spts_decode_layer {
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* k_cache;
  void* v_cache;
  int cap;
} spts_decode_layer;

/* A whole decode step in one call: the new token's residual row x [d] (bf16,
 * device, updated in place) at position pos through layers[0 .. n_layers) in
 * order.  Per layer, with z = RMSNorm(x) when prenorm (unit gain, eps) else x:
 *   q, k, v = z Wq^T, z Wk^T, z Wv^T (RoPE at pos on q and k when rope_table
 *   is not NULL); k, v go to row lengths[l] of the layer's cache;
 *   x += Wo decode_attention(q, rows 0 .. lengths[l]);
 *   x += Wd (silu(z' Wg^T) * (z' Wu^T)),  z' = RMSNorm(x) when prenorm,
 * each product rounded to bf16 as in the single calls above (the decode
 * phase of [SPTS] Fig. A(c): every layer attends to its own cache, which after
 * MSDP holds that layer's candidates, Table 5).  lengths: host int[n_layers],
 * rows filled in each cache, incremented on success.  rope_table: from
 * spts_rope_table with table_rows rows (pos < table_rows), or NULL.
 * Requires dh == 128, Hq/Hkv == 4; d, f and Hq*dh multiples of 512, at most
 * 16384; lengths[l] < cap for every layer.  Every argument is checked before
 * the first launch: on an error nothing runs and lengths is unchanged.
 * Workspace: spts_decode_step_workspace(1 + max lengths[l], Hq, f). */
spts_status spts_decode_step(spts_ctx* ctx, void* x, int d, int pos, const spts_decode_layer* layers,
                             int n_layers, int* lengths, int Hq, int Hkv, int dh, int f, float eps,
                             int prenorm, const float* rope_table, int table_rows, float scale);

/* table[p, c, 0..1] = (cos, sin)(p * theta^(-2c/dh)) for p < max_pos, c < dh/2,
 * angle formed in fp64 and rounded to fp32. */
spts_status spts_rope_table(spts_ctx* ctx, int max_pos, int dh, double theta, float* table);

/* out[i,:] = bf16(x[i,:] / sqrt(mean(x[i,:]^2) + eps)), unit gain.  d % 8 == 0. */
spts_status spts_rmsnorm(spts_ctx* ctx, const void* x, int n, int d, float eps, void* out);

#ifdef __cplusplus
}
#endif

#endif /* SPTS_H */
