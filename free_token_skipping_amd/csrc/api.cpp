// C-ABI host layer: argument validation, workspace carving and kernel launch
// for every call declared in include/spts.h.  Validation runs on the host
// before anything is enqueued; no exception leaves this file.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "../../include/spts.h"
#include "kernels.hpp"

struct spts_ctx {
  hipStream_t stream;
  void* ws;
  size_t ws_bytes;
  char err[512];
};

namespace {

using namespace spts;

spts_status fail(spts_ctx* c, spts_status st, const char* fmt, ...) {
  if (c) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(c->err, sizeof(c->err), fmt, ap);
    va_end(ap);
  }
  return st;
}

spts_status hip_status(spts_ctx* c, hipError_t e, const char* what) {
  if (e == hipSuccess) return SPTS_OK;
  return fail(c, SPTS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, st, ...)                     \
  do {                                             \
    if (!(cond)) return fail(ctx, st, __VA_ARGS__); \
  } while (0)

#define CHECK_CTX() \
  do {              \
    if (!ctx) return SPTS_ERR_INVALID; \
    ctx->err[0] = 0; \
  } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, SPTS_ERR_INVALID, "%s is NULL", #p)
#define REQUIRE_ALIGN(p) REQUIRE(aligned16(p), SPTS_ERR_ALIGN, "%s is not 16-byte aligned", #p)

// Upper bound on the elements of one K or V operand of the PAP probe (its
// kernels form element offsets in 64 bits; row counts and strides are int).
constexpr long kMaxElems = 1L << 40;
// The GEMM forms the byte offset of a weight (B operand) row in 32 bits, so
// every weight must stay below 4 GiB; activation (A) rows use 64-bit offsets.
constexpr long kMaxWeightBytes = 1L << 32;

}  // namespace

extern "C" {

const char* spts_status_name(spts_status s) {
  switch (s) {
    case SPTS_OK: return "SPTS_OK";
    case SPTS_ERR_INVALID: return "SPTS_ERR_INVALID";
    case SPTS_ERR_SHAPE: return "SPTS_ERR_SHAPE";
    case SPTS_ERR_DTYPE: return "SPTS_ERR_DTYPE";
    case SPTS_ERR_ALIGN: return "SPTS_ERR_ALIGN";
    case SPTS_ERR_NOMEM: return "SPTS_ERR_NOMEM";
    case SPTS_ERR_HIP: return "SPTS_ERR_HIP";
    case SPTS_ERR_UNSUPPORTED: return "SPTS_ERR_UNSUPPORTED";
  }
  return "SPTS_UNKNOWN";
}

spts_status spts_create(spts_ctx** out, void* hip_stream) {
  if (!out) return SPTS_ERR_INVALID;
  spts_ctx* c = new (std::nothrow) spts_ctx;
  if (!c) return SPTS_ERR_NOMEM;
  c->stream = reinterpret_cast<hipStream_t>(hip_stream);
  c->ws = nullptr;
  c->ws_bytes = 0;
  c->err[0] = 0;
  *out = c;
  return SPTS_OK;
}

spts_status spts_destroy(spts_ctx* ctx) {
  if (!ctx) return SPTS_ERR_INVALID;
  delete ctx;
  return SPTS_OK;
}

spts_status spts_set_stream(spts_ctx* ctx, void* hip_stream) {
  CHECK_CTX();
  ctx->stream = reinterpret_cast<hipStream_t>(hip_stream);
  return SPTS_OK;
}

spts_status spts_set_workspace(spts_ctx* ctx, void* dev_ptr, size_t bytes) {
  CHECK_CTX();
  REQUIRE(dev_ptr != nullptr || bytes == 0, SPTS_ERR_INVALID, "workspace pointer is NULL");
  REQUIRE(aligned16(dev_ptr), SPTS_ERR_ALIGN, "workspace is not 16-byte aligned");
  ctx->ws = dev_ptr;
  ctx->ws_bytes = bytes;
  return SPTS_OK;
}

const char* spts_last_error(const spts_ctx* ctx) { return ctx ? ctx->err : "NULL context"; }

spts_status spts_check(spts_ctx* ctx) {
  CHECK_CTX();
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "stream");
  return hip_status(ctx, hipGetLastError(), "pending");
}

// ------------------------------------------------------------ workspace sizes

size_t spts_probe_attention_workspace(int n, int P, int Hq) {
  if (n <= 0 || P <= 0 || Hq <= 0) return 0;
  return probe_workspace(n, P, Hq);
}
size_t spts_score_topk_workspace(int n) { return n > 0 ? topk_workspace(n) : 0; }
static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t spts_ltp_probe_workspace(int n, int d, int r) {
  if (n <= 0 || d <= 0 || r <= 0) return 0;
  const size_t t2 = round256((size_t)n * 2 * r * 2);              // z U as bf16 hi/lo
  const size_t part = round256((size_t)n * (d / 256) * 4);        // row sums of squares
  return t2 + part + gemm_split_workspace(n, d, r, EPI_SPLIT);    // split-K partials of z U
}
// fp32 t in the QUAD lanes' order: rows padded to whole 256-row tiles
static size_t tperm_bytes(int n, int r) { return round256((size_t)((n + 255) / 256) * 256 * r * 4); }
// T3 [n, 3r] = [hi | lo | hi] of z U | t (quad_perm order) | partial quadratic
// forms [n, (r/256) * k-slices] | split-K partials
size_t spts_ltp_gram_workspace(int n, int d, int r) {
  if (n <= 0 || d <= 0 || r <= 0) return 0;
  const size_t t3 = round256((size_t)n * 3 * r * 2);
  const size_t part = round256((size_t)n * (r / 256) * gemm_quad_ksplit(n, 3 * r, r) * 4);
  return t3 + tperm_bytes(n, r) + part + gemm_split_workspace(n, d, r, EPI_SPLIT);
}
// T2 [n, 4r] | H2 [n, 2 d_low] | Td3 [n, 3r] (bf16 hi/lo pairs) | row sums | h C (quad_perm order) | split-K partials
// (Td3 holds h C as [hi | lo | hi]; the direct form reads its first 2r columns.)
static void ltp_structured_layout(int n, int d, int r, int d_low, size_t off[6]) {
  const int parts_direct = d / 256, parts_gram = (r / 256) * gemm_quad_ksplit(n, 3 * r, r);
  off[0] = 0;
  off[1] = off[0] + round256((size_t)n * 4 * r * 2);
  off[2] = off[1] + round256((size_t)n * 2 * d_low * 2);
  off[3] = off[2] + round256((size_t)n * 3 * r * 2);
  off[4] = off[3] + round256((size_t)n * (parts_direct > parts_gram ? parts_direct : parts_gram) * 4);
  off[5] = off[4] + tperm_bytes(n, r);
}
size_t spts_ltp_structured_workspace(int n, int d, int r, int d_low) {
  if (n <= 0 || d <= 0 || r <= 0 || d_low <= 0) return 0;
  size_t off[6];
  ltp_structured_layout(n, d, r, d_low, off);
  const size_t s1 = gemm_split_workspace(n, d, 2 * r, EPI_SPLIT);
  const size_t s3 = gemm_split_workspace(n, 2 * d_low, r, EPI_SPLIT);
  return off[5] + (s1 > s3 ? s1 : s3);
}
size_t spts_linear_workspace(int m, int kdim, int n) {
  if (m <= 0 || kdim <= 0 || n <= 0) return 0;
  return gemm_split_workspace(m, kdim, n, EPI_STORE);
}
size_t spts_linear_kv_workspace(int m, int kdim, int nk, int nv) {
  if (m <= 0 || kdim <= 0 || nk <= 0 || nv <= 0) return 0;
  return gemm_split_workspace(m, kdim, nk + nv, EPI_KV);
}
size_t spts_linear_swiglu_workspace(int m, int kdim, int f) {
  if (m <= 0 || kdim <= 0 || f <= 0) return 0;
  return gemm_split_workspace(m, kdim, 2 * f, EPI_SWIGLU);
}
// H [k, f] bf16, then the split workspace of whichever of the two GEMMs needs more
size_t spts_reduced_ffn_workspace(int k, int d, int f) {
  if (k <= 0 || d <= 0 || f <= 0) return 0;
  const size_t s1 = gemm_split_workspace(k, d, 2 * f, EPI_SWIGLU);
  const size_t s2 = gemm_split_workspace(k, f, d, EPI_STORE);
  return round256((size_t)k * f * 2) + (s1 > s2 ? s1 : s2);
}
size_t spts_msdp_stage_workspace(int n_prev) { return n_prev > 0 ? topk_workspace(n_prev) : 0; }

// ------------------------------------------------------------------------ PAP

spts_status spts_probe_attention(spts_ctx* ctx, spts_dtype dtype, const void* q_probe, const void* k,
                                 int n, int P, int Hq, int Hkv, int dh, float scale, float* scores) {
  CHECK_CTX();
  REQUIRE_PTR(q_probe); REQUIRE_PTR(k); REQUIRE_PTR(scores);
  REQUIRE_ALIGN(q_probe); REQUIRE_ALIGN(k); REQUIRE_ALIGN(scores);
  REQUIRE(n > 0 && P > 0 && P <= n, SPTS_ERR_SHAPE, "need 0 < P <= n (P=%d n=%d)", P, n);
  REQUIRE(Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPTS_ERR_SHAPE, "Hq %% Hkv != 0 (Hq=%d Hkv=%d)", Hq, Hkv);
  REQUIRE((long)n * Hkv * dh < kMaxElems, SPTS_ERR_SHAPE, "too large");
  const size_t need = probe_workspace(n, P, Hq);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  if (dtype == SPTS_BF16) {
    REQUIRE(dh == 128, SPTS_ERR_UNSUPPORTED, "bf16 probe needs dh == 128 (dh=%d)", dh);
    REQUIRE(P == 32 || P == 64 || P == 128, SPTS_ERR_UNSUPPORTED, "bf16 probe needs P in {32,64,128} (P=%d)", P);
    REQUIRE((Hq / Hkv) % 4 == 0, SPTS_ERR_UNSUPPORTED, "bf16 probe needs Hq/Hkv %% 4 == 0");
    return hip_status(ctx, launch_probe_bf16(reinterpret_cast<const uint16_t*>(q_probe),
                                             reinterpret_cast<const uint16_t*>(k), n, P, Hq, Hkv, scale,
                                             scores, ctx->ws, ctx->stream), "probe_attention");
  }
  if (dtype == SPTS_F32) {
    REQUIRE(dh > 0 && dh <= 128, SPTS_ERR_UNSUPPORTED, "fp32 probe needs 0 < dh <= 128");
    return hip_status(ctx, launch_probe_f32(reinterpret_cast<const float*>(q_probe),
                                            reinterpret_cast<const float*>(k), n, P, Hq, Hkv, dh, scale,
                                            scores, ctx->ws, ctx->stream), "probe_attention");
  }
  return fail(ctx, SPTS_ERR_DTYPE, "probe_attention: dtype %d not supported", (int)dtype);
}

// --------------------------------------------------------------------- select

spts_status spts_score_topk(spts_ctx* ctx, const float* s_a, const float* s_b, float w_a, float w_b,
                            int n, int k, int n_forced, int32_t* idx, float* fused_out) {
  CHECK_CTX();
  REQUIRE_PTR(s_a); REQUIRE_PTR(idx);
  REQUIRE_ALIGN(s_a); REQUIRE_ALIGN(idx);
  if (s_b) REQUIRE_ALIGN(s_b);
  if (fused_out) REQUIRE_ALIGN(fused_out);
  REQUIRE(n >= 1, SPTS_ERR_SHAPE, "n must be >= 1");
  REQUIRE(n <= kTopkMaxN, SPTS_ERR_UNSUPPORTED, "top-k over %d scores: at most 2^30", n);
  REQUIRE(n_forced >= 0 && n_forced <= k && n_forced <= n, SPTS_ERR_SHAPE,
          "need 0 <= n_forced <= k and n_forced <= n (n=%d k=%d n_forced=%d)", n, k, n_forced);
  const size_t need = topk_workspace(n);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  return hip_status(ctx, launch_topk(s_a, s_b, w_a, w_b, false, n, k, n_forced, idx, fused_out, ctx->ws,
                                     ctx->stream),
                    "score_topk");
}

spts_status spts_score_topk_noalloc(spts_ctx* ctx, const float* s_a, const float* s_b, float w_a, float w_b,
                                    int n, int k, int n_forced, int32_t* idx, float* fused_out) {
  CHECK_CTX();
  REQUIRE_PTR(s_a); REQUIRE_PTR(idx);
  REQUIRE_ALIGN(s_a); REQUIRE_ALIGN(idx);
  if (s_b) REQUIRE_ALIGN(s_b);
  if (fused_out) REQUIRE_ALIGN(fused_out);
  REQUIRE(n >= 1, SPTS_ERR_SHAPE, "n must be >= 1");
  REQUIRE(n <= kTopkMaxN, SPTS_ERR_UNSUPPORTED, "top-k over %d scores: at most 2^30", n);
  REQUIRE(n <= kTopkNoallocMaxN, SPTS_ERR_UNSUPPORTED,
          "score_topk_noalloc holds at most %d scores in its static scratch (n=%d)", kTopkNoallocMaxN, n);
  REQUIRE(n_forced >= 0 && n_forced <= k && n_forced <= n, SPTS_ERR_SHAPE,
          "need 0 <= n_forced <= k and n_forced <= n (n=%d k=%d n_forced=%d)", n, k, n_forced);
  return hip_status(ctx, launch_topk_noalloc(s_a, s_b, w_a, w_b, false, n, k, n_forced, idx, fused_out, ctx->stream),
                    "score_topk_noalloc");
}

spts_status spts_score_topk_batched(spts_ctx* ctx, const float* s, int64_t s_stride, int batch, int n, int k,
                                    int n_forced, int32_t* idx, int64_t idx_stride) {
  CHECK_CTX();
  REQUIRE(batch >= 0, SPTS_ERR_SHAPE, "batch must be >= 0");
  REQUIRE(n >= 1, SPTS_ERR_SHAPE, "n must be >= 1");
  REQUIRE(n <= 32768, SPTS_ERR_UNSUPPORTED, "batched top-k holds a row in registers: n <= 32768 (got %d)", n);
  REQUIRE(n_forced >= 0 && n_forced <= k && n_forced <= n, SPTS_ERR_SHAPE,
          "need 0 <= n_forced <= k and n_forced <= n (n=%d k=%d n_forced=%d)", n, k, n_forced);
  REQUIRE(s_stride >= n && idx_stride >= (k < n ? k : n), SPTS_ERR_SHAPE, "row strides shorter than the rows");
  if (batch == 0) return SPTS_OK;
  REQUIRE_PTR(s); REQUIRE_PTR(idx);
  REQUIRE_ALIGN(s); REQUIRE_ALIGN(idx);
  return hip_status(ctx, launch_topk_batched(s, (long)s_stride, batch, n, k, n_forced, idx, (long)idx_stride,
                                             ctx->stream),
                    "score_topk_batched");
}

spts_status spts_score_topk_multiply(spts_ctx* ctx, const float* s_a, const float* s_b, int n, int k,
                                     int n_forced, int32_t* idx, float* fused_out) {
  CHECK_CTX();
  REQUIRE_PTR(s_a); REQUIRE_PTR(s_b); REQUIRE_PTR(idx);
  REQUIRE_ALIGN(s_a); REQUIRE_ALIGN(s_b); REQUIRE_ALIGN(idx);
  if (fused_out) REQUIRE_ALIGN(fused_out);
  REQUIRE(n >= 1, SPTS_ERR_SHAPE, "n must be >= 1");
  REQUIRE(n <= kTopkMaxN, SPTS_ERR_UNSUPPORTED, "top-k over %d scores: at most 2^30", n);
  REQUIRE(n_forced >= 0 && n_forced <= k && n_forced <= n, SPTS_ERR_SHAPE,
          "need 0 <= n_forced <= k and n_forced <= n (n=%d k=%d n_forced=%d)", n, k, n_forced);
  const size_t need = topk_workspace(n);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  return hip_status(ctx, launch_topk(s_a, s_b, 0.f, 0.f, true, n, k, n_forced, idx, fused_out, ctx->ws,
                                     ctx->stream),
                    "score_topk_multiply");
}

// ------------------------------------------------------------- gather/scatter

static int dtype_bytes(spts_dtype t) {
  switch (t) {
    case SPTS_BF16: return 2;
    case SPTS_F32: return 4;
    case SPTS_I32: return 4;
  }
  return 0;
}

spts_status spts_gather(spts_ctx* ctx, spts_dtype dtype, const void* src, const int32_t* idx, int k,
                        int row_elems, void* dst) {
  CHECK_CTX();
  const int eb = dtype_bytes(dtype);
  REQUIRE(eb > 0, SPTS_ERR_DTYPE, "gather: bad dtype %d", (int)dtype);
  REQUIRE(k >= 0 && row_elems > 0, SPTS_ERR_SHAPE, "gather: need k >= 0, row_elems > 0");
  if (k == 0) return SPTS_OK;
  REQUIRE_PTR(src); REQUIRE_PTR(idx); REQUIRE_PTR(dst);
  REQUIRE_ALIGN(src); REQUIRE_ALIGN(idx); REQUIRE_ALIGN(dst);
  return hip_status(ctx, launch_gather(src, idx, k, (long)row_elems * eb, dst, ctx->stream), "gather");
}

spts_status spts_scatter(spts_ctx* ctx, spts_dtype dtype, const void* src, const int32_t* idx, int k,
                         int row_elems, void* dst, int accumulate) {
  CHECK_CTX();
  const int eb = dtype_bytes(dtype);
  REQUIRE(eb > 0, SPTS_ERR_DTYPE, "scatter: bad dtype %d", (int)dtype);
  REQUIRE(k >= 0 && row_elems > 0, SPTS_ERR_SHAPE, "scatter: need k >= 0, row_elems > 0");
  REQUIRE(accumulate == 0 || accumulate == 1, SPTS_ERR_INVALID, "accumulate must be 0 or 1");
  if (k == 0) return SPTS_OK;
  REQUIRE_PTR(src); REQUIRE_PTR(idx); REQUIRE_PTR(dst);
  REQUIRE_ALIGN(src); REQUIRE_ALIGN(idx); REQUIRE_ALIGN(dst);
  hipError_t e;
  if (!accumulate) e = launch_scatter(src, idx, k, (long)row_elems * eb, dst, ctx->stream);
  else if (dtype == SPTS_BF16)
    e = launch_scatter_add_bf16(reinterpret_cast<const uint16_t*>(src), idx, k, row_elems,
                                reinterpret_cast<uint16_t*>(dst), ctx->stream);
  else if (dtype == SPTS_F32)
    e = launch_scatter_add_f32(reinterpret_cast<const float*>(src), idx, k, row_elems,
                               reinterpret_cast<float*>(dst), ctx->stream);
  else
    e = launch_scatter_add_i32(reinterpret_cast<const int32_t*>(src), idx, k, row_elems,
                               reinterpret_cast<int32_t*>(dst), ctx->stream);
  return hip_status(ctx, e, "scatter");
}

// ----------------------------------------------------------- reduced attention

spts_status spts_reduced_attention(spts_ctx* ctx, spts_dtype dtype, const void* q_sel, const int32_t* idx,
                                   const void* k, const void* v, int kq, int n, int Hq, int Hkv, int dh,
                                   float scale, void* o_sel) {
  CHECK_CTX();
  REQUIRE(kq >= 0 && n > 0 && kq <= n, SPTS_ERR_SHAPE, "need 0 <= kq <= n (kq=%d n=%d)", kq, n);
  REQUIRE(Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPTS_ERR_SHAPE, "Hq %% Hkv != 0");
  if (kq == 0) return SPTS_OK;
  REQUIRE_PTR(q_sel); REQUIRE_PTR(idx); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(o_sel);
  REQUIRE_ALIGN(q_sel); REQUIRE_ALIGN(idx); REQUIRE_ALIGN(k); REQUIRE_ALIGN(v); REQUIRE_ALIGN(o_sel);
  if (dtype == SPTS_BF16) {
    REQUIRE(dh == 128, SPTS_ERR_UNSUPPORTED, "bf16 attention needs dh == 128");
    REQUIRE((long)n * Hkv * dh < (1L << 31), SPTS_ERR_UNSUPPORTED, "K/V larger than 2^31 elements");
    REQUIRE((Hq / Hkv) % 4 == 0, SPTS_ERR_UNSUPPORTED, "bf16 attention needs Hq/Hkv %% 4 == 0");
    return hip_status(ctx, launch_attn_bf16(reinterpret_cast<const uint16_t*>(q_sel), idx,
                                            reinterpret_cast<const uint16_t*>(k),
                                            reinterpret_cast<const uint16_t*>(v), kq, n, Hq, Hkv, scale,
                                            reinterpret_cast<uint16_t*>(o_sel), ctx->stream),
                      "reduced_attention");
  }
  if (dtype == SPTS_F32) {
    REQUIRE(dh > 0 && dh <= 128, SPTS_ERR_UNSUPPORTED, "fp32 attention needs 0 < dh <= 128");
    return hip_status(ctx, launch_attn_f32(reinterpret_cast<const float*>(q_sel), idx,
                                           reinterpret_cast<const float*>(k), reinterpret_cast<const float*>(v),
                                           kq, n, Hq, Hkv, dh, scale, reinterpret_cast<float*>(o_sel),
                                           ctx->stream),
                      "reduced_attention");
  }
  return fail(ctx, SPTS_ERR_DTYPE, "reduced_attention: dtype %d not supported", (int)dtype);
}

// ------------------------------------------------------------------------ GEMM

static spts_status weight_size_ok(spts_ctx* ctx, long rows, long cols) {
  REQUIRE(rows * cols * 2 < kMaxWeightBytes, SPTS_ERR_UNSUPPORTED,
          "weight of %ld x %ld bf16 elements is 4 GiB or more", rows, cols);
  return SPTS_OK;
}

static spts_status gemm_shape_ok(spts_ctx* ctx, int m, int kdim, int n) {
  REQUIRE(m >= 0 && kdim > 0 && n > 0, SPTS_ERR_SHAPE, "bad GEMM sizes m=%d k=%d n=%d", m, kdim, n);
  REQUIRE(kdim % 64 == 0, SPTS_ERR_UNSUPPORTED, "inner dimension %d is not a multiple of 64", kdim);
  REQUIRE(n % 256 == 0, SPTS_ERR_UNSUPPORTED, "output width %d is not a multiple of 256", n);
  return weight_size_ok(ctx, n, kdim);
}

spts_status spts_linear(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m, int kdim, const void* w,
                        int n, void* out, const int32_t* out_rows, int accumulate) {
  CHECK_CTX();
  spts_status st = gemm_shape_ok(ctx, m, kdim, n);
  if (st != SPTS_OK) return st;
  REQUIRE(accumulate == 0 || accumulate == 1, SPTS_ERR_INVALID, "accumulate must be 0 or 1");
  if (m == 0) return SPTS_OK;
  REQUIRE_PTR(a); REQUIRE_PTR(w); REQUIRE_PTR(out);
  REQUIRE_ALIGN(a); REQUIRE_ALIGN(w); REQUIRE_ALIGN(out);
  if (a_rows) REQUIRE_ALIGN(a_rows);
  if (out_rows) REQUIRE_ALIGN(out_rows);
  GemmArgs g{};
  g.a = reinterpret_cast<const uint16_t*>(a); g.a_rows = a_rows; g.m = m; g.k = kdim; g.lda = kdim;
  g.b0 = reinterpret_cast<const uint16_t*>(w); g.ldb = kdim; g.n = n;
  g.out = out; g.ldc = n; g.out_rows = out_rows; g.accumulate = accumulate;
  g.partial = reinterpret_cast<float*>(ctx->ws); g.partial_bytes = ctx->ws_bytes;
  return hip_status(ctx, launch_gemm(g, EPI_STORE, ctx->stream), "linear");
}

spts_status spts_linear_rope(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m, int kdim,
                             const void* w, int n, void* out, const int32_t* pos, const float* table) {
  CHECK_CTX();
  spts_status st = gemm_shape_ok(ctx, m, kdim, n);
  if (st != SPTS_OK) return st;
  if (m == 0) return SPTS_OK;
  REQUIRE_PTR(a); REQUIRE_PTR(w); REQUIRE_PTR(out); REQUIRE_PTR(pos); REQUIRE_PTR(table);
  REQUIRE_ALIGN(a); REQUIRE_ALIGN(w); REQUIRE_ALIGN(out); REQUIRE_ALIGN(table);
  GemmArgs g{};
  g.a = reinterpret_cast<const uint16_t*>(a); g.a_rows = a_rows; g.m = m; g.k = kdim; g.lda = kdim;
  g.b0 = reinterpret_cast<const uint16_t*>(w); g.ldb = kdim; g.n = n;
  g.out = out; g.ldc = n; g.pos = pos; g.rope_table = table;
  g.partial = reinterpret_cast<float*>(ctx->ws); g.partial_bytes = ctx->ws_bytes;
  return hip_status(ctx, launch_gemm(g, EPI_ROPE, ctx->stream), "linear_rope");
}

spts_status spts_linear_kv(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m, int kdim,
                           const void* wk, int nk, const void* wv, int nv, void* k_out, void* v_out,
                           const int32_t* pos, const float* table) {
  CHECK_CTX();
  REQUIRE(nk > 0 && nv > 0, SPTS_ERR_SHAPE, "bad K/V widths nk=%d nv=%d", nk, nv);
  spts_status st = gemm_shape_ok(ctx, m, kdim, nk);
  if (st != SPTS_OK) return st;
  st = gemm_shape_ok(ctx, m, kdim, nv);
  if (st != SPTS_OK) return st;
  REQUIRE((pos == nullptr) == (table == nullptr), SPTS_ERR_INVALID, "pos and table go together");
  if (m == 0) return SPTS_OK;
  REQUIRE_PTR(a); REQUIRE_PTR(wk); REQUIRE_PTR(wv); REQUIRE_PTR(k_out); REQUIRE_PTR(v_out);
  REQUIRE_ALIGN(a); REQUIRE_ALIGN(wk); REQUIRE_ALIGN(wv); REQUIRE_ALIGN(k_out); REQUIRE_ALIGN(v_out);
  if (a_rows) REQUIRE_ALIGN(a_rows);
  if (table) REQUIRE_ALIGN(table);
  GemmArgs g{};
  g.a = reinterpret_cast<const uint16_t*>(a); g.a_rows = a_rows; g.m = m; g.k = kdim; g.lda = kdim;
  g.b0 = reinterpret_cast<const uint16_t*>(wk); g.b1 = reinterpret_cast<const uint16_t*>(wv);
  g.ldb = kdim; g.n = nk + nv; g.n0 = nk;
  g.out = k_out; g.ldc = nk; g.out2 = v_out; g.ldc2 = nv;
  g.pos = pos; g.rope_table = table;
  g.partial = reinterpret_cast<float*>(ctx->ws); g.partial_bytes = ctx->ws_bytes;
  return hip_status(ctx, launch_gemm(g, EPI_KV, ctx->stream), "linear_kv");
}

spts_status spts_linear_swiglu(spts_ctx* ctx, const void* a, const int32_t* a_rows, int m, int kdim,
                               const void* w_gate, const void* w_up, int f, void* h_out) {
  CHECK_CTX();
  REQUIRE(m >= 0 && kdim > 0 && f > 0, SPTS_ERR_SHAPE, "bad SwiGLU GEMM sizes");
  REQUIRE(kdim % 64 == 0 && f % 128 == 0, SPTS_ERR_UNSUPPORTED, "SwiGLU GEMM needs kdim %% 64 == 0, f %% 128 == 0");
  {
    const spts_status st = weight_size_ok(ctx, f, kdim);
    if (st != SPTS_OK) return st;
  }
  if (m == 0) return SPTS_OK;
  REQUIRE_PTR(a); REQUIRE_PTR(w_gate); REQUIRE_PTR(w_up); REQUIRE_PTR(h_out);
  REQUIRE_ALIGN(a); REQUIRE_ALIGN(w_gate); REQUIRE_ALIGN(w_up); REQUIRE_ALIGN(h_out);
  if (a_rows) REQUIRE_ALIGN(a_rows);
  GemmArgs g{};
  g.a = reinterpret_cast<const uint16_t*>(a); g.a_rows = a_rows; g.m = m; g.k = kdim; g.lda = kdim;
  g.b0 = reinterpret_cast<const uint16_t*>(w_gate); g.b1 = reinterpret_cast<const uint16_t*>(w_up);
  g.ldb = kdim; g.n = 2 * f; g.out = h_out; g.ldc = f;
  g.partial = reinterpret_cast<float*>(ctx->ws); g.partial_bytes = ctx->ws_bytes;
  return hip_status(ctx, launch_gemm(g, EPI_SWIGLU, ctx->stream), "linear_swiglu");
}

spts_status spts_rope_table(spts_ctx* ctx, int max_pos, int dh, double theta, float* table) {
  CHECK_CTX();
  REQUIRE_PTR(table);
  REQUIRE(max_pos > 0 && dh > 0 && dh % 2 == 0 && theta > 0, SPTS_ERR_SHAPE, "bad rope table shape");
  return hip_status(ctx, launch_rope_table(max_pos, dh, theta, table, ctx->stream), "rope_table");
}

spts_status spts_rmsnorm(spts_ctx* ctx, const void* x, int n, int d, float eps, void* out) {
  CHECK_CTX();
  REQUIRE(n >= 0 && d > 0 && d % 8 == 0, SPTS_ERR_SHAPE, "rmsnorm needs d %% 8 == 0");
  if (n == 0) return SPTS_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(out);
  REQUIRE_ALIGN(x); REQUIRE_ALIGN(out);
  return hip_status(ctx, launch_rmsnorm(reinterpret_cast<const uint16_t*>(x), n, d, eps,
                                        reinterpret_cast<uint16_t*>(out), ctx->stream), "rmsnorm");
}

// ------------------------------------------------------------------------ LTP

spts_status spts_ltp_probe(spts_ctx* ctx, const void* z, const void* u_t, const void* v_t, int n, int d,
                           int r, float* score) {
  CHECK_CTX();
  REQUIRE(n >= 0 && d > 0 && r > 0, SPTS_ERR_SHAPE, "bad LTP sizes");
  REQUIRE(d % 256 == 0 && r % 256 == 0, SPTS_ERR_UNSUPPORTED, "LTP needs d %% 256 == 0 and r %% 256 == 0");
  {
    const spts_status st = weight_size_ok(ctx, d, r);
    if (st != SPTS_OK) return st;
  }
  if (n == 0) return SPTS_OK;
  REQUIRE_PTR(z); REQUIRE_PTR(u_t); REQUIRE_PTR(v_t); REQUIRE_PTR(score);
  REQUIRE_ALIGN(z); REQUIRE_ALIGN(u_t); REQUIRE_ALIGN(v_t); REQUIRE_ALIGN(score);
  const size_t need = spts_ltp_probe_workspace(n, d, r);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  uint16_t* t2 = reinterpret_cast<uint16_t*>(ctx->ws);
  const size_t t2_bytes = round256((size_t)n * 2 * r * 2);
  const size_t part_bytes = round256((size_t)n * (d / 256) * 4);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ctx->ws) + t2_bytes);
  float* split_ws = reinterpret_cast<float*>(reinterpret_cast<char*>(ctx->ws) + t2_bytes + part_bytes);
  // T = z U, stored as bf16 hi + lo halves [n, 2r]
  GemmArgs g1{};
  g1.a = reinterpret_cast<const uint16_t*>(z); g1.m = n; g1.k = d; g1.lda = d;
  g1.b0 = reinterpret_cast<const uint16_t*>(u_t); g1.ldb = d; g1.n = r;
  g1.out = t2; g1.ldc = 2 * r;
  g1.partial = split_ws; g1.partial_bytes = ctx->ws_bytes - t2_bytes - part_bytes;
  hipError_t e = launch_gemm(g1, EPI_SPLIT, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "ltp_probe (z U)");
  // (T_hi + T_lo) V: inner dimension 2r with V's columns read modulo r
  GemmArgs g2{};
  g2.a = t2; g2.m = n; g2.k = 2 * r; g2.lda = 2 * r;
  g2.b0 = reinterpret_cast<const uint16_t*>(v_t); g2.ldb = r; g2.kwrap = r; g2.n = d;
  g2.out = part; g2.ldc = d / 256;
  e = launch_gemm(g2, EPI_SUMSQ, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "ltp_probe (T V)");
  return hip_status(ctx, launch_rowsum_sqrt(part, n, d / 256, score, ctx->stream), "ltp_probe (norm)");
}

spts_status spts_ltp_gram(spts_ctx* ctx, const void* v_t, int d, int r, void* gram) {
  CHECK_CTX();
  REQUIRE(d > 0 && r > 0, SPTS_ERR_SHAPE, "bad LTP Gram sizes");
  REQUIRE(r % 256 == 0, SPTS_ERR_UNSUPPORTED, "LTP Gram needs r %% 256 == 0");
  {
    const spts_status st = weight_size_ok(ctx, d, r);
    if (st != SPTS_OK) return st;
  }
  REQUIRE_PTR(v_t); REQUIRE_PTR(gram);
  REQUIRE_ALIGN(v_t); REQUIRE_ALIGN(gram);
  return hip_status(ctx, launch_ltp_gram(reinterpret_cast<const uint16_t*>(v_t), d, r,
                                         reinterpret_cast<uint16_t*>(gram), ctx->stream), "ltp_gram");
}

spts_status spts_ltp_probe_gram(spts_ctx* ctx, const void* z, const void* u_t, const void* gram, int n, int d,
                                int r, float* score) {
  CHECK_CTX();
  REQUIRE(n >= 0 && d > 0 && r > 0, SPTS_ERR_SHAPE, "bad LTP sizes");
  REQUIRE(d % 256 == 0 && r % 256 == 0, SPTS_ERR_UNSUPPORTED, "LTP needs d %% 256 == 0 and r %% 256 == 0");
  {
    spts_status st = weight_size_ok(ctx, r, d);
    if (st == SPTS_OK) st = weight_size_ok(ctx, r, 3L * r);
    if (st != SPTS_OK) return st;
  }
  if (n == 0) return SPTS_OK;
  REQUIRE_PTR(z); REQUIRE_PTR(u_t); REQUIRE_PTR(gram); REQUIRE_PTR(score);
  REQUIRE_ALIGN(z); REQUIRE_ALIGN(u_t); REQUIRE_ALIGN(gram); REQUIRE_ALIGN(score);
  const size_t need = spts_ltp_gram_workspace(n, d, r);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  const int ks = gemm_quad_ksplit(n, 3 * r, r);
  char* ws = reinterpret_cast<char*>(ctx->ws);
  uint16_t* t3 = reinterpret_cast<uint16_t*>(ws);
  const size_t t3_bytes = round256((size_t)n * 3 * r * 2);
  float* tperm = reinterpret_cast<float*>(ws + t3_bytes);
  const size_t tp_bytes = tperm_bytes(n, r);
  const size_t part_bytes = round256((size_t)n * (r / 256) * ks * 4);
  float* part = reinterpret_cast<float*>(ws + t3_bytes + tp_bytes);
  const size_t pre = t3_bytes + tp_bytes + part_bytes;
  float* split_ws = reinterpret_cast<float*>(ws + pre);
  // T = z U as bf16 [hi | lo | hi] [n, 3r]
  GemmArgs g1{};
  g1.a = reinterpret_cast<const uint16_t*>(z); g1.m = n; g1.k = d; g1.lda = d;
  g1.b0 = reinterpret_cast<const uint16_t*>(u_t); g1.ldb = d; g1.n = r;
  g1.out = t3; g1.ldc = 3 * r; g1.split3 = 1; g1.tperm = tperm;
  g1.partial = split_ws; g1.partial_bytes = ctx->ws_bytes - pre;
  hipError_t e = launch_gemm(g1, EPI_SPLIT, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "ltp_probe_gram (z U)");
  // Y = [hi|lo|hi](T) [hi|hi|lo](G)^T = T G less lo(T) lo(G); each k-slice
  // adds its part of sum_c Y[m, c] T[m, c] per row
  GemmArgs g2{};
  g2.a = t3; g2.m = n; g2.k = 3 * r; g2.lda = 3 * r;
  g2.b0 = reinterpret_cast<const uint16_t*>(gram); g2.ldb = 3 * r; g2.n = r;
  g2.out = part; g2.tperm = tperm;
  e = launch_gemm(g2, EPI_QUAD, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "ltp_probe_gram (T G T^T)");
  return hip_status(ctx, launch_rowsum_sqrt(part, n, (r / 256) * ks, score, ctx->stream), "ltp_probe_gram (norm)");
}

// The structured proxy's score; the last factor D enters either directly
// (last = d_t, the norm of (h C) D from row sums of squares) or through its
// Gram operand (last = [hi | hi | lo](D D^T), the quadratic form of h C).
static spts_status ltp_structured(spts_ctx* ctx, const void* z, const void* a_gu_t, const void* b_gate,
                                  const void* b_up, const void* c_t, const void* last, bool gram, int n, int d,
                                  int r, int d_low, float* score, const char* name) {
  CHECK_CTX();
  REQUIRE(n >= 0 && d > 0 && r > 0 && d_low > 0, SPTS_ERR_SHAPE, "bad structured LTP sizes");
  REQUIRE(d % 256 == 0 && r % 256 == 0 && d_low % 256 == 0, SPTS_ERR_UNSUPPORTED,
          "structured LTP needs d, r and d_low multiples of 256 (d=%d r=%d d_low=%d)", d, r, d_low);
  {
    spts_status st = weight_size_ok(ctx, 2L * r, d);
    if (st == SPTS_OK) st = weight_size_ok(ctx, d_low, 4L * r);
    if (st == SPTS_OK) st = gram ? weight_size_ok(ctx, r, 3L * r) : weight_size_ok(ctx, d, r);
    if (st == SPTS_OK) st = weight_size_ok(ctx, r, d_low);
    if (st != SPTS_OK) return st;
  }
  if (n == 0) return SPTS_OK;
  REQUIRE_PTR(z); REQUIRE_PTR(a_gu_t); REQUIRE_PTR(b_gate); REQUIRE_PTR(b_up); REQUIRE_PTR(c_t);
  REQUIRE_PTR(last); REQUIRE_PTR(score);
  REQUIRE_ALIGN(z); REQUIRE_ALIGN(a_gu_t); REQUIRE_ALIGN(b_gate); REQUIRE_ALIGN(b_up); REQUIRE_ALIGN(c_t);
  REQUIRE_ALIGN(last); REQUIRE_ALIGN(score);
  const size_t need = spts_ltp_structured_workspace(n, d, r, d_low);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  size_t off[6];
  ltp_structured_layout(n, d, r, d_low, off);
  char* ws = reinterpret_cast<char*>(ctx->ws);
  uint16_t* t2 = reinterpret_cast<uint16_t*>(ws + off[0]);
  uint16_t* h2 = reinterpret_cast<uint16_t*>(ws + off[1]);
  uint16_t* td3 = reinterpret_cast<uint16_t*>(ws + off[2]);
  float* part = reinterpret_cast<float*>(ws + off[3]);
  float* tperm = reinterpret_cast<float*>(ws + off[4]);
  float* split_ws = reinterpret_cast<float*>(ws + off[5]);
  const size_t split_bytes = ctx->ws_bytes - off[5];
  // [z A_g | z A_u] as hi/lo pairs: T2 row = [Tg_hi | Tu_hi | Tg_lo | Tu_lo]
  GemmArgs g1{};
  g1.a = reinterpret_cast<const uint16_t*>(z); g1.m = n; g1.k = d; g1.lda = d;
  g1.b0 = reinterpret_cast<const uint16_t*>(a_gu_t); g1.ldb = d; g1.n = 2 * r;
  g1.out = t2; g1.ldc = 4 * r;
  g1.partial = split_ws; g1.partial_bytes = split_bytes;
  hipError_t e = launch_gemm(g1, EPI_SPLIT, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, name);
  // h = silu(T_g B_g) * (T_u B_u) over the hi/lo pairs (the packed B blocks pick
  // the gate or up columns of T2), written as hi/lo pairs
  GemmArgs g2{};
  g2.a = t2; g2.m = n; g2.k = 4 * r; g2.lda = 4 * r;
  g2.b0 = reinterpret_cast<const uint16_t*>(b_gate); g2.b1 = reinterpret_cast<const uint16_t*>(b_up);
  g2.ldb = 4 * r; g2.n = 2 * d_low; g2.out = h2; g2.ldc = 2 * d_low;
  e = launch_gemm(g2, EPI_SWIGLU_SPLIT, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, name);
  // h C over the hi/lo pairs (C's columns read modulo d_low), as [hi | lo | hi]
  GemmArgs g3{};
  g3.a = h2; g3.m = n; g3.k = 2 * d_low; g3.lda = 2 * d_low;
  g3.b0 = reinterpret_cast<const uint16_t*>(c_t); g3.ldb = d_low; g3.kwrap = d_low; g3.n = r;
  g3.out = td3; g3.ldc = 3 * r; g3.split3 = 1; g3.tperm = gram ? tperm : nullptr;
  g3.partial = split_ws; g3.partial_bytes = split_bytes;
  e = launch_gemm(g3, EPI_SPLIT, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, name);
  GemmArgs g4{};
  g4.a = td3; g4.m = n; g4.lda = 3 * r; g4.out = part;
  int parts;
  if (gram) {
    // (h C) G (h C)^T, G = D D^T: each k-slice adds its part per row
    g4.k = 3 * r; g4.b0 = reinterpret_cast<const uint16_t*>(last); g4.ldb = 3 * r; g4.n = r; g4.tperm = tperm;
    e = launch_gemm(g4, EPI_QUAD, ctx->stream);
    parts = (r / 256) * gemm_quad_ksplit(n, 3 * r, r);
  } else {
    // ||(h C) D||: row sums of squares per 256 columns
    g4.k = 2 * r; g4.b0 = reinterpret_cast<const uint16_t*>(last); g4.ldb = r; g4.kwrap = r; g4.n = d;
    e = launch_gemm(g4, EPI_SUMSQ, ctx->stream);
    parts = d / 256;
  }
  if (e != hipSuccess) return hip_status(ctx, e, name);
  return hip_status(ctx, launch_rowsum_sqrt(part, n, parts, score, ctx->stream), name);
}

spts_status spts_ltp_probe_structured(spts_ctx* ctx, const void* z, const void* a_gu_t, const void* b_gate,
                                      const void* b_up, const void* c_t, const void* d_t, int n, int d, int r,
                                      int d_low, float* score) {
  return ltp_structured(ctx, z, a_gu_t, b_gate, b_up, c_t, d_t, false, n, d, r, d_low, score,
                        "ltp_probe_structured");
}

spts_status spts_ltp_probe_structured_gram(spts_ctx* ctx, const void* z, const void* a_gu_t, const void* b_gate,
                                           const void* b_up, const void* c_t, const void* gram, int n, int d,
                                           int r, int d_low, float* score) {
  return ltp_structured(ctx, z, a_gu_t, b_gate, b_up, c_t, gram, true, n, d, r, d_low, score,
                        "ltp_probe_structured_gram");
}

// --------------------------------------------------------------------- decode

size_t spts_decode_attention_workspace(int L, int Hq) {
  return (L > 0 && Hq > 0) ? round256(decode_attn_workspace(L, Hq)) : 0;
}

static spts_status gemv_shape_ok(spts_ctx* ctx, int kdim, int n) {
  REQUIRE(kdim > 0 && n > 0, SPTS_ERR_SHAPE, "bad decode projection sizes kdim=%d n=%d", kdim, n);
  REQUIRE(gemv_supported_k(kdim), SPTS_ERR_UNSUPPORTED, "decode projections need kdim %% 512 == 0, <= 16384 (got %d)",
          kdim);
  return SPTS_OK;
}

spts_status spts_decode_linear(spts_ctx* ctx, const void* x, const void* w, int kdim, int n, void* out,
                               int accumulate) {
  CHECK_CTX();
  spts_status st = gemv_shape_ok(ctx, kdim, n);
  if (st != SPTS_OK) return st;
  REQUIRE(accumulate == 0 || accumulate == 1, SPTS_ERR_INVALID, "accumulate must be 0 or 1");
  REQUIRE_PTR(x); REQUIRE_PTR(w); REQUIRE_PTR(out);
  REQUIRE_ALIGN(x); REQUIRE_ALIGN(w);
  return hip_status(ctx, launch_gemv(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                                     nullptr, kdim, n, reinterpret_cast<uint16_t*>(out), accumulate ? 3 : 0, 0,
                                     nullptr, ctx->stream),
                    "decode_linear");
}

spts_status spts_decode_linear_rope(spts_ctx* ctx, const void* x, const void* w, int kdim, int n, void* out,
                                    int pos, const float* table) {
  CHECK_CTX();
  spts_status st = gemv_shape_ok(ctx, kdim, n);
  if (st != SPTS_OK) return st;
  REQUIRE(n % 128 == 0, SPTS_ERR_UNSUPPORTED, "decode RoPE needs 128-wide heads (n=%d)", n);
  REQUIRE(pos >= 0, SPTS_ERR_SHAPE, "pos must be >= 0");
  REQUIRE_PTR(x); REQUIRE_PTR(w); REQUIRE_PTR(out); REQUIRE_PTR(table);
  REQUIRE_ALIGN(x); REQUIRE_ALIGN(w); REQUIRE_ALIGN(table);
  return hip_status(ctx, launch_gemv(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                                     nullptr, kdim, n, reinterpret_cast<uint16_t*>(out), 1, pos, table, ctx->stream),
                    "decode_linear_rope");
}

spts_status spts_decode_swiglu(spts_ctx* ctx, const void* x, const void* w_gate, const void* w_up, int kdim, int f,
                               void* h_out) {
  CHECK_CTX();
  spts_status st = gemv_shape_ok(ctx, kdim, f);
  if (st != SPTS_OK) return st;
  REQUIRE_PTR(x); REQUIRE_PTR(w_gate); REQUIRE_PTR(w_up); REQUIRE_PTR(h_out);
  REQUIRE_ALIGN(x); REQUIRE_ALIGN(w_gate); REQUIRE_ALIGN(w_up);
  return hip_status(ctx, launch_gemv(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w_gate),
                                     reinterpret_cast<const uint16_t*>(w_up), kdim, f,
                                     reinterpret_cast<uint16_t*>(h_out), 2, 0, nullptr, ctx->stream),
                    "decode_swiglu");
}

spts_status spts_decode_attention(spts_ctx* ctx, const void* q, const void* k_cache, const void* v_cache, int L,
                                  int Hq, int Hkv, int dh, float scale, void* o) {
  CHECK_CTX();
  REQUIRE(L > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPTS_ERR_SHAPE, "bad decode attention sizes");
  REQUIRE(dh == 128 && Hq / Hkv == 4, SPTS_ERR_UNSUPPORTED, "decode attention needs dh == 128 and Hq/Hkv == 4");
  REQUIRE((long)L * Hkv * dh < (1L << 40), SPTS_ERR_UNSUPPORTED, "cache too large");
  REQUIRE_PTR(q); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache); REQUIRE_PTR(o);
  REQUIRE_ALIGN(q); REQUIRE_ALIGN(k_cache); REQUIRE_ALIGN(v_cache);
  const size_t need = spts_decode_attention_workspace(L, Hq);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  return hip_status(ctx, launch_decode_attn(reinterpret_cast<const uint16_t*>(q),
                                            reinterpret_cast<const uint16_t*>(k_cache),
                                            reinterpret_cast<const uint16_t*>(v_cache), L, Hq, Hkv, scale,
                                            reinterpret_cast<uint16_t*>(o), ctx->ws, ctx->stream),
                    "decode_attention");
}

size_t spts_decode_step_workspace(int max_len, int Hq, int f) {
  return (max_len > 0 && Hq > 0 && f > 0) ? round256(decode_layer_workspace(max_len, Hq, f)) : 0;
}

spts_status spts_decode_step(spts_ctx* ctx, void* x, int d, int pos, const spts_decode_layer* layers, int n_layers,
                             int* lengths, int Hq, int Hkv, int dh, int f, float eps, int prenorm,
                             const float* rope_table, int table_rows, float scale) {
  CHECK_CTX();
  REQUIRE(n_layers >= 0 && d > 0 && f > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPTS_ERR_SHAPE,
          "bad decode step sizes");
  REQUIRE(dh == 128 && Hq / Hkv == 4, SPTS_ERR_UNSUPPORTED, "decode step needs dh == 128 and Hq/Hkv == 4");
  REQUIRE(gemv_supported_k(d) && gemv_supported_k(f) && gemv_supported_k(Hq * dh), SPTS_ERR_UNSUPPORTED,
          "decode step needs d, f and Hq*dh multiples of 512, at most 16384 (d=%d f=%d)", d, f);
  REQUIRE(prenorm == 0 || prenorm == 1, SPTS_ERR_INVALID, "prenorm must be 0 or 1");
  REQUIRE(pos >= 0, SPTS_ERR_SHAPE, "pos must be >= 0");
  REQUIRE(rope_table == nullptr || pos < table_rows, SPTS_ERR_SHAPE, "RoPE table has %d rows, pos %d", table_rows,
          pos);
  REQUIRE_PTR(x);
  REQUIRE_ALIGN(x);
  if (n_layers == 0) return SPTS_OK;
  REQUIRE_PTR(layers);
  REQUIRE_PTR(lengths);
  int max_len = 0;
  for (int l = 0; l < n_layers; ++l) {
    const spts_decode_layer& Ly = layers[l];
    REQUIRE(Ly.wq && Ly.wk && Ly.wv && Ly.wo && Ly.w_gate && Ly.w_up && Ly.w_down && Ly.k_cache && Ly.v_cache,
            SPTS_ERR_INVALID, "layer %d: NULL weight or cache pointer", l);
    REQUIRE(aligned16(Ly.wq) && aligned16(Ly.wk) && aligned16(Ly.wv) && aligned16(Ly.wo) && aligned16(Ly.w_gate) &&
                aligned16(Ly.w_up) && aligned16(Ly.w_down) && aligned16(Ly.k_cache) && aligned16(Ly.v_cache),
            SPTS_ERR_ALIGN, "layer %d: weight or cache pointer not 16-byte aligned", l);
    REQUIRE(lengths[l] >= 0 && lengths[l] < Ly.cap, SPTS_ERR_SHAPE, "layer %d: cache holds %d of %d rows", l,
            lengths[l], Ly.cap);
    REQUIRE((long)Ly.cap * Hkv * dh < (1L << 40), SPTS_ERR_UNSUPPORTED, "layer %d: cache too large", l);
    max_len = lengths[l] + 1 > max_len ? lengths[l] + 1 : max_len;
  }
  const size_t need = spts_decode_step_workspace(max_len, Hq, f);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  for (int l = 0; l < n_layers; ++l) {
    const spts_decode_layer& Ly = layers[l];
    DecodeLayerPtrs w{reinterpret_cast<const uint16_t*>(Ly.wq), reinterpret_cast<const uint16_t*>(Ly.wk),
                      reinterpret_cast<const uint16_t*>(Ly.wv), reinterpret_cast<const uint16_t*>(Ly.wo),
                      reinterpret_cast<const uint16_t*>(Ly.w_gate), reinterpret_cast<const uint16_t*>(Ly.w_up),
                      reinterpret_cast<const uint16_t*>(Ly.w_down), reinterpret_cast<uint16_t*>(Ly.k_cache),
                      reinterpret_cast<uint16_t*>(Ly.v_cache)};
    const spts_status st = hip_status(ctx, launch_decode_layer(reinterpret_cast<uint16_t*>(x), d, pos, w, lengths[l],
                                                               Hq, Hkv, f, eps, prenorm == 1, rope_table, scale,
                                                               ctx->ws, ctx->stream),
                                      "decode_step");
    if (st != SPTS_OK) return st;
  }
  for (int l = 0; l < n_layers; ++l) lengths[l] += 1;
  return SPTS_OK;
}

// ------------------------------------------------------------------------ FFN

spts_status spts_reduced_ffn(spts_ctx* ctx, const void* z, const int32_t* rows, const void* w_gate,
                             const void* w_up, const void* w_down, int k, int d, int f, void* y_sel,
                             const int32_t* y_rows, int accumulate) {
  CHECK_CTX();
  REQUIRE(k >= 0 && d > 0 && f > 0, SPTS_ERR_SHAPE, "bad FFN sizes");
  REQUIRE(d % 256 == 0 && f % 128 == 0, SPTS_ERR_UNSUPPORTED, "FFN needs d %% 256 == 0 and f %% 128 == 0");
  REQUIRE(accumulate == 0 || accumulate == 1, SPTS_ERR_INVALID, "accumulate must be 0 or 1");
  {
    const spts_status st = weight_size_ok(ctx, f, d);
    if (st != SPTS_OK) return st;
  }
  if (k == 0) return SPTS_OK;
  REQUIRE_PTR(z); REQUIRE_PTR(w_gate); REQUIRE_PTR(w_up); REQUIRE_PTR(w_down); REQUIRE_PTR(y_sel);
  REQUIRE_ALIGN(z); REQUIRE_ALIGN(w_gate); REQUIRE_ALIGN(w_up); REQUIRE_ALIGN(w_down); REQUIRE_ALIGN(y_sel);
  if (rows) REQUIRE_ALIGN(rows);
  if (y_rows) REQUIRE_ALIGN(y_rows);
  // H must fit; the split part of the workspace is optional (a GEMM whose
  // plan needs more than what is left runs unsplit)
  const size_t h_bytes = round256((size_t)k * f * 2);
  REQUIRE(ctx->ws_bytes >= h_bytes, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, h_bytes);
  uint16_t* H = reinterpret_cast<uint16_t*>(ctx->ws);
  float* split_ws = reinterpret_cast<float*>(reinterpret_cast<char*>(ctx->ws) + h_bytes);
  const size_t split_bytes = ctx->ws_bytes - h_bytes;
  GemmArgs g1{};
  g1.a = reinterpret_cast<const uint16_t*>(z); g1.a_rows = rows; g1.m = k; g1.k = d; g1.lda = d;
  g1.b0 = reinterpret_cast<const uint16_t*>(w_gate); g1.b1 = reinterpret_cast<const uint16_t*>(w_up);
  g1.ldb = d; g1.n = 2 * f; g1.out = H; g1.ldc = f;
  g1.partial = split_bytes ? split_ws : nullptr; g1.partial_bytes = split_bytes;
  hipError_t e = launch_gemm(g1, EPI_SWIGLU, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "reduced_ffn (gate/up)");
  GemmArgs g2{};
  g2.a = H; g2.m = k; g2.k = f; g2.lda = f;
  g2.b0 = reinterpret_cast<const uint16_t*>(w_down); g2.ldb = f; g2.n = d;
  g2.out = y_sel; g2.ldc = d; g2.out_rows = y_rows; g2.accumulate = accumulate;
  g2.partial = split_bytes ? split_ws : nullptr; g2.partial_bytes = split_bytes;
  return hip_status(ctx, launch_gemm(g2, EPI_STORE, ctx->stream), "reduced_ffn (down)");
}

// ------------------------------------------------------------------------ MSDP

spts_status spts_msdp_stage(spts_ctx* ctx, const float* scores, int n_prev, int budget, int n_forced,
                            const int32_t* pos_prev, int32_t* keep, int32_t* pos_new, const void* x_prev,
                            void* x_new, int d) {
  CHECK_CTX();
  REQUIRE_PTR(scores); REQUIRE_PTR(pos_prev); REQUIRE_PTR(keep); REQUIRE_PTR(pos_new);
  REQUIRE_ALIGN(scores); REQUIRE_ALIGN(pos_prev); REQUIRE_ALIGN(keep); REQUIRE_ALIGN(pos_new);
  REQUIRE(n_prev <= kTopkMaxN, SPTS_ERR_UNSUPPORTED, "MSDP stage over %d candidates: at most 2^30", n_prev);
  REQUIRE(n_prev >= 1 && budget >= n_forced && n_forced >= 0 && budget <= n_prev, SPTS_ERR_SHAPE,
          "need n_forced <= budget <= n_prev (n_prev=%d budget=%d n_forced=%d)", n_prev, budget, n_forced);
  if (x_prev) {
    REQUIRE_PTR(x_new); REQUIRE_ALIGN(x_prev); REQUIRE_ALIGN(x_new);
    REQUIRE(d > 0 && d % 8 == 0, SPTS_ERR_SHAPE, "msdp_stage needs d %% 8 == 0");
  }
  const size_t need = topk_workspace(n_prev);
  REQUIRE(ctx->ws_bytes >= need, SPTS_ERR_NOMEM, "workspace %zu < %zu bytes", ctx->ws_bytes, need);
  hipError_t e = launch_topk(scores, nullptr, 0.f, 0.f, false, n_prev, budget, n_forced, keep, nullptr, ctx->ws,
                             ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "msdp_stage (select)");
  e = launch_gather(pos_prev, keep, budget, 4, pos_new, ctx->stream);
  if (e != hipSuccess) return hip_status(ctx, e, "msdp_stage (positions)");
  if (x_prev) {
    e = launch_gather(x_prev, keep, budget, (long)d * 2, x_new, ctx->stream);
    if (e != hipSuccess) return hip_status(ctx, e, "msdp_stage (rows)");
  }
  return SPTS_OK;
}

}  // extern "C"
