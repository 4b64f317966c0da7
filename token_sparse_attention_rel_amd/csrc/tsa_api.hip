// C ABI of libtsa: argument validation, then kernel launches on the caller's stream.
//
// Every entry point validates all arguments before enqueuing anything, so a
// rejected call writes nothing.  Nothing here allocates, frees or
// synchronises; the only state kept between calls is a per-device cache of
// the attention kernel's resident workgroup count.
#include <math.h>

#include <mutex>

#include "../../include/tsa.h"
#include "kernels.h"

namespace {

using tsa::RowSource;

constexpr int64_t kMaxRows = (int64_t{1} << 31) - 1;
// Largest byte range a kernel addresses through one buffer resource (32-bit offsets).
constexpr int64_t kMaxBufferBytes = (int64_t{1} << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

tsa_status from_hip(hipError_t e) { return e == hipSuccess ? TSA_OK : TSA_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

#ifdef TSA_DEBUG
// Debug builds check the documented preconditions of every index list before any
// kernel reads it: entries in [0, limit) and, for token lists, strictly increasing.
// A violation comes back as TSA_ERR_SHAPE (the check synchronises the stream);
// release builds skip it.
__device__ int debug_violation;

__global__ void debug_reset_kernel(int* flag) { *flag = 0; }

__global__ void debug_rows_kernel(const int32_t* rows, long n, long limit, int increasing, int* flag) {
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long>(gridDim.x) * blockDim.x) {
    const long r = rows[i];
    if (r < 0 || r >= limit || (increasing && i > 0 && static_cast<long>(rows[i - 1]) >= r)) *flag = 1;
  }
}

bool debug_rows_ok(const int32_t* rows, int64_t n, int64_t limit, bool increasing, hipStream_t s) {
  int* flag = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&flag), HIP_SYMBOL(debug_violation)) != hipSuccess) return false;
  hipLaunchKernelGGL(debug_reset_kernel, dim3(1), dim3(1), 0, s, flag);
  const long blocks = n / 256 + 1 < 1024 ? n / 256 + 1 : 1024;
  hipLaunchKernelGGL(debug_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, rows,
                     static_cast<long>(n), static_cast<long>(limit), increasing ? 1 : 0, flag);
  int h = 1;
  if (hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return false;
  if (hipStreamSynchronize(s) != hipSuccess) return false;
  return h == 0;
}
#define TSA_CHECK_ROWS(rows, n, limit, increasing, stream)                                  \
  do {                                                                                      \
    if ((rows) && !debug_rows_ok((rows), (n), (limit), (increasing), as_stream(stream))) \
      return TSA_ERR_SHAPE;                                                                 \
  } while (0)
#else
#define TSA_CHECK_ROWS(rows, n, limit, increasing, stream) \
  do {                                                     \
  } while (0)
#endif

}  // namespace

extern "C" {

int tsa_abi_version(void) { return TSA_ABI_VERSION; }

const char* tsa_status_string(int status) {
  switch (status) {
    case TSA_OK: return "ok";
    case TSA_ERR_INVALID_ARG: return "invalid argument";
    case TSA_ERR_SHAPE: return "invalid shape";
    case TSA_ERR_DTYPE: return "unsupported dtype";
    case TSA_ERR_ALIGNMENT: return "buffer not 16-byte aligned";
    case TSA_ERR_WORKSPACE: return "workspace missing or too small";
    case TSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t tsa_select_workspace_bytes(int64_t n_rows) {
  (void)n_rows;
  return 0;
}

tsa_status tsa_select_active(const void* x_cur, const void* x_ref, int64_t ref_row_offset,
                             int64_t n_rows, int64_t dim, int dtype, int score_kind, int mode,
                             int64_t k, float tau, const uint8_t* aux_in, int64_t step,
                             float* scores_out, uint8_t* mask_out, int32_t* idx_out,
                             int32_t* pidx_out, int32_t* n_active_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  (void)workspace;
  if (mode < TSA_SELECT_TOPK || mode > TSA_SELECT_SCHEDULE) return TSA_ERR_INVALID_ARG;
  if (score_kind != TSA_SCORE_REL_L1 && score_kind != TSA_SCORE_ABS_L1) return TSA_ERR_INVALID_ARG;
  if (n_rows < 0 || n_rows > kMaxRows) return TSA_ERR_SHAPE;
  const bool scored = mode == TSA_SELECT_TOPK || mode == TSA_SELECT_THRESHOLD;
  if (!mask_out || !idx_out || !n_active_out) return TSA_ERR_INVALID_ARG;
  if (scored) {
    if (dtype != TSA_F32 && dtype != TSA_BF16) return TSA_ERR_DTYPE;
    if (!x_cur || !scores_out) return TSA_ERR_INVALID_ARG;
    if (dim <= 0 || dim % 8 != 0) return TSA_ERR_SHAPE;
    if (!aligned16(x_cur) || (x_ref && !aligned16(x_ref)) || !aligned16(scores_out))
      return TSA_ERR_ALIGNMENT;
    if (mode == TSA_SELECT_TOPK && (k < 0 || k > n_rows)) return TSA_ERR_SHAPE;
    if (mode == TSA_SELECT_THRESHOLD && isnan(tau)) return TSA_ERR_INVALID_ARG;
  } else {
    if (!aux_in) return TSA_ERR_INVALID_ARG;
    if (mode == TSA_SELECT_SCHEDULE && step < 0) return TSA_ERR_SHAPE;
  }
  if (!aligned4(idx_out) || (pidx_out && !aligned4(pidx_out)) || !aligned4(n_active_out))
    return TSA_ERR_ALIGNMENT;
  if (workspace_bytes < tsa_select_workspace_bytes(n_rows)) return TSA_ERR_WORKSPACE;
  if (n_rows == 0) return TSA_OK;

  hipStream_t s = as_stream(stream);
  if (scored) {
    hipError_t e = tsa::launch_scores(x_cur, x_ref, ref_row_offset, n_rows, dim, dtype,
                                      score_kind == TSA_SCORE_REL_L1, scores_out, s);
    if (e != hipSuccess) return TSA_ERR_HIP;
  }
  return from_hip(tsa::launch_select(scores_out, aux_in, static_cast<int>(n_rows), mode,
                                     static_cast<int>(k), tau, step, mask_out, idx_out, pidx_out,
                                     n_active_out, nullptr, 0, s));
}

tsa_status tsa_token_scores(const void* x_cur, const void* x_ref, int64_t ref_row_offset, int64_t n_rows,
                            int64_t dim, int dtype, int score_kind, float* scores_out, void* stream) {
  if (!x_cur || !scores_out) return TSA_ERR_INVALID_ARG;
  if (score_kind != TSA_SCORE_REL_L1 && score_kind != TSA_SCORE_ABS_L1) return TSA_ERR_INVALID_ARG;
  if (dtype != TSA_F32 && dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (n_rows < 0 || n_rows > kMaxRows || dim <= 0 || dim % 8 != 0) return TSA_ERR_SHAPE;
  if (!aligned16(x_cur) || (x_ref && !aligned16(x_ref)) || !aligned16(scores_out)) return TSA_ERR_ALIGNMENT;
  if (n_rows == 0) return TSA_OK;
  return from_hip(tsa::launch_scores(x_cur, x_ref, ref_row_offset, n_rows, dim, dtype,
                                     score_kind == TSA_SCORE_REL_L1, scores_out, as_stream(stream)));
}

tsa_status tsa_assign_groups(const float* scores, int64_t n, int n_groups,
                             const int64_t* group_counts, const uint8_t* group_periods,
                             uint8_t* period_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!scores || !group_counts || !group_periods || !period_out) return TSA_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows) return TSA_ERR_SHAPE;
  if (n_groups < 1 || n_groups > 16) return TSA_ERR_SHAPE;
  int64_t total = 0;
  for (int g = 0; g < n_groups; ++g) {
    if (group_counts[g] < 0) return TSA_ERR_SHAPE;
    total += group_counts[g];
  }
  if (total != n) return TSA_ERR_SHAPE;
  if (!aligned16(scores)) return TSA_ERR_ALIGNMENT;
  const size_t need = tsa_select_workspace_bytes(n) + static_cast<size_t>(n);
  if (n > 0 && (!workspace || workspace_bytes < need)) return TSA_ERR_WORKSPACE;
  if (n == 0) return TSA_OK;

  hipStream_t s = as_stream(stream);
  uint8_t* group = static_cast<uint8_t*>(workspace) + tsa_select_workspace_bytes(n);
  // Group of a token = number of rank boundaries it falls behind; the top-c
  // sets for increasing cumulative counts c are nested (one total order).
  int64_t cum = 0;
  for (int g = 0; g + 1 < n_groups; ++g) {
    cum += group_counts[g];
    hipError_t e = tsa::launch_select(scores, nullptr, static_cast<int>(n), TSA_SELECT_TOPK,
                                      static_cast<int>(cum), 0.f, 0, nullptr, nullptr, nullptr,
                                      nullptr, group, g == 0, s);
    if (e != hipSuccess) return TSA_ERR_HIP;
  }
  tsa::GroupPeriods table{};
  for (int g = 0; g < n_groups; ++g) table.p[g] = group_periods[g];
  return from_hip(tsa::launch_map_groups(n_groups > 1 ? group : nullptr, static_cast<int>(n), table,
                                         period_out, s));
}

tsa_status tsa_qkv_active(const void* x, int x_dtype, int64_t n_x_rows, const int32_t* rows,
                          int64_t n, int64_t dim, const tsa_bf16* w_qkv, tsa_bf16* q_out,
                          tsa_bf16* k_out, tsa_bf16* v_out, int out_is_cache, int64_t n_cache,
                          const tsa_bf16* eps, int64_t src_row_offset, float sigma,
                          void* stream) {
  if (!x || !w_qkv || !k_out || !v_out) return TSA_ERR_INVALID_ARG;
  if (x_dtype != TSA_F32 && x_dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (eps && x_dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (out_is_cache && !rows) return TSA_ERR_INVALID_ARG;
  if (eps && isnan(sigma)) return TSA_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows || n_x_rows < 0 || n_x_rows > kMaxRows) return TSA_ERR_SHAPE;
  if (dim <= 0 || dim % 64 != 0 || dim > (int64_t{1} << 20)) return TSA_ERR_SHAPE;
  if (!rows && n > n_x_rows) return TSA_ERR_SHAPE;
  if (out_is_cache && (n_cache < 0 || n_cache > kMaxRows)) return TSA_ERR_SHAPE;
  // the weight is read through one 32-bit buffer range
  if (3 * dim * dim * 2 > kMaxBufferBytes) return TSA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w_qkv) || (q_out && !aligned16(q_out)) || !aligned16(k_out) ||
      !aligned16(v_out) || (eps && !aligned16(eps)) || (rows && !aligned4(rows)))
    return TSA_ERR_ALIGNMENT;
  if (n == 0) return TSA_OK;
  TSA_CHECK_ROWS(rows, n, out_is_cache && n_cache < n_x_rows ? n_cache : n_x_rows, true, stream);
  RowSource src{x, x_dtype, n_x_rows, rows, eps, src_row_offset, sigma};
  tsa::QkvOut out{q_out, k_out, v_out, out_is_cache ? 1 : 0};
  return from_hip(tsa::launch_qkv(src, n, dim, w_qkv, out, tsa::RopeSpec{}, as_stream(stream)));
}

tsa_status tsa_qkv_active_rope(const void* x, int x_dtype, int64_t n_x_rows, const int32_t* rows,
                               int64_t n, int64_t dim, const tsa_bf16* w_qkv, tsa_bf16* q_out,
                               tsa_bf16* k_out, tsa_bf16* v_out, int out_is_cache, int64_t n_cache,
                               const tsa_bf16* eps, int64_t src_row_offset, float sigma, int heads,
                               int64_t height, int64_t width, float rope_base, void* stream) {
  if (heads < 1 || heads > 4096 || dim % heads != 0 || (dim / heads) % 2 != 0 || dim / heads < 6)
    return TSA_ERR_SHAPE;
  if (height < 1 || width < 1 || height > kMaxRows || width > kMaxRows || height * width > kMaxRows)
    return TSA_ERR_SHAPE;
  if (!(rope_base > 0.f) || isinf(rope_base)) return TSA_ERR_INVALID_ARG;
  // same validation as tsa_qkv_active
  if (!x || !w_qkv || !k_out || !v_out) return TSA_ERR_INVALID_ARG;
  if (x_dtype != TSA_F32 && x_dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (eps && x_dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (out_is_cache && !rows) return TSA_ERR_INVALID_ARG;
  if (eps && isnan(sigma)) return TSA_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows || n_x_rows < 0 || n_x_rows > kMaxRows) return TSA_ERR_SHAPE;
  if (dim <= 0 || dim % 64 != 0 || dim > (int64_t{1} << 20)) return TSA_ERR_SHAPE;
  if (!rows && n > n_x_rows) return TSA_ERR_SHAPE;
  if (out_is_cache && (n_cache < 0 || n_cache > kMaxRows)) return TSA_ERR_SHAPE;
  if (3 * dim * dim * 2 > kMaxBufferBytes) return TSA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w_qkv) || (q_out && !aligned16(q_out)) || !aligned16(k_out) ||
      !aligned16(v_out) || (eps && !aligned16(eps)) || (rows && !aligned4(rows)))
    return TSA_ERR_ALIGNMENT;
  if (n == 0) return TSA_OK;
  TSA_CHECK_ROWS(rows, n, out_is_cache && n_cache < n_x_rows ? n_cache : n_x_rows, true, stream);
  RowSource src{x, x_dtype, n_x_rows, rows, eps, src_row_offset, sigma};
  tsa::QkvOut out{q_out, k_out, v_out, out_is_cache ? 1 : 0};
  tsa::RopeSpec rope;
  rope.heads = heads;
  rope.height = height;
  rope.width = width;
  rope.log2_base = log2f(rope_base);
  return from_hip(tsa::launch_qkv(src, n, dim, w_qkv, out, rope, as_stream(stream)));
}

tsa_status tsa_qkv_rows_to_cache(const tsa_bf16* a, int64_t n, int64_t dim, const int32_t* rows,
                                 const tsa_bf16* w_qkv, tsa_bf16* q_out, tsa_bf16* k_cache, tsa_bf16* v_cache,
                                 int64_t n_cache, int heads, int64_t height, int64_t width, float rope_base,
                                 void* stream) {
  if (!a || !rows || !w_qkv || !k_cache || !v_cache) return TSA_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows || n_cache < 0 || n_cache > kMaxRows) return TSA_ERR_SHAPE;
  if (dim <= 0 || dim % 64 != 0 || dim > (int64_t{1} << 20)) return TSA_ERR_SHAPE;
  if (3 * dim * dim * 2 > kMaxBufferBytes) return TSA_ERR_SHAPE;
  tsa::RopeSpec rope;
  if (heads != 0) {
    if (heads < 1 || heads > 4096 || dim % heads != 0 || (dim / heads) % 2 != 0 || dim / heads < 6)
      return TSA_ERR_SHAPE;
    if (height < 1 || width < 1 || height > kMaxRows || width > kMaxRows || height * width > kMaxRows)
      return TSA_ERR_SHAPE;
    if (!(rope_base > 0.f) || isinf(rope_base)) return TSA_ERR_INVALID_ARG;
    rope.heads = heads;
    rope.height = height;
    rope.width = width;
    rope.log2_base = log2f(rope_base);
  }
  if (!aligned16(a) || !aligned16(w_qkv) || (q_out && !aligned16(q_out)) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned4(rows))
    return TSA_ERR_ALIGNMENT;
  if (n == 0) return TSA_OK;
  TSA_CHECK_ROWS(rows, n, n_cache, true, stream);
  RowSource src{a, TSA_BF16, n, nullptr, nullptr, 0, 0.f};
  tsa::QkvOut out{q_out, k_cache, v_cache, 1, rows};
  return from_hip(tsa::launch_qkv(src, n, dim, w_qkv, out, rope, as_stream(stream)));
}

tsa_status tsa_kv_cache_sync(const tsa_bf16* k_a, const tsa_bf16* v_a, const int32_t* rows,
                             int64_t n, tsa_bf16* k_cache, tsa_bf16* v_cache, int64_t n_cache,
                             int64_t dim, void* stream) {
  if (!k_a || !v_a || !rows || !k_cache || !v_cache) return TSA_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows || n_cache < 0 || n_cache > kMaxRows) return TSA_ERR_SHAPE;
  if (n > n_cache || dim <= 0 || dim % 8 != 0) return TSA_ERR_SHAPE;
  if (!aligned16(k_a) || !aligned16(v_a) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(rows))
    return TSA_ERR_ALIGNMENT;
  if (n == 0) return TSA_OK;
  TSA_CHECK_ROWS(rows, n, n_cache, true, stream);
  return from_hip(tsa::launch_copy_rows2(k_a, v_a, rows, n, k_cache, v_cache, dim,
                                         as_stream(stream)));
}

tsa_status tsa_sparse_query_attention(const tsa_bf16* q, const tsa_bf16* k_cache,
                                      const tsa_bf16* v_cache, int64_t n_q, int64_t n_kv,
                                      int heads, int head_dim, float scale, tsa_bf16* out,
                                      const int32_t* out_rows, int64_t n_out, float* lse_out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !out) return TSA_ERR_INVALID_ARG;
  if (isnan(scale) || isinf(scale)) return TSA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return TSA_ERR_SHAPE;
  if (heads < 1 || heads > 4096) return TSA_ERR_SHAPE;
  if (n_q < 0 || n_q > kMaxRows || n_kv < 1 || n_kv > kMaxRows) return TSA_ERR_SHAPE;
  if (out_rows && (n_out < 0 || n_out > kMaxRows)) return TSA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (out_rows && !aligned4(out_rows)) || (lse_out && !aligned4(lse_out)) ||
      (workspace && !aligned16(workspace)))
    return TSA_ERR_ALIGNMENT;
  if (n_q == 0) return TSA_OK;
  if (workspace && workspace_bytes < tsa::attention_workspace_bytes(n_q, n_kv, heads, head_dim))
    return TSA_ERR_WORKSPACE;
  TSA_CHECK_ROWS(out_rows, n_q, n_out, true, stream);
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf(static_cast<float>(head_dim));
  return from_hip(tsa::launch_attention(q, k_cache, v_cache, n_q, n_kv, heads, head_dim, sc, out,
                                        out_rows, lse_out, workspace, workspace_bytes,
                                        as_stream(stream)));
}

tsa_status tsa_frame_causal_attention(const tsa_bf16* q, const tsa_bf16* k_cache, const tsa_bf16* v_cache,
                                      int64_t n_q, int64_t n_kv, int heads, int head_dim, float scale,
                                      const int32_t* q_tokens, int64_t frame_tokens, tsa_bf16* out,
                                      const int32_t* out_rows, int64_t n_out, float* lse_out, void* stream) {
  if (!q || !k_cache || !v_cache || !out || !q_tokens) return TSA_ERR_INVALID_ARG;
  if (isnan(scale) || isinf(scale)) return TSA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return TSA_ERR_SHAPE;
  if (heads < 1 || heads > 4096) return TSA_ERR_SHAPE;
  if (n_q < 0 || n_q > kMaxRows || n_kv < 1 || n_kv > kMaxRows) return TSA_ERR_SHAPE;
  if (frame_tokens < 1 || frame_tokens > kMaxRows) return TSA_ERR_SHAPE;
  if (out_rows && (n_out < 0 || n_out > kMaxRows)) return TSA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned4(q_tokens) ||
      (out_rows && !aligned4(out_rows)) || (lse_out && !aligned4(lse_out)))
    return TSA_ERR_ALIGNMENT;
  if (n_q == 0) return TSA_OK;
  TSA_CHECK_ROWS(q_tokens, n_q, kMaxRows, false, stream);
  TSA_CHECK_ROWS(out_rows, n_q, n_out, true, stream);
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf(static_cast<float>(head_dim));
  return from_hip(tsa::launch_attention_causal(q, k_cache, v_cache, n_q, n_kv, heads, head_dim, sc, q_tokens,
                                               frame_tokens, out, out_rows, lse_out, as_stream(stream)));
}

size_t tsa_attention_workspace_bytes(int64_t n_q, int64_t n_kv, int heads, int head_dim) {
  if ((head_dim != 64 && head_dim != 128) || heads < 1 || heads > 4096 || n_q < 1 || n_q > kMaxRows ||
      n_kv < 1 || n_kv > kMaxRows)
    return 0;
  return tsa::attention_workspace_bytes(n_q, n_kv, heads, head_dim);
}

tsa_status tsa_scatter_out(const tsa_bf16* o_a, const int32_t* rows, int64_t n, tsa_bf16* out,
                           int64_t n_out, int64_t dim, void* stream) {
  if (!o_a || !rows || !out) return TSA_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows || n_out < 0 || n_out > kMaxRows) return TSA_ERR_SHAPE;
  if (n > n_out || dim <= 0 || dim % 8 != 0) return TSA_ERR_SHAPE;
  if (!aligned16(o_a) || !aligned16(out) || !aligned4(rows)) return TSA_ERR_ALIGNMENT;
  if (n == 0) return TSA_OK;
  TSA_CHECK_ROWS(rows, n, n_out, true, stream);
  return from_hip(
      tsa::launch_copy_rows2(o_a, nullptr, rows, n, out, nullptr, dim, as_stream(stream)));
}

tsa_status tsa_gather_rows(const tsa_bf16* x, int64_t n_x_rows, const int32_t* rows, int64_t n,
                           int64_t dim, const tsa_bf16* eps, int64_t src_row_offset, float sigma,
                           tsa_bf16* dst, void* stream) {
  if (!x || !rows || !dst) return TSA_ERR_INVALID_ARG;
  if (eps && isnan(sigma)) return TSA_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows || n_x_rows < 0 || n_x_rows > kMaxRows) return TSA_ERR_SHAPE;
  if (dim <= 0 || dim % 8 != 0) return TSA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(dst) || (eps && !aligned16(eps)) || !aligned4(rows))
    return TSA_ERR_ALIGNMENT;
  if (n == 0) return TSA_OK;
  TSA_CHECK_ROWS(rows, n, n_x_rows, true, stream);
  RowSource src{x, TSA_BF16, n_x_rows, rows, eps, src_row_offset, sigma};
  return from_hip(tsa::launch_gather_rows(src, n, dim, dst, as_stream(stream)));
}

tsa_status tsa_euler_update(void* x, int x_dtype, const tsa_bf16* v_hat, int64_t n_rows, int64_t dim,
                            float dt, void* stream) {
  if (!x || !v_hat || isnan(dt) || isinf(dt)) return TSA_ERR_INVALID_ARG;
  if (x_dtype != TSA_F32 && x_dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (n_rows < 0 || n_rows > kMaxRows || dim <= 0 || dim % 8 != 0 || dim > kMaxRows) return TSA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(v_hat)) return TSA_ERR_ALIGNMENT;
  if (n_rows == 0) return TSA_OK;
  return from_hip(tsa::launch_euler(x, x_dtype, v_hat, n_rows * dim, dt, as_stream(stream)));
}

tsa_status tsa_lif_mask(const void* x, int dtype, int64_t frames, int64_t hw, int64_t dim, int score_kind,
                        float tau_short, float tau_long, uint8_t* mask_out, float* short_out,
                        float* long_out, void* stream) {
  if (!x || !mask_out || isnan(tau_short) || isnan(tau_long)) return TSA_ERR_INVALID_ARG;
  if (score_kind != TSA_SCORE_REL_L1 && score_kind != TSA_SCORE_ABS_L1) return TSA_ERR_INVALID_ARG;
  if (dtype != TSA_F32 && dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (frames < 1 || hw < 1 || frames > kMaxRows || hw > kMaxRows || frames * hw > kMaxRows)
    return TSA_ERR_SHAPE;
  if (dim <= 0 || dim % 8 != 0 || dim > tsa::lif_max_dim(dtype)) return TSA_ERR_SHAPE;
  if (!aligned16(x) || (short_out && !aligned4(short_out)) || (long_out && !aligned4(long_out)))
    return TSA_ERR_ALIGNMENT;
  return from_hip(tsa::launch_lif_mask(x, dtype, frames, hw, dim, score_kind == TSA_SCORE_REL_L1, tau_short,
                                       tau_long, mask_out, short_out, long_out, as_stream(stream)));
}

tsa_status tsa_restore_frames(void* buf, int dtype, const uint8_t* mask, int64_t frames, int64_t hw,
                              int64_t dim, void* stream) {
  if (!buf || !mask) return TSA_ERR_INVALID_ARG;
  if (dtype != TSA_F32 && dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (frames < 1 || hw < 1 || frames > kMaxRows || hw > kMaxRows || frames * hw > kMaxRows)
    return TSA_ERR_SHAPE;
  if (dim <= 0 || dim % 8 != 0 || dim > kMaxRows) return TSA_ERR_SHAPE;
  const int64_t row_bytes = dim * (dtype == TSA_F32 ? 4 : 2);
  if (hw * (row_bytes / 16) > kMaxRows * 64) return TSA_ERR_SHAPE;  // grid size
  if (!aligned16(buf)) return TSA_ERR_ALIGNMENT;
  if (frames == 1) return TSA_OK;
  return from_hip(tsa::launch_restore(buf, mask, frames, hw, row_bytes, as_stream(stream)));
}

size_t tsa_reuse_workspace_bytes(int64_t n_rows, int heads) {
  if (n_rows <= 0 || heads <= 0) return 0;
  return static_cast<size_t>(2) * static_cast<size_t>(n_rows) * static_cast<size_t>(heads) * 3 * 4;
}

}  // extern "C"

namespace {

// Argument checks of tsa_timeripple_reuse (everything but the workspace).
tsa_status check_reuse(const tsa_bf16* v, int64_t n_rows, int heads, int head_dim, int64_t height, int64_t width,
                       const float* thetas, const tsa_bf16* v_eff, const int32_t* src_out, const float* delta_out) {
  if (!v || !v_eff || !thetas) return TSA_ERR_INVALID_ARG;
  for (int a = 0; a < 3; ++a)
    if (isnan(thetas[a]) || thetas[a] < 0.f) return TSA_ERR_INVALID_ARG;
  if (heads < 1 || heads > 4096 || (head_dim != 64 && head_dim != 128)) return TSA_ERR_SHAPE;
  if (n_rows < 0 || n_rows > kMaxRows) return TSA_ERR_SHAPE;
  if (height < 1 || width < 1 || height > kMaxRows || width > kMaxRows || height * width > kMaxRows)
    return TSA_ERR_SHAPE;
  // token entries (n * heads * 3) and 4-byte channel pairs are indexed with 32-bit grids
  if (n_rows * heads * 3 > kMaxRows || n_rows * heads * (head_dim / 2) > kMaxRows * 256) return TSA_ERR_SHAPE;
  const int64_t row_bytes = static_cast<int64_t>(heads) * head_dim * 2;
  const uintptr_t vb = reinterpret_cast<uintptr_t>(v), eb = reinterpret_cast<uintptr_t>(v_eff);
  const uintptr_t span = static_cast<uintptr_t>(n_rows * row_bytes);
  if (n_rows > 0 && vb < eb + span && eb < vb + span) return TSA_ERR_INVALID_ARG;  // overlap
  if (!aligned16(v) || !aligned16(v_eff) || (src_out && !aligned4(src_out)) || (delta_out && !aligned4(delta_out)))
    return TSA_ERR_ALIGNMENT;
  return TSA_OK;
}

// Scratch of tsa_timeripple_reuse_noalloc: the source and root tables (n * heads * 3
// int32 each) for up to kNoallocMaxTokenHeads token-heads.  One copy per GPU, held
// until the process ends; every entry a call reads is written earlier in the same call,
// so nothing has to start at zero.
constexpr int64_t kNoallocMaxTokenHeads = int64_t{1} << 20;
constexpr size_t kNoallocScratchBytes = 2 * 3 * 4 * static_cast<size_t>(kNoallocMaxTokenHeads);  // 24 MiB
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
constexpr int kNoallocMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kNoallocMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the current device (looked up the first time the
// device is seen, with that device current).
tsa_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocMaxDevices) return TSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TSA_OK;
}

}  // namespace

extern "C" {

tsa_status tsa_timeripple_reuse(const tsa_bf16* v, int64_t n_rows, int heads, int head_dim, int64_t height,
                                int64_t width, const float* thetas, tsa_bf16* v_eff, int32_t* src_out,
                                float* delta_out, void* workspace, size_t workspace_bytes, void* stream) {
  const tsa_status st = check_reuse(v, n_rows, heads, head_dim, height, width, thetas, v_eff, src_out, delta_out);
  if (st != TSA_OK) return st;
  if (n_rows == 0) return TSA_OK;
  if (!workspace || workspace_bytes < tsa_reuse_workspace_bytes(n_rows, heads)) return TSA_ERR_WORKSPACE;
  if (!aligned4(workspace)) return TSA_ERR_ALIGNMENT;
  int* ws_src = static_cast<int*>(workspace);
  int* ws_root = ws_src + n_rows * heads * 3;
  return from_hip(tsa::launch_reuse(v, n_rows, heads, head_dim, height, width, thetas, v_eff, src_out, delta_out,
                                    ws_src, ws_root, as_stream(stream)));
}

size_t tsa_reuse_noalloc_max_token_heads(void) { return static_cast<size_t>(kNoallocMaxTokenHeads); }

tsa_status tsa_timeripple_reuse_noalloc(const tsa_bf16* v, int64_t n_rows, int heads, int head_dim, int64_t height,
                                        int64_t width, const float* thetas, tsa_bf16* v_eff, int32_t* src_out,
                                        float* delta_out, void* stream) {
  const tsa_status st = check_reuse(v, n_rows, heads, head_dim, height, width, thetas, v_eff, src_out, delta_out);
  if (st != TSA_OK) return st;
  if (n_rows * heads > kNoallocMaxTokenHeads) return TSA_ERR_SHAPE;
  if (n_rows == 0) return TSA_OK;
  void* ws = nullptr;
  const tsa_status sst = noalloc_scratch(&ws);
  if (sst != TSA_OK) return sst;
  int* ws_src = static_cast<int*>(ws);
  int* ws_root = ws_src + n_rows * heads * 3;
  return from_hip(tsa::launch_reuse(v, n_rows, heads, head_dim, height, width, thetas, v_eff, src_out, delta_out,
                                    ws_src, ws_root, as_stream(stream)));
}

}  // extern "C"
