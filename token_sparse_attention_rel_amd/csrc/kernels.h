// Host-side launchers of the tsa kernels (one per .hip file), called by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

// Mirrors of the public enums (include/tsa.h) used inside the kernels.
enum { kDtypeF32 = 0, kDtypeBf16 = 1 };
enum { kSelectTopk = 0, kSelectThreshold = 1, kSelectMask = 2, kSelectSchedule = 3 };

struct GroupPeriods {
  uint8_t p[16];
};

// select.hip
hipError_t launch_scores(const void* x_cur, const void* x_ref, long ref_off, long n_rows,
                         long dim, int dtype, int relative, float* scores, hipStream_t s);
hipError_t launch_select(const float* scores, const uint8_t* aux, int n, int mode, int k,
                         float tau, long step, uint8_t* mask, int* idx, int* pidx, int* n_active,
                         uint8_t* group_accum, int accum_first, hipStream_t s);
hipError_t launch_map_groups(const uint8_t* group, int n, const GroupPeriods& table,
                             uint8_t* period_out, hipStream_t s);

// rowops.hip
struct RowSource {
  const void* x;        // token rows [n_x_rows, dim]
  int x_dtype;          // kDtypeF32 / kDtypeBf16
  long n_x_rows;
  const int* rows;      // token of row r, or nullptr for r
  const uint16_t* eps;  // recovery noise [n_x_rows, dim] or nullptr
  long src_off;         // recovery: clean row of token t is x[t - src_off]
  float sigma;
};
hipError_t launch_gather_rows(const RowSource& src, long n, long dim, uint16_t* dst,
                              hipStream_t s);
hipError_t launch_copy_rows2(const uint16_t* a, const uint16_t* b, const int* rows, long n,
                             uint16_t* da, uint16_t* db, long dim, hipStream_t s);

// qkv_gemm.hip
struct QkvOut {
  uint16_t* q;      // [n, dim] or nullptr
  uint16_t* k;      // compact [n, dim] or cache [n_cache, dim]
  uint16_t* v;
  int to_cache;     // k/v row r goes to row rows[r]
  const int* rows = nullptr;  // token of product row r when it differs from the row read
                              // (compact input rows); nullptr: the token read
};
// 3D rotary positions applied to Q and K in the epilogue (heads == 0: none).
struct RopeSpec {
  int heads = 0;
  long height = 1;  // token t sits at frame t / (height*width), row (t / width) % height,
  long width = 1;   // column t % width
  float log2_base = 0.f;
};
hipError_t launch_qkv(const RowSource& src, long n, long dim, const uint16_t* w_qkv,
                      const QkvOut& out, const RopeSpec& rope, hipStream_t s);

// attention.hip
// ws == nullptr: one workgroup per query tile.  Otherwise the split schedule of
// the last round when it pays, with ws of at least attention_workspace_bytes()
// bytes (hipErrorInvalidValue if smaller).
size_t attention_workspace_bytes(long n_q, long n_kv, int heads, int head_dim);
hipError_t launch_attention_causal(const uint16_t* q, const uint16_t* k, const uint16_t* v, long n_q,
                                   long n_kv, int heads, int head_dim, float scale, const int* q_tokens,
                                   long frame_tokens, uint16_t* out, const int* out_rows, float* lse,
                                   hipStream_t s);
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, long n_q,
                            long n_kv, int heads, int head_dim, float scale, uint16_t* out,
                            const int* out_rows, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t s);

// frames.hip
hipError_t launch_euler(void* x, int x_dtype, const uint16_t* v, long n_elems, float dt, hipStream_t s);
long lif_max_dim(int dtype);
hipError_t launch_lif_mask(const void* x, int dtype, long frames, long hw, long dim, int relative, float tau_s,
                           float tau_l, uint8_t* mask, float* short_out, float* long_out, hipStream_t s);
hipError_t launch_restore(void* buf, const uint8_t* mask, long frames, long hw, long row_bytes, hipStream_t s);

// reuse.hip (ws_src, ws_root: n * heads * 3 int32 each)
hipError_t launch_reuse(const uint16_t* v, long n, int heads, int head_dim, long height, long width,
                        const float theta[3], uint16_t* eff, int* src_out, float* delta_out, int* ws_src,
                        int* ws_root, hipStream_t s);

}  // namespace tsa
