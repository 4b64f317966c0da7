// a4 + a5 (+ a6): QKV projection of the selected token rows on bf16 MFMA.
//
// HSA page §2.2 item 1: only the active tokens go through the Q/K/V
// projections.  LIPAR page §2.C: pruned tokens get K/V from their recovered
// row (clean previous latent re-noised with fresh noise).
//
// The product is computed transposed, C^T[col, tok] = sum_k W[col, k] * A[tok, k],
// with both operands K-contiguous (W is [3D, D] output-feature-major, A rows
// are token rows), so every MFMA operand is one 16-byte LDS read.  The gather
// of token rows (or the recovery arithmetic) happens in the A-tile loader,
// so the compact input matrix never exists in HBM.  In the accumulator
// layout of v_mfma_f32_32x32x16_bf16 each lane holds one token and four
// consecutive output features per group, so the epilogue writes 8-byte
// pieces of a token row -- straight into the cache row of that token when
// the cache sync is fused.
//
// Tile: 128 output features x 128 tokens x 64 (K) per step, 4 waves in a 2x2
// arrangement, each wave 64 x 64 (2 x 2 MFMA blocks).  Global -> register
// prefetch of the next K step overlaps the MFMAs of the current one.
#include "common.h"
#include "kernels.h"

namespace tsa {

constexpr int kGemmBM = 128;  // output features per block
constexpr int kGemmBN = 128;  // tokens per block
constexpr int kGemmBK = 64;
constexpr int kGemmLD = kGemmBK + 8;  // LDS row stride (elements): 144 B, conflict-free 16-byte reads

enum { kSrcBf16 = 0, kSrcF32 = 1, kSrcRecover = 2 };

struct GemmArgs {
  const void* x;
  long n_x_rows;
  const int* rows;
  const uint16_t* eps;
  long src_off;
  float sigma;
  long n;       // token rows
  long dim;     // D (= K)
  long col0;    // first output feature handled (0, or D for K/V only)
  long ncols;   // 3D - col0
  const uint16_t* w;
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  int to_cache;
};

template <int SRC>
__device__ __forceinline__ u32x4 load_a_chunk(const GemmArgs& a, long tok, bool valid,
                                              bool has_clean, long k0) {
  if (!valid) return u32x4{0u, 0u, 0u, 0u};
  if (SRC == kSrcBf16) {
    return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + tok * a.dim + k0);
  } else if (SRC == kSrcF32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + tok * a.dim + k0);
    const f32x4 lo = p[0], hi = p[1];
    return u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                 pack_bf16x2(hi[2], hi[3])};
  } else {
    const u32x4 e = *reinterpret_cast<const u32x4*>(a.eps + tok * a.dim + k0);
    const u32x4 c = has_clean ? *reinterpret_cast<const u32x4*>(
                                    static_cast<const uint16_t*>(a.x) + (tok - a.src_off) * a.dim + k0)
                              : u32x4{0u, 0u, 0u, 0u};
    float fc[8], fe[8];
    unpack8(c, fc);
    unpack8(e, fe);
    const float oms = 1.0f - a.sigma;
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = pack_bf16x2(fmaf(oms, fc[2 * i], a.sigma * fe[2 * i]),
                         fmaf(oms, fc[2 * i + 1], a.sigma * fe[2 * i + 1]));
    return r;
  }
}

template <int SRC>
__global__ __launch_bounds__(256, 2) void qkv_gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) uint16_t ws[kGemmBM * kGemmLD];
  __shared__ __align__(16) uint16_t as[kGemmBN * kGemmLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long c_base = a.col0 + static_cast<long>(blockIdx.x) * kGemmBM;  // absolute feature
  const long t_base = static_cast<long>(blockIdx.y) * kGemmBN;            // compact token row
  const long c_end = a.col0 + a.ncols;

  // Loader slots: 4 rows per thread of each tile, 16-byte chunk (tid & 7) of the K slice.
  const int lrow = tid >> 3;
  const int lcol = (tid & 7) * 8;
  const uint16_t* wrow[4];
  bool wvalid[4];
  long tok[4];
  bool tvalid[4], tclean[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long c = c_base + lrow + 32 * j;
    wvalid[j] = c < c_end;
    wrow[j] = a.w + (wvalid[j] ? c : 0) * a.dim + lcol;
    const long r = t_base + lrow + 32 * j;
    tvalid[j] = r < a.n;
    tok[j] = tvalid[j] ? (a.rows ? static_cast<long>(a.rows[r]) : r) : 0;
    const long src = tok[j] - a.src_off;
    tclean[j] = src >= 0 && src < a.n_x_rows;
  }

  u32x4 wreg[4], areg[4];
  auto load_tiles = [&](long k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wreg[j] = wvalid[j] ? *reinterpret_cast<const u32x4*>(wrow[j] + k0) : u32x4{0u, 0u, 0u, 0u};
      areg[j] = load_a_chunk<SRC>(a, tok[j], tvalid[j], tclean[j], k0 + lcol);
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4*>(&ws[(lrow + 32 * j) * kGemmLD + lcol]) = wreg[j];
      *reinterpret_cast<u32x4*>(&as[(lrow + 32 * j) * kGemmLD + lcol]) = areg[j];
    }
  };

  const int wc = wave >> 1;  // feature half of the block
  const int wt = wave & 1;   // token half of the block
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load_tiles(0);
  store_tiles();
  __syncthreads();

  const int l32 = lane & 31;
  const int khalf = (lane >> 5) * 8;
  for (long k0 = 0; k0 < a.dim; k0 += kGemmBK) {
    const bool more = k0 + kGemmBK < a.dim;
    if (more) load_tiles(k0 + kGemmBK);
#pragma unroll
    for (int ks = 0; ks < kGemmBK / 16; ++ks) {
      const int kk = ks * 16 + khalf;
      bf16x8 fw[2], ft[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fw[i] = *reinterpret_cast<const bf16x8*>(&ws[(wc * 64 + i * 32 + l32) * kGemmLD + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        ft[j] = *reinterpret_cast<const bf16x8*>(&as[(wt * 64 + j * 32 + l32) * kGemmLD + kk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], ft[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      store_tiles();
      __syncthreads();
    }
  }

  // Epilogue: lane holds token (l32) and features 8g + 4*(lane/32) + 0..3 of each 32-block.
  const int fsub = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long r = t_base + wt * 64 + j * 32 + l32;
    if (r >= a.n) continue;
    const long t = a.rows ? static_cast<long>(a.rows[r]) : r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const long c = c_base + wc * 64 + i * 32 + g * 8 + fsub;
        if (c >= c_end) continue;
        const long part = c / a.dim;
        const long cc = c - part * a.dim;
        uint16_t* base;
        long row;
        if (part == 0) {
          base = a.q;
          row = r;
        } else {
          base = part == 1 ? a.k : a.v;
          row = a.to_cache ? t : r;
        }
        const u32x2 val{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                        pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        *reinterpret_cast<u32x2*>(base + row * a.dim + cc) = val;
      }
    }
  }
}

hipError_t launch_qkv(const RowSource& src, long n, long dim, const uint16_t* w_qkv,
                      const QkvOut& out, hipStream_t s) {
  GemmArgs a;
  a.x = src.x;
  a.n_x_rows = src.n_x_rows;
  a.rows = src.rows;
  a.eps = src.eps;
  a.src_off = src.src_off;
  a.sigma = src.sigma;
  a.n = n;
  a.dim = dim;
  a.col0 = out.q ? 0 : dim;
  a.ncols = 3 * dim - a.col0;
  a.w = w_qkv;
  a.q = out.q;
  a.k = out.k;
  a.v = out.v;
  a.to_cache = out.to_cache;
  const dim3 grid(static_cast<unsigned>((a.ncols + kGemmBM - 1) / kGemmBM),
                  static_cast<unsigned>((n + kGemmBN - 1) / kGemmBN));
  if (src.eps) {
    hipLaunchKernelGGL(qkv_gemm_kernel<kSrcRecover>, grid, dim3(256), 0, s, a);
  } else if (src.x_dtype == kDtypeF32) {
    hipLaunchKernelGGL(qkv_gemm_kernel<kSrcF32>, grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(qkv_gemm_kernel<kSrcBf16>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tsa
