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
// Optionally the epilogue rotates Q and K by their tokens' 3D positions (rotary
// embedding over time / height / width channel groups) before rounding.
//
// Tile: 256 output features x 256 tokens x 64 (K) per step, 8 waves in a 4x2
// arrangement, each wave 64 features x 128 tokens (2 x 4 MFMA blocks): six
// 16-byte LDS reads feed eight MFMAs, and each staged K slice is shared by 256
// columns and 256 tokens.  Two LDS buffers, one barrier per K step.  Grids of
// fewer than four such tiles per CU use 128 x 128 tiles on 4 waves instead (two
// workgroups per CU).  bf16 rows -- the common case -- are copied from HBM straight
// into LDS (qkv_gemm_lds_kernel: no registers, the next K step's copy in flight
// while the current one is multiplied); rows that need arithmetic on the way (the
// recovery blend, fp32 input) go through registers, loaded two K steps ahead
// (qkv_gemm_kernel).  All rows arrive through
// range-checked buffer loads (invalid rows read as zeros, no per-step selects);
// token rows of 2 GiB or more (whose byte offsets exceed the buffer loads' 32 bits)
// take kernel variants (BIG) that address every row with a 64-bit pointer instead.
#include "common.h"
#include "kernels.h"

namespace tsa {

constexpr int kGemmBK = 64;
constexpr int kGemmLD = kGemmBK + 8;  // LDS row stride (elements): 144 B, conflict-free 16-byte reads

// Workgroup tile: WF x WT waves, each BF x BT MFMA blocks of 32 x 32 (features x tokens).
template <int WF, int WT, int BF, int BT, int MIN_BLOCKS>
struct GemmTile {
  static constexpr int kWavesT = WT;
  static constexpr int kBF = BF;                      // 32-feature MFMA blocks per wave
  static constexpr int kBT = BT;                      // 32-token MFMA blocks per wave
  static constexpr int kThreads = 64 * WF * WT;
  static constexpr int kBM = WF * BF * 32;            // output features per block
  static constexpr int kBN = WT * BT * 32;            // tokens per block
  static constexpr int kLoadRows = kThreads / 8;      // tile rows staged per load round
  static constexpr int kLoadW = kBM / kLoadRows;      // 16-byte W chunks per thread and K step
  static constexpr int kLoadA = kBN / kLoadRows;      // 16-byte A chunks per thread and K step
  static constexpr int kMinBlocks = MIN_BLOCKS;       // resident workgroups per CU
};
// 256 x 256 on 8 waves of 64 x 128 (one workgroup per CU; LDS: 144 KB register-staged with
// padded rows, 128 KB LDS-direct with unpadded swizzled rows) for grids that fill the chip
// several times; 128 x 128 on 4 waves of 64 x 64 (72 / 64 KB, two per CU) for smaller ones,
// where the large tile's last wave of workgroups would leave CUs idle.
using TileLarge = GemmTile<4, 2, 2, 4, 1>;
using TileSmall = GemmTile<2, 2, 2, 2, 2>;
// The large tile is used from this many workgroups on (four per CU of a 256-CU chip).
constexpr long kLargeTileMinBlocks = 1024;

enum { kSrcBf16 = 0, kSrcF32 = 1, kSrcRecover = 2 };

struct GemmArgs {
  const void* x;
  long n_x_rows;
  const int* rows;      // token row read for product row r (nullptr: r)
  const int* out_rows;  // token of product row r for the cache rows and positions
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
  // rotary positions of Q and K (rope_d == 0: none)
  int rope_d;        // head dim
  int rope_dt;       // channels of the time axis; the height and width axes get rope_ds each
  int rope_ds;
  long rope_hw;      // tokens per frame
  long rope_w;       // tokens per row
  float rope_log2_base;
};

// Rotate the channel pair (x0, x1) = (feature j, j+1) of a head (j even) by the
// position of its token along the pair's axis: the time axis owns channels
// [0, dt), the height axis [dt, dt+ds), the width axis [dt+ds, d); pair i of
// an axis group of size n turns by pos * base^(-2i/n).  pos = (frame, row, column).
__device__ __forceinline__ void rope_pair(const GemmArgs& a, const float pos[3], int j, float& x0, float& x1) {
  int i, n, ax;
  if (j < a.rope_dt) {
    i = j >> 1;
    n = a.rope_dt;
    ax = 0;
  } else if (j < a.rope_dt + a.rope_ds) {
    i = (j - a.rope_dt) >> 1;
    n = a.rope_ds;
    ax = 1;
  } else {
    i = (j - a.rope_dt - a.rope_ds) >> 1;
    n = a.rope_ds;
    ax = 2;
  }
  const float freq = exp2f(-(2.0f * static_cast<float>(i) / static_cast<float>(n)) * a.rope_log2_base);
  float sn, cs;
  sincosf(pos[ax] * freq, &sn, &cs);
  const float y0 = x0 * cs - x1 * sn;
  const float y1 = x0 * sn + x1 * cs;
  x0 = y0;
  x1 = y1;
}

// Word 3 of a raw buffer resource on gfx9-class GPUs; offsets past num_records read zero.
constexpr int kBufferRsrcFlags = 0x00020000;
// A per-lane offset that is always out of range: the load returns zeros.
constexpr int kOutOfRange = 0x7FFFFFF0;
// Largest byte range one buffer resource describes here (its offsets are 32-bit).
constexpr long kMaxRangeBytes = 0x7FFFFFFF;

// Token tiles handled together per XCD: the workgroups that run at the same
// time on one XCD then share few W panels and few token tiles in its L2.
constexpr int kTokGroup = 4;

// First output feature (absolute) and first compact token row of this workgroup's tile.
// Tile order: XCD-aware, then groups of kTokGroup token tiles with the token tile
// varying fastest, so concurrently running workgroups share W panels.
template <typename TL>
__device__ __forceinline__ void tile_origin(const GemmArgs& a, long& c_base, long& t_base) {
  const long n_col = (a.ncols + TL::kBM - 1) / TL::kBM;
  const long n_tok = (a.n + TL::kBN - 1) / TL::kBN;
  const long L = xcd_remap(blockIdx.x, n_col * n_tok);
  const long grp = L / (kTokGroup * n_col);
  const long first_tok = grp * kTokGroup;
  const long gsize = (n_tok - first_tok) < kTokGroup ? (n_tok - first_tok) : kTokGroup;
  const long local = L - grp * kTokGroup * n_col;
  const long tok_tile = first_tok + local % gsize;
  const long col_tile = local / gsize;
  c_base = a.col0 + col_tile * TL::kBM;
  t_base = tok_tile * TL::kBN;
}

// Epilogue: lane holds token (l32) and features 8g + 4*(lane/32) + 0..3 of each 32-block.
// Q goes to compact row r; K and V to compact row r or, fused cache sync, to the
// token's cache row.  Optionally Q and K are rotated by the token's 3D position.
template <typename TL>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const f32x16 (&acc)[TL::kBF][TL::kBT],
                                           long c_base, long t_base, int wc, int wt, int lane) {
  constexpr int kWaveBF = TL::kBF, kWaveBT = TL::kBT;
  const long c_end = a.col0 + a.ncols;
  const int l32 = lane & 31;
  const int fsub = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < kWaveBT; ++j) {
    const long r = t_base + (wt * kWaveBT + j) * 32 + l32;
    if (r >= a.n) continue;
    const long t = a.out_rows ? static_cast<long>(a.out_rows[r]) : r;
    float pos[3] = {0.f, 0.f, 0.f};
    if (a.rope_d) {
      const unsigned tu = static_cast<unsigned>(t), hw = static_cast<unsigned>(a.rope_hw),
                     w = static_cast<unsigned>(a.rope_w);
      const unsigned in_frame = tu % hw;
      pos[0] = static_cast<float>(tu / hw);
      pos[1] = static_cast<float>(in_frame / w);
      pos[2] = static_cast<float>(in_frame % w);
    }
#pragma unroll
    for (int i = 0; i < kWaveBF; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const long c = c_base + (wc * kWaveBF + i) * 32 + g * 8 + fsub;
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
        float o[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (a.rope_d && part < 2) {
          const int hj = static_cast<int>(cc % a.rope_d);
          rope_pair(a, pos, hj, o[0], o[1]);
          rope_pair(a, pos, hj + 2, o[2], o[3]);
        }
        const u32x2 val{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(base + row * a.dim + cc) = val;
      }
    }
  }
}

// Rows that need arithmetic on the way (the recovery blend, fp32 input): staged
// through registers, loaded two K steps ahead and converted when stored to padded
// LDS rows one step ahead.
template <int SRC, typename TL, bool BIG = false>
__global__ __launch_bounds__(TL::kThreads, TL::kMinBlocks) void qkv_gemm_kernel(GemmArgs a) {
  static_assert(SRC == kSrcRecover || SRC == kSrcF32, "bf16 rows take qkv_gemm_lds_kernel");
  static_assert(!BIG || SRC == kSrcRecover, "fp32 rows are always read through 64-bit pointers");
  constexpr int kGemmBM = TL::kBM, kGemmBN = TL::kBN, kGemmWavesT = TL::kWavesT;
  constexpr int kWaveBF = TL::kBF, kWaveBT = TL::kBT;
  constexpr int kLoadRows = TL::kLoadRows, kLoadW = TL::kLoadW, kLoadA = TL::kLoadA;
  __shared__ __align__(16) uint16_t ws[2][kGemmBM * kGemmLD];
  __shared__ __align__(16) uint16_t as[2][kGemmBN * kGemmLD];

  long c_base, t_base;
  tile_origin<TL>(a, c_base, t_base);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long c_end = a.col0 + a.ncols;

  // Loader slots: rows lrow + kLoadRows*j of each tile, 16-byte chunk (tid & 7) of the K slice.
  const int lrow = tid >> 3;
  const int lcol = (tid & 7) * 8;
  const long dim = a.dim;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w), 0, static_cast<int>(3 * dim * dim * 2), kBufferRsrcFlags);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.x), 0, static_cast<int>(a.n_x_rows * dim * 2), kBufferRsrcFlags);
  // The A chunks are loaded raw and converted only when written to LDS, one K
  // step later, so the conversion never waits on a load just issued.
  //   recovery: raw[0] = clean chunk (zeros when the token has no clean row), raw[1] = noise
  //   fp32:     raw[0], raw[1] = the two 16-byte halves (invalid rows read row 0, zeroed at the store)
  const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.eps), 0, SRC == kSrcRecover ? static_cast<int>(a.n_x_rows * dim * 2) : 0,
      kBufferRsrcFlags);
  int w_off[kLoadW], x_off[kLoadA], e_off[kLoadA];
  long ftok[kLoadA];
  bool tvalid[kLoadA], tclean[kLoadA];
  // BIG recovery rows: 64-bit pointers to the clean and noise chunks (row 0 when the
  // row has none; the value read is then replaced by zeros)
  const uint16_t* xp[BIG ? kLoadA : 1];
  const uint16_t* ep[BIG ? kLoadA : 1];
#pragma unroll
  for (int j = 0; j < kLoadW; ++j) {
    const long c = c_base + lrow + kLoadRows * j;
    w_off[j] = c < c_end ? static_cast<int>((c * dim + lcol) * 2) : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < kLoadA; ++j) {
    const long r = t_base + lrow + kLoadRows * j;
    tvalid[j] = r < a.n;
    const long tok = tvalid[j] ? (a.rows ? static_cast<long>(a.rows[r]) : r) : 0;
    ftok[j] = tok;
    if constexpr (SRC == kSrcRecover) {
      const long src = tok - a.src_off;
      const bool clean = tvalid[j] && src >= 0 && src < a.n_x_rows;
      tclean[j] = clean;
      if constexpr (BIG) {
        xp[j] = static_cast<const uint16_t*>(a.x) + (clean ? src : 0) * dim + lcol;
        ep[j] = a.eps + tok * dim + lcol;
        x_off[j] = e_off[j] = 0;
      } else {
        x_off[j] = clean ? static_cast<int>((src * dim + lcol) * 2) : kOutOfRange;
        e_off[j] = tvalid[j] ? static_cast<int>((tok * dim + lcol) * 2) : kOutOfRange;
      }
    } else {
      tclean[j] = false;
      x_off[j] = tvalid[j] ? static_cast<int>((tok * dim + lcol) * 2) : kOutOfRange;
      e_off[j] = kOutOfRange;
    }
  }

  u32x4 wreg[kLoadW], araw[kLoadA][2];
  auto load_tiles = [&](long k0) {
    const int so = static_cast<int>(k0 * 2);
#pragma unroll
    for (int j = 0; j < kLoadW; ++j)
      wreg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, w_off[j], so, 0));
#pragma unroll
    for (int j = 0; j < kLoadA; ++j) {
      if constexpr (SRC == kSrcF32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + ftok[j] * dim + k0 + lcol);
        araw[j][0] = __builtin_bit_cast(u32x4, p[0]);
        araw[j][1] = __builtin_bit_cast(u32x4, p[1]);
      } else if constexpr (BIG) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(xp[j] + k0);
        const u32x4 e = *reinterpret_cast<const u32x4*>(ep[j] + k0);
        araw[j][0] = tclean[j] ? c : u32x4{0u, 0u, 0u, 0u};
        araw[j][1] = tvalid[j] ? e : u32x4{0u, 0u, 0u, 0u};
      } else {
        araw[j][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, x_off[j], so, 0));
        araw[j][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ers, e_off[j], so, 0));
      }
    }
  };
  auto a_chunk = [&](int j) -> u32x4 {
    if constexpr (SRC == kSrcRecover) {
      return recover8(araw[j][0], araw[j][1], 1.0f - a.sigma, a.sigma);
    } else {
      const f32x4 lo = __builtin_bit_cast(f32x4, araw[j][0]), hi = __builtin_bit_cast(f32x4, araw[j][1]);
      const u32x4 v{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                    pack_bf16x2(hi[2], hi[3])};
      return tvalid[j] ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kLoadW; ++j)
      *reinterpret_cast<u32x4*>(&ws[buf][(lrow + kLoadRows * j) * kGemmLD + lcol]) = wreg[j];
#pragma unroll
    for (int j = 0; j < kLoadA; ++j)
      *reinterpret_cast<u32x4*>(&as[buf][(lrow + kLoadRows * j) * kGemmLD + lcol]) = a_chunk(j);
  };

  const int wc = wave / kGemmWavesT;  // feature slice of the block
  const int wt = wave % kGemmWavesT;  // token half of the block
  f32x16 acc[kWaveBF][kWaveBT];
#pragma unroll
  for (int i = 0; i < kWaveBF; ++i)
#pragma unroll
    for (int j = 0; j < kWaveBT; ++j) acc[i][j] = f32x16{};

  const long n_k = dim / kGemmBK;
  load_tiles(0);
  store_tiles(0);
  if (n_k > 1) load_tiles(kGemmBK);
  __syncthreads();

  const int l32 = lane & 31;
  const int khalf = (lane >> 5) * 8;
  for (long ks = 0; ks < n_k; ++ks) {
    const int buf = static_cast<int>(ks & 1);
#pragma unroll
    for (int kk16 = 0; kk16 < kGemmBK / 16; ++kk16) {
      const int kk = kk16 * 16 + khalf;
      bf16x8 fw[kWaveBF], ft[kWaveBT];
#pragma unroll
      for (int i = 0; i < kWaveBF; ++i)
        fw[i] = *reinterpret_cast<const bf16x8*>(&ws[buf][((wc * kWaveBF + i) * 32 + l32) * kGemmLD + kk]);
#pragma unroll
      for (int j = 0; j < kWaveBT; ++j)
        ft[j] = *reinterpret_cast<const bf16x8*>(&as[buf][((wt * kWaveBT + j) * 32 + l32) * kGemmLD + kk]);
#pragma unroll
      for (int i = 0; i < kWaveBF; ++i)
#pragma unroll
        for (int j = 0; j < kWaveBT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], ft[j], acc[i][j], 0, 0, 0);
    }
    // Stage K slice ks+1 into the other buffer (last read in step ks-1, before the
    // previous barrier), publish it, then fetch slice ks+2.
    if (ks + 1 < n_k) store_tiles(buf ^ 1);
    __syncthreads();
    if (ks + 2 < n_k) load_tiles((ks + 2) * kGemmBK);
  }

  store_tile<TL>(a, acc, c_base, t_base, wc, wt, lane);
}

// One 16-byte piece per lane from a range-checked buffer straight into LDS: lane i
// writes bytes 16i .. 16i+15 after `lds` (wave-uniform), no registers involved.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rs, uint16_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
// The same copy from a 64-bit address per lane (rows past one buffer range).  (A
// helper of its own: written straight into a kernel template's lambda, the builtin
// keeps the host compiler from emitting that kernel's launch stub.)
__device__ __forceinline__ void lds_copy16_global(const uint16_t* src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
// Wait until every copy this wave issued has landed in LDS (vmcnt 0).
__device__ __forceinline__ void lds_copy_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// bf16 token rows, which need no conversion: the operand tiles go from HBM to LDS
// without passing through registers.  LDS rows are unpadded (64 elements, 128 bytes);
// 16-byte chunk c of row r sits at chunk c ^ ((r / 2) % 8), so the 16 rows that one
// quarter-wave of a ds_read_b128 touches (one chunk column) fall on 16 distinct
// 16-byte bank groups.  One copy instruction moves 8 rows (1 KB) of a tile; each K step
// is copied into the buffer not being multiplied while the other one is, and every
// buffer is an LDS array of its own, so the only waits for the copies are at the
// barrier that ends the step.
template <typename TL, bool BIG = false>
__global__ __launch_bounds__(TL::kThreads, TL::kMinBlocks) void qkv_gemm_lds_kernel(GemmArgs a) {
  constexpr int kGemmBM = TL::kBM, kGemmBN = TL::kBN, kGemmWavesT = TL::kWavesT;
  constexpr int kWaveBF = TL::kBF, kWaveBT = TL::kBT;
  constexpr int kWaves = TL::kThreads / 64;
  constexpr int kCopyW = kGemmBM / 8 / kWaves, kCopyA = kGemmBN / 8 / kWaves;  // copies per wave and step
  static_assert(kCopyW * 8 * kWaves == kGemmBM && kCopyA * 8 * kWaves == kGemmBN, "8-row copies per wave");
  __shared__ __align__(16) uint16_t ws0[kGemmBM * kGemmBK], ws1[kGemmBM * kGemmBK];
  __shared__ __align__(16) uint16_t as0[kGemmBN * kGemmBK], as1[kGemmBN * kGemmBK];

  long c_base, t_base;
  tile_origin<TL>(a, c_base, t_base);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // LDS destinations in scalars
  const long c_end = a.col0 + a.ncols;
  const long dim = a.dim;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w), 0, static_cast<int>(3 * dim * dim * 2), kBufferRsrcFlags);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.x), 0, static_cast<int>(BIG ? kMaxRangeBytes : a.n_x_rows * dim * 2), kBufferRsrcFlags);
  // Copy j of this wave: lane L fetches the logical chunk stored at physical chunk L % 8
  // of tile row 8 * (wave * per + j) + L / 8; rows past the matrix read zeros (BIG:
  // row 0, whose products are not stored).
  int w_off[kCopyW], a_off[kCopyA];
  const uint16_t* a_ptr[BIG ? kCopyA : 1];
#pragma unroll
  for (int j = 0; j < kCopyW; ++j) {
    const int row = 8 * (wave_s * kCopyW + j) + (lane >> 3);
    const int lc = (lane & 7) ^ ((row >> 1) & 7);
    const long c = c_base + row;
    w_off[j] = c < c_end ? static_cast<int>((c * dim + lc * 8) * 2) : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < kCopyA; ++j) {
    const int row = 8 * (wave_s * kCopyA + j) + (lane >> 3);
    const int lc = (lane & 7) ^ ((row >> 1) & 7);
    const long r = t_base + row;
    const long tok = r < a.n ? (a.rows ? static_cast<long>(a.rows[r]) : r) : 0;
    if constexpr (BIG) {
      a_ptr[j] = static_cast<const uint16_t*>(a.x) + tok * dim + lc * 8;
      a_off[j] = 0;
    } else {
      a_off[j] = r < a.n ? static_cast<int>((tok * dim + lc * 8) * 2) : kOutOfRange;
    }
  }
  auto copy_step = [&](uint16_t* wbuf, uint16_t* abuf, long k0) {
    const int so = static_cast<int>(k0 * 2);
#pragma unroll
    for (int j = 0; j < kCopyW; ++j) lds_copy16(wrs, wbuf + (wave_s * kCopyW + j) * 8 * kGemmBK, w_off[j], so);
#pragma unroll
    for (int j = 0; j < kCopyA; ++j) {
      uint16_t* dst = abuf + (wave_s * kCopyA + j) * 8 * kGemmBK;
      if constexpr (BIG)
        lds_copy16_global(a_ptr[j] + k0, dst);
      else
        lds_copy16(xrs, dst, a_off[j], so);
    }
  };

  const int wc = wave / kGemmWavesT;  // feature slice of the block
  const int wt = wave % kGemmWavesT;  // token slice of the block
  f32x16 acc[kWaveBF][kWaveBT];
#pragma unroll
  for (int i = 0; i < kWaveBF; ++i)
#pragma unroll
    for (int j = 0; j < kWaveBT; ++j) acc[i][j] = f32x16{};

  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int swz = (l32 >> 1) & 7;  // rows of an MFMA block start at multiples of 32
  auto multiply = [&](const uint16_t* wb, const uint16_t* ab) {
#pragma unroll
    for (int kk16 = 0; kk16 < kGemmBK / 16; ++kk16) {
      const int pc = ((2 * kk16 + hi) ^ swz) * 8;  // physical chunk of logical chunk 2*kk16 + hi
      bf16x8 fw[kWaveBF], ft[kWaveBT];
#pragma unroll
      for (int i = 0; i < kWaveBF; ++i)
        fw[i] = *reinterpret_cast<const bf16x8*>(&wb[((wc * kWaveBF + i) * 32 + l32) * kGemmBK + pc]);
#pragma unroll
      for (int j = 0; j < kWaveBT; ++j)
        ft[j] = *reinterpret_cast<const bf16x8*>(&ab[((wt * kWaveBT + j) * 32 + l32) * kGemmBK + pc]);
#pragma unroll
      for (int i = 0; i < kWaveBF; ++i)
#pragma unroll
        for (int j = 0; j < kWaveBT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], ft[j], acc[i][j], 0, 0, 0);
    }
  };

  const long n_k = dim / kGemmBK;
  copy_step(ws0, as0, 0);
  lds_copy_wait();
  __syncthreads();
  long ks = 0;
  for (; ks + 2 <= n_k; ks += 2) {
    copy_step(ws1, as1, (ks + 1) * kGemmBK);
    __builtin_amdgcn_sched_barrier(0);  // the copies go out before the MFMAs
    multiply(ws0, as0);
    lds_copy_wait();
    __syncthreads();
    if (ks + 2 < n_k) copy_step(ws0, as0, (ks + 2) * kGemmBK);
    __builtin_amdgcn_sched_barrier(0);
    multiply(ws1, as1);
    lds_copy_wait();
    __syncthreads();
  }
  if (ks < n_k) multiply(ws0, as0);  // odd step count: the last step was copied into buffer 0

  store_tile<TL>(a, acc, c_base, t_base, wc, wt, lane);
}

template <typename TL>
void launch_tile(const GemmArgs& a, const RowSource& src, long n, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.ncols + TL::kBM - 1) / TL::kBM * ((n + TL::kBN - 1) / TL::kBN)));
  // bf16 token rows (and noise rows) beyond one buffer range
  const bool big = src.n_x_rows * a.dim * 2 > kMaxRangeBytes;
  if (src.eps && big) {
    hipLaunchKernelGGL((qkv_gemm_kernel<kSrcRecover, TL, true>), grid, dim3(TL::kThreads), 0, s, a);
  } else if (src.eps) {
    hipLaunchKernelGGL((qkv_gemm_kernel<kSrcRecover, TL>), grid, dim3(TL::kThreads), 0, s, a);
  } else if (src.x_dtype == kDtypeF32) {
    hipLaunchKernelGGL((qkv_gemm_kernel<kSrcF32, TL>), grid, dim3(TL::kThreads), 0, s, a);
  } else if (big) {
    hipLaunchKernelGGL((qkv_gemm_lds_kernel<TL, true>), grid, dim3(TL::kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((qkv_gemm_lds_kernel<TL>), grid, dim3(TL::kThreads), 0, s, a);
  }
}

hipError_t launch_qkv(const RowSource& src, long n, long dim, const uint16_t* w_qkv,
                      const QkvOut& out, const RopeSpec& rope, hipStream_t s) {
  GemmArgs a;
  a.x = src.x;
  a.n_x_rows = src.n_x_rows;
  a.rows = src.rows;
  a.out_rows = out.rows ? out.rows : src.rows;
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
  a.rope_d = 0;
  if (rope.heads > 0) {
    a.rope_d = static_cast<int>(dim / rope.heads);
    a.rope_ds = 2 * (a.rope_d / 6);
    a.rope_dt = a.rope_d - 2 * a.rope_ds;
    a.rope_hw = rope.height * rope.width;
    a.rope_w = rope.width;
    a.rope_log2_base = rope.log2_base;
  }
  const long tiles_large =
      (a.ncols + TileLarge::kBM - 1) / TileLarge::kBM * ((n + TileLarge::kBN - 1) / TileLarge::kBN);
  if (tiles_large >= kLargeTileMinBlocks)
    launch_tile<TileLarge>(a, src, n, s);
  else
    launch_tile<TileSmall>(a, src, n, s);
  return hipGetLastError();
}

}  // namespace tsa
