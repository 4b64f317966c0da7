// a7: attention of the active queries over the full cached K/V (+ fused a8 scatter).
//
// HSA page §2.2 items 3-4: the active tokens' queries attend to the whole
// per-layer cache -- fresh K/V rows for active tokens, stale but valid rows
// for skipped ones -- so the cost is |A_i| * N instead of N^2.  Full
// bidirectional softmax attention, no mask.
//
// Flash-style single pass with an online softmax, bf16 MFMA, fp32 state.
// A workgroup of 4 waves owns 128 queries of one head; each wave owns 32.
// Key/value tiles of 64 rows are staged row-major through two LDS buffers
// (one barrier per tile); the next tile's global loads are in flight while
// the current one is computed.
//
// Layout trick: the score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16.  In that instruction's accumulator layout a lane
// holds ONE query (lane % 32) and 16 keys, so the running max, the sum and
// the rescale factor of a query all live in one lane (plus its partner lane
// +-32, reached with a single cross-lane exchange per tile).  The output is
// accumulated transposed too, O^T = V^T P^T: the probabilities a lane holds
// are exactly the B operand it must supply, provided the V^T operand uses
// the same key order inside each 16-key chunk -- which the transposing LDS
// reads of row-major V deliver directly.  No probabilities travel through LDS.
#include "common.h"
#include "kernels.h"

namespace tsa {

constexpr int kAttnBM = 128;  // queries per workgroup
constexpr int kAttnBN = 64;   // keys per tile

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  long n_q;
  long n_kv;
  int heads;
  float scale_log2;  // softmax scale * log2(e)
  uint16_t* out;
  const int* out_rows;
  float* lse;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i%4 of the 4-element pieces addressed by lanes i/4, 4+i/4,
// 8+i/4 and 12+i/4.  With lane j of the group pointing at
// V[key0 + j/4][dim0 + 4*(j%4)], lane i ends up with V[key0 + 0..3][dim0 + i]:
// four consecutive keys of one dimension -- a column of V, as the MFMA needs.
// `p` must point into a __shared__ array; the cast is an address-space cast.
__device__ __forceinline__ v4i16 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<uint16_t*>(p));
}

template <int HD>
__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs a) {
  constexpr int BN = kAttnBN;
  // K rows: stride HD+8 elements (16-byte reads down a column hit distinct banks).
  // V rows: stride HD+32 elements = 64 mod 256 bytes, so the four rows touched by
  // a 32-lane half of a transposing read land on disjoint banks.
  constexpr int LDK = HD + 8;
  constexpr int LDV = HD + 32;
  constexpr int NM = HD / 16;          // MFMA steps over the head dim
  constexpr int NDB = HD / 32;         // 32-wide output dim blocks
  constexpr int CPR = HD / 8;          // 16-byte chunks per K/V row
  constexpr int NCH = BN * CPR / 256;  // chunks per thread per tile (K and V each)

  __shared__ __align__(16) uint16_t ks[2][BN * LDK];
  __shared__ __align__(16) uint16_t vs[2][BN * LDV];

  const long n_qt = (a.n_q + kAttnBM - 1) / kAttnBM;
  const long tile = xcd_remap(blockIdx.x, n_qt * a.heads);
  const int head = static_cast<int>(tile / n_qt);
  const long qt = tile - static_cast<long>(head) * n_qt;

  const long D = static_cast<long>(a.heads) * HD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const long qrow = qt * kAttnBM + wave * 32 + l32;
  const bool qvalid = qrow < a.n_q;
  bf16x8 qf[NM];
  {
    const uint16_t* qp = a.q + (qvalid ? qrow : 0) * D + head * HD + 8 * hi;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      u32x4 t = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * m) : u32x4{0u, 0u, 0u, 0u};
      qf[m] = __builtin_bit_cast(bf16x8, t);
    }
  }

  const uint16_t* kbase = a.k + head * HD;
  const uint16_t* vbase = a.v + head * HD;

  u32x4 kreg[NCH], vreg[NCH];
  auto load = [&](long kv0) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int id = tid + 256 * j;
      const long key = kv0 + id / CPR;
      const long off = key * D + (id % CPR) * 8;
      const bool ok = key < a.n_kv;
      kreg[j] = ok ? *reinterpret_cast<const u32x4*>(kbase + off) : u32x4{0u, 0u, 0u, 0u};
      vreg[j] = ok ? *reinterpret_cast<const u32x4*>(vbase + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int id = tid + 256 * j;
      *reinterpret_cast<u32x4*>(&ks[buf][(id / CPR) * LDK + (id % CPR) * 8]) = kreg[j];
      *reinterpret_cast<u32x4*>(&vs[buf][(id / CPR) * LDV + (id % CPR) * 8]) = vreg[j];
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = a.scale_log2;

  // Per-lane offsets of the transposing V reads: group g = lane/16 covers
  // keys 4*(g/2) + 0..3 (+8 for the second read) and dims 16*(g%2) + 0..15.
  const int grp = lane >> 4, gl = lane & 15;
  const int v_off = (4 * (grp >> 1) + (gl >> 2)) * LDV + 16 * (grp & 1) + 4 * (gl & 3);

  load(0);
  store(0);
  if (BN < a.n_kv) load(BN);
  __syncthreads();

  const long n_tiles = (a.n_kv + BN - 1) / BN;
  for (long t = 0; t < n_tiles; ++t) {
    const int buf = static_cast<int>(t & 1);
    const long kv0 = t * BN;
    const uint16_t* kt = ks[buf];
    const uint16_t* vt = vs[buf];

    // S^T block kb: keys 32*kb + 8*(r/4) + 4*hi + r%4 (r = 0..15), query l32.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&kt[(kb * 32 + l32) * LDK + 16 * m + 8 * hi]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m], s[kb], 0, 0, 0);
      }
    }
    if (kv0 + BN > a.n_kv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const long key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= a.n_kv) s[kb][r] = -__builtin_inff();
        }
    }

    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);

    // Probabilities, packed as the B operand of the four 16-key PV chunks:
    // chunk ch = 2*kb + r/8, slot 8*hi + 4*((r/4)%2) + r%4 <-> key 16*ch + 8*((r/4)%2) + 4*hi + r%4.
    bf16x8 pf[4];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_new));
        psum += p;
        pf[2 * kb + (r >> 3)][r & 7] = static_cast<__bf16>(p);
      }
    l_run = fmaf(l_run, alpha, psum);
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    m_run = m_new;

    // O^T[dim, query] += V^T[dim, key] P^T[key, query], 16 keys per MFMA; the
    // A operand (V^T) comes from two transposing reads of row-major V.
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vp = vt + 16 * ch * LDV + 32 * db + v_off;
        const v4i16 lo = ds_read_tr16(vp);
        const v4i16 hi4 = ds_read_tr16(vp + 8 * LDV);
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ch], acc[db], 0, 0, 0);
      }
    }

    // Stage tile t+1 (already in registers) into the other buffer, then fetch t+2.
    // The other buffer was last read during tile t-1, before the previous barrier.
    if (t + 1 < n_tiles) store(buf ^ 1);
    __syncthreads();
    if (t + 2 < n_tiles) load(kv0 + 2 * BN);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    const long orow = a.out_rows ? static_cast<long>(a.out_rows[qrow]) : qrow;
    uint16_t* op = a.out + orow * D + head * HD + 4 * hi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 val{pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                        pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + db * 32 + g * 8) = val;
      }
    if (a.lse && hi == 0) a.lse[head * a.n_q + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, long n_q,
                            long n_kv, int heads, int head_dim, float scale, uint16_t* out,
                            const int* out_rows, float* lse, hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.heads = heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.out_rows = out_rows;
  a.lse = lse;
  const long n_qt = (n_q + kAttnBM - 1) / kAttnBM;
  const dim3 grid(static_cast<unsigned>(n_qt * heads));
  if (head_dim == 128) {
    hipLaunchKernelGGL(attention_kernel<128>, grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attention_kernel<64>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tsa
