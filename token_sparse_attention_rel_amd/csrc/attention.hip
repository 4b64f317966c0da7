// a7: attention of the active queries over the full cached K/V (+ fused a8 scatter).
//
// HSA page §2.2 items 3-4: the active tokens' queries attend to the whole
// per-layer cache -- fresh K/V rows for active tokens, stale but valid rows
// for skipped ones -- so the cost is |A_i| * N instead of N^2.  Full
// bidirectional softmax attention, no mask.
//
// Flash-style single pass with an online softmax, bf16 MFMA, fp32 state.
// A workgroup of 4 waves owns 128 queries of one head; each wave owns 32.
// Key/value tiles of 64 rows are staged through LDS (K row-major, V
// transposed) and double-buffered through registers.
//
// Layout trick: the score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16.  In that instruction's accumulator layout a lane
// holds ONE query (lane % 32) and 16 keys, so the running max, the sum and
// the rescale factor of a query all live in one lane (plus its partner lane
// +-32, reached with a single cross-lane exchange per tile).  The output is
// accumulated transposed too, O^T = V^T P^T: the probabilities a lane holds
// are exactly the B operand it must supply, provided the key order inside
// each 16-key chunk is permuted consistently -- which the transposed V
// store into LDS does (bits 2 and 3 of the key offset swapped).  No
// probabilities travel through LDS.
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

// Key offset within a 16-key chunk -> LDS position (swap bits 2 and 3).
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Element e (0..7) of two 8 x bf16 vectors, packed as (a_e, b_e).
__device__ __forceinline__ uint32_t pair16(const u32x4 a, const u32x4 b, int e) {
  const uint32_t wa = a[e >> 1], wb = b[e >> 1];
  return (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

template <int HD>
__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs a) {
  constexpr int BN = kAttnBN;
  constexpr int LDK = HD + 8;               // K row stride in LDS (elements)
  constexpr int LDV = BN + 8;               // V^T row stride in LDS (elements)
  constexpr int NM = HD / 16;               // MFMA steps over the head dim
  constexpr int NDB = HD / 32;              // 32-wide output dim blocks
  constexpr int CPR = HD / 8;               // 16-byte chunks per K/V row
  constexpr int KCH = BN * CPR / 256;       // K chunks per thread
  constexpr int KPT = BN * HD / 8 / 256;    // V keys per thread (8 dims each)
  static_assert(KPT == 2 || KPT == 4, "unsupported head dim");

  __shared__ __align__(16) uint16_t ks[BN * LDK];
  __shared__ __align__(16) uint16_t vt[HD * LDV];

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
  const int vkg = tid / CPR;  // V key group (KPT keys)
  const int vdg = tid % CPR;  // V dim group (8 dims)

  u32x4 kreg[KCH], vreg[KPT];
  auto load = [&](long kv0) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int id = tid + 256 * j;
      const long key = kv0 + id / CPR;
      kreg[j] = key < a.n_kv
                    ? *reinterpret_cast<const u32x4*>(kbase + key * D + (id % CPR) * 8)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const long key = kv0 + vkg * KPT + j;
      vreg[j] = key < a.n_kv ? *reinterpret_cast<const u32x4*>(vbase + key * D + vdg * 8)
                             : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int id = tid + 256 * j;
      *reinterpret_cast<u32x4*>(&ks[(id / CPR) * LDK + (id % CPR) * 8]) = kreg[j];
    }
    const int pos = vt_pos(vkg * KPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* dst = &vt[(vdg * 8 + e) * LDV + pos];
      if (KPT == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{pair16(vreg[0], vreg[1], e), pair16(vreg[2], vreg[3], e)};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = pair16(vreg[0], vreg[1], e);
      }
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

  load(0);
  store();
  __syncthreads();

  for (long kv0 = 0; kv0 < a.n_kv; kv0 += BN) {
    const bool more = kv0 + BN < a.n_kv;
    if (more) load(kv0 + BN);

    // S^T block kb: keys 32*kb + 8*(r/4) + 4*hi + r%4 (r = 0..15), query l32.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks[(kb * 32 + l32) * LDK + 16 * m + 8 * hi]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m], s[kb], 0, 0, 0);
      }
    }
    if (!more && kv0 + BN > a.n_kv) {
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

    // Probabilities, packed as the B operand of the four 16-key PV chunks.
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

    // O^T[dim, query] += V^T[dim, key] P^T[key, query], 16 keys per MFMA.
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vt[(db * 32 + l32) * LDV + 16 * ch + 8 * hi]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ch], acc[db], 0, 0, 0);
      }
    }

    __syncthreads();
    if (more) {
      store();
      __syncthreads();
    }
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
