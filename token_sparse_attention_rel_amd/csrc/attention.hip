// a7: attention of the active queries over the full cached K/V (+ fused a8 scatter).
//
// HSA page §2.2 items 3-4: the active tokens' queries attend to the whole
// per-layer cache -- fresh K/V rows for active tokens, stale but valid rows
// for skipped ones -- so the cost is |A_i| * N instead of N^2.  Full
// bidirectional softmax attention, no mask.
//
// Flash-style single pass with an online softmax, bf16 MFMA, fp32 state.
// A workgroup of 8 waves (4 for head_dim 64) owns 32 queries per wave of one
// head.
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tsa {

constexpr int kAttnBN = 32;  // keys per tile

// Waves per workgroup (32 queries each): 8 for head_dim 128, so every thread
// stages one 16-byte chunk of K and of V per tile and one K/V tile in LDS feeds
// 256 queries; 4 for head_dim 64 (a 32 x 64 tile has 256 chunks).
template <int HD>
constexpr int attn_waves() { return HD == 128 ? 8 : 4; }

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

// Softmax rescale policy: the running max used for the exponent, m, is only
// moved when a new score exceeds it by more than kLazyMax (log2 units), so
// probabilities stay <= 2**kLazyMax and the O rescale is almost never needed.
// Any consistent shift gives the same normalised output.
constexpr float kLazyMax = 8.0f;

// Word 3 of a raw buffer resource on gfx9-class GPUs (32-bit elements, no swizzle);
// out-of-range offsets then read as zero.
constexpr int kBufferRsrcFlags = 0x00020000;

template <bool B>
using Flag = std::integral_constant<bool, B>;

template <int HD>
__global__ __launch_bounds__(64 * attn_waves<HD>(), 2) void attention_kernel(AttnArgs a) {
  constexpr int BN = kAttnBN;
  constexpr int NT = 64 * attn_waves<HD>();  // threads
  constexpr int BM = 32 * attn_waves<HD>();  // queries per workgroup
  // K rows: stride HD+8 elements (16-byte reads down a column hit distinct banks).
  // V rows: stride HD+32 elements = 64 mod 256 bytes, so the four rows touched by
  // a 32-lane half of a transposing read land on disjoint banks.
  constexpr int LDK = HD + 8;
  constexpr int LDV = HD + 32;
  constexpr int NM = HD / 16;          // MFMA steps over the head dim
  constexpr int NDB = HD / 32;         // 32-wide output dim blocks
  constexpr int CPR = HD / 8;          // 16-byte chunks per K/V row
  constexpr int NCH = BN * CPR / NT;   // chunks per thread per tile (K and V each)
  static_assert(NCH >= 1, "tile too small for the workgroup");

  __shared__ __align__(16) uint16_t ks[2][BN * LDK];
  __shared__ __align__(16) uint16_t vs[2][BN * LDV];

  const long n_qt = (a.n_q + BM - 1) / BM;
  const long tile = xcd_remap(blockIdx.x, n_qt * a.heads);
  const int head = static_cast<int>(tile / n_qt);
  const long qt = tile - static_cast<long>(head) * n_qt;

  const long D = static_cast<long>(a.heads) * HD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const long qrow = qt * BM + wave * 32 + l32;
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

  // K/V tiles are fetched with range-checked buffer loads: rows past the end
  // of the cache read as zeros, so prefetches beyond the last tile need no branch.
  const long n_kv = a.n_kv;
  const int kv_bytes = static_cast<int>(((n_kv - 1) * D + HD) * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.k + head * HD), 0, kv_bytes, kBufferRsrcFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.v + head * HD), 0, kv_bytes, kBufferRsrcFlags);
  // Loader: chunk id = tid + NT*j covers row id / CPR, 16-byte column id % CPR.
  int g_off[NCH];
  uint32_t k_lds[NCH], v_lds[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int id = tid + NT * j;
    g_off[j] = static_cast<int>(((id / CPR) * D + (id % CPR) * 8) * 2);
    k_lds[j] = (id / CPR) * LDK + (id % CPR) * 8;
    v_lds[j] = (id / CPR) * LDV + (id % CPR) * 8;
  }
  auto gload = [&](u32x4* r, __amdgpu_buffer_rsrc_t rs, long kv0) {
    const long boff = kv0 * D * 2;
    const int so = boff < kv_bytes ? static_cast<int>(boff) : kv_bytes;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, g_off[j], so, 0));
  };
  auto sstore = [&](uint16_t* buf, const uint32_t* off, const u32x4* r) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) *reinterpret_cast<u32x4*>(buf + off[j]) = r[j];
  };

  // S^T block (32 keys x 32 queries): keys 8*(r/4) + 4*hi + r%4 (r = 0..15), query l32.
  auto qk = [&](const uint16_t* kt) {
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8*>(&kt[l32 * LDK + 8 * hi]), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int m = 1; m < NM; ++m)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(&kt[l32 * LDK + 16 * m + 8 * hi]), qf[m], s, 0, 0, 0);
    return s;
  };
  auto mask_tail = [&](f32x16& s, long kv0) {
    if (kv0 + BN > n_kv) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kv0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= n_kv) s[r] = -__builtin_inff();
    }
  };

  // Transposing V reads: group g = lane/16 covers keys 4*(g/2) + 0..3 (+8 for the
  // second read) and dims 16*(g%2) + 0..15 of each 32-wide dim block.
  const int grp = lane >> 4, gl = lane & 15;
  const int v_off = (4 * (grp >> 1) + (gl >> 2)) * LDV + 16 * (grp & 1) + 4 * (gl & 3);
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  // O^T[dim, query] += V^T[dim, key] P^T[key, query] over one 32-key tile (two 16-key chunks).
  auto pv = [&](const uint16_t* vt, const bf16x8* pf) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vp = vt + 16 * ch * LDV + 32 * db + v_off;
        const v4i16 lo = ds_read_tr16(vp);
        const v4i16 hi4 = ds_read_tr16(vp + 8 * LDV);
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ch], acc[db], 0, 0, 0);
      }
  };

  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = a.scale_log2;
  const long n_t = (n_kv + BN - 1) / BN;

  // Prologue: K tiles 0 and 1 in LDS, S of tile 0; registers hold K(2) and V(0).
  u32x4 kr[NCH], vr[NCH];
  gload(kr, krs, 0);
  sstore(ks[0], k_lds, kr);
  gload(kr, krs, BN);
  sstore(ks[1], k_lds, kr);
  __syncthreads();
  gload(kr, krs, 2 * BN);
  gload(vr, vrs, 0);
  f32x16 s_cur = qk(ks[0]);
  mask_tail(s_cur, 0);
  __syncthreads();  // every wave is done with K(0) before K(2) overwrites it

  bf16x8 p_prev[2];
  // Iteration t: MFMA work PV(t-1) and QK(t+1) interleaved with the softmax of
  // tile t on the VALU; then stage V(t) and K(t+2) and fetch V(t+1) and K(t+3).
  // A buffer is rewritten only after the barrier that follows its last read.
  auto iteration = [&](long t, auto has_prev, auto has_next, auto may_mask) {
    const int b = static_cast<int>(t & 1);
    f32x16 s_next;
    if constexpr (decltype(has_prev)::value) pv(vs[b ^ 1], p_prev);
    if constexpr (decltype(has_next)::value) s_next = qk(ks[b ^ 1]);

    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float cand = mx * c;
    const bool upd = cand > m_run + kLazyMax;
    const float m_new = upd ? cand : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    bf16x8 pf[2];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s_cur[r], c, -m_new));
      psum += p;
      pf[r >> 3][r & 7] = static_cast<__bf16>(p);
    }
    l_run = fmaf(l_run, alpha, psum);
    {
      // Keep the softmax in this block: its results are consumed only in the next
      // iteration, and left alone the compiler sinks it past the barrier, where it
      // can no longer overlap the MFMAs above.  (An empty asm that reads them.)
      const u32x4 p0 = __builtin_bit_cast(u32x4, pf[0]), p1 = __builtin_bit_cast(u32x4, pf[1]);
      asm volatile("" ::"v"(p0[0]), "v"(p0[1]), "v"(p0[2]), "v"(p0[3]), "v"(p1[0]), "v"(p1[1]),
                   "v"(p1[2]), "v"(p1[3]), "v"(l_run), "v"(alpha));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(may_mask)::value) mask_tail(s_next, (t + 1) * BN);

    sstore(vs[b], v_lds, vr);
    sstore(ks[b], k_lds, kr);
    __syncthreads();
    gload(vr, vrs, (t + 1) * BN);
    gload(kr, krs, (t + 3) * BN);
    if constexpr (decltype(has_next)::value) s_cur = s_next;
    p_prev[0] = pf[0];
    p_prev[1] = pf[1];
    // O now holds tiles < t (PV(t-1) was issued above) at the old max: bring it
    // to the new one before PV(t) is added in the next iteration.
    if (__ballot(upd)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
  };

  if (n_t == 1) {
    iteration(0, Flag<false>{}, Flag<false>{}, Flag<false>{});
  } else {
    iteration(0, Flag<false>{}, Flag<true>{}, Flag<true>{});
    for (long t = 1; t + 2 < n_t; ++t) iteration(t, Flag<true>{}, Flag<true>{}, Flag<false>{});
    if (n_t > 2) iteration(n_t - 2, Flag<true>{}, Flag<true>{}, Flag<true>{});
    iteration(n_t - 1, Flag<true>{}, Flag<false>{}, Flag<false>{});
  }
  pv(vs[(n_t - 1) & 1], p_prev);

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
  if (head_dim == 128) {
    constexpr int bm = 32 * attn_waves<128>();
    const dim3 grid(static_cast<unsigned>((n_q + bm - 1) / bm * heads));
    hipLaunchKernelGGL(attention_kernel<128>, grid, dim3(64 * attn_waves<128>()), 0, s, a);
  } else {
    constexpr int bm = 32 * attn_waves<64>();
    const dim3 grid(static_cast<unsigned>((n_q + bm - 1) / bm * heads));
    hipLaunchKernelGGL(attention_kernel<64>, grid, dim3(64 * attn_waves<64>()), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tsa
