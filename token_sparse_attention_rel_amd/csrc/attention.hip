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
// Key/value tiles of 32 rows are staged row-major through rings of four LDS
// slots, two tiles per barrier; the next pair's global loads are in flight
// while the current pair is computed.  They arrive through range-checked buffer
// loads with 32-bit offsets: a K or V cache of 2 GiB or more takes kernels
// that place the buffer range at each tile's first row.
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
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tsa {

constexpr int kAttnBN = 32;  // keys per tile
constexpr int kMaxDevices = 64;
// Split schedule limits: at most kMaxPieces pieces per tile, each at least
// kMinPieceTiles key tiles long, and at most kMaxPieceSlots pieces per resident
// workgroup in total (this bounds the workspace).
constexpr int kMaxPieces = 64;
constexpr int kMinPieceTiles = 4;
constexpr int kMaxPieceSlots = 6;

// Waves per workgroup and 32-query blocks per wave.  head_dim 128: 8 waves of
// 32 queries, two per SIMD, so that one wave's softmax runs while the other's
// MFMAs do; every thread then stages one 16-byte chunk of K and of V per tile.
// (Four waves of two blocks each -- one wave per SIMD with up to 512 VGPRs, each
// K/V fragment feeding two MFMAs -- measured about 9% slower on MI355X: a lone
// wave cannot hide its own LDS and MFMA latencies.)  head_dim 64: 4 waves of 32
// queries (a 32 x 64 tile has 256 16-byte chunks).  A workgroup covers 256
// (128) queries of one head.
template <int HD>
constexpr int attn_waves() { return HD == 128 ? 8 : 4; }
template <int HD>
constexpr int attn_qblocks() { return 1; }
template <int HD>
constexpr int attn_blocks() { return attn_waves<HD>() * attn_qblocks<HD>(); }
template <int HD>
constexpr int attn_rows() { return 32 * attn_blocks<HD>(); }
// Resident workgroups per CU the register budget is sized for.
template <int HD>
constexpr int attn_min_blocks() { return 2; }

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
  // frame-causal variant: query r is token q_tokens[r] and sees the keys of the frames up
  // to its own, j < (q_tokens[r] / frame_tokens + 1) * frame_tokens
  const int* q_tokens;
  long frame_tokens;
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
// Largest byte range one buffer resource describes here (its offsets are 32-bit).
constexpr long kMaxRangeBytes = 0x7FFFFFFF;

template <bool B>
using Flag = std::integral_constant<bool, B>;

// Partial result of one segment, laid out as the registers hold it (lane fastest):
// O^T accumulators [block][NDB*16][64], then the shift m and the sum l [block][64],
// block = wave * (blocks per wave) + block of the wave.
template <int HD>
constexpr long attn_piece_floats() { return attn_blocks<HD>() * 64L * (HD / 32 * 16 + 2); }

// Keys [t0*BN, t1*BN) of query tile `tile` (head-major numbering).  part == nullptr:
// normalise and write the bf16 output rows (+ LSE); otherwise write the partial
// (unnormalised O, shift, sum) to `part` for a later merge.  ks / vs are the
// four-slot LDS rings of K and V tiles (tile t in slot (t - t0) mod 4).
template <int HD, bool CAUSAL = false, bool BIG = false>
__device__ __forceinline__ void attend_segment(const AttnArgs& a, uint16_t* ks_base, uint16_t* vs_base,
                                               long tile, long t0, long t1, float* part) {
  constexpr int BN = kAttnBN;
  constexpr int NW = attn_waves<HD>();
  constexpr int QB = attn_qblocks<HD>();
  constexpr int NT = 64 * NW;             // threads
  constexpr int BM = attn_rows<HD>();     // queries per workgroup
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

  // Slot i of each ring; plain offsets from the LDS base keep every access an LDS one.
  auto ks = [&](int i) { return ks_base + i * (BN * LDK); };
  auto vs = [&](int i) { return vs_base + i * (BN * LDV); };

  const long n_qt = (a.n_q + BM - 1) / BM;
  const int head = static_cast<int>(tile / n_qt);
  const long qt = tile - static_cast<long>(head) * n_qt;

  const long D = static_cast<long>(a.heads) * HD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Block qb of this wave holds queries qrow0 + 32 * qb.
  const long qrow0 = qt * BM + wave * 32 * QB + l32;
  bf16x8 qf[QB][NM];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long qrow = qrow0 + 32 * qb;
    const bool qvalid = qrow < a.n_q;
    const uint16_t* qp = a.q + (qvalid ? qrow : 0) * D + head * HD + 8 * hi;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      u32x4 t = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * m) : u32x4{0u, 0u, 0u, 0u};
      qf[qb][m] = __builtin_bit_cast(bf16x8, t);
    }
  }

  const long n_kv = a.n_kv;
  // Frame-causal limits: lim[qb] = keys visible to this lane's query; the workgroup's
  // smallest and largest limits bound the key range and the tiles that need masking.
  long lim[QB];
  long lim_lo = n_kv;
  if constexpr (CAUSAL) {
    __shared__ long lim_part[2][NW];
    long lo = n_kv, hi_ = 1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const long qrow = qrow0 + 32 * qb;
      lim[qb] = n_kv;
      if (qrow < a.n_q) {
        const long f = static_cast<long>(a.q_tokens[qrow]) / a.frame_tokens;
        lim[qb] = (f + 1) * a.frame_tokens < n_kv ? (f + 1) * a.frame_tokens : n_kv;
        lo = lim[qb] < lo ? lim[qb] : lo;
        hi_ = lim[qb] > hi_ ? lim[qb] : hi_;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const long o_lo = __shfl_xor(lo, off, 64), o_hi = __shfl_xor(hi_, off, 64);
      lo = o_lo < lo ? o_lo : lo;
      hi_ = o_hi > hi_ ? o_hi : hi_;
    }
    if (lane == 0) {
      lim_part[0][wave] = lo;
      lim_part[1][wave] = hi_;
    }
    __syncthreads();
    lo = lim_part[0][0];
    hi_ = lim_part[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      lo = lim_part[0][w] < lo ? lim_part[0][w] : lo;
      hi_ = lim_part[1][w] > hi_ ? lim_part[1][w] : hi_;
    }
    lim_lo = lo;
    const long t_hi = (hi_ + BN - 1) / BN;  // key tiles any query of the workgroup sees
    t1 = t1 < t_hi ? t1 : t_hi;
  }

  // K/V tiles are fetched with range-checked buffer loads: rows past the end
  // of the cache read as zeros, so prefetches beyond the last tile need no branch.
  // A head's K/V below 2 GiB is one buffer range, the tile's first row its offset;
  // a larger cache (BIG) gets a range based at each tile's first row instead.
  struct KvSrc {
    __amdgpu_buffer_rsrc_t rs;
    const uint16_t* base;  // the head's first element
  };
  const long kv_elems = (n_kv - 1) * D + HD;  // from the head's first element to its last
  const int kv_bytes = static_cast<int>(BIG ? kMaxRangeBytes : kv_elems * 2);
  const KvSrc krs{__builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.k + head * HD), 0, kv_bytes,
                                                    kBufferRsrcFlags),
                  a.k + head * HD};
  const KvSrc vrs{__builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v + head * HD), 0, kv_bytes,
                                                    kBufferRsrcFlags),
                  a.v + head * HD};
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
  auto gload = [&](u32x4* r, const KvSrc& src, long kv0) {
    if constexpr (BIG) {
      // bytes from row kv0 to the end of the head's last row; none left: every load reads zero
      const long e0 = kv0 * D;
      const long rem = (kv_elems - e0) * 2;
      const int nrec = rem <= 0 ? 0 : rem > kMaxRangeBytes ? static_cast<int>(kMaxRangeBytes) : static_cast<int>(rem);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(src.base + (rem > 0 ? e0 : 0)), 0, nrec, kBufferRsrcFlags);
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, g_off[j], 0, 0));
    } else {
      const long boff = kv0 * D * 2;
      const int so = boff < kv_bytes ? static_cast<int>(boff) : kv_bytes;
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.rs, g_off[j], so, 0));
    }
  };
  auto sstore = [&](uint16_t* buf, const uint32_t* off, const u32x4* r) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) *reinterpret_cast<u32x4*>(buf + off[j]) = r[j];
  };

  // K operand of step m (dims 16m..16m+15) for S^T = K Q^T.
  auto k_frag = [&](const uint16_t* kt, int m) {
    return *reinterpret_cast<const bf16x8*>(&kt[l32 * LDK + 16 * m + 8 * hi]);
  };
  // S^T blocks (32 keys x 32 queries): keys 8*(r/4) + 4*hi + r%4 (r = 0..15), query l32.
  auto qk = [&](const uint16_t* kt, f32x16* s) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const bf16x8 kf = k_frag(kt, m);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][m], m == 0 ? f32x16{} : s[qb], 0, 0, 0);
    }
  };
  auto mask_tail = [&](f32x16* s, long kv0) {
    if constexpr (CAUSAL) {
      if (kv0 + BN > lim_lo) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kv0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= lim[qb]) s[qb][r] = -__builtin_inff();
      }
    } else if (kv0 + BN > n_kv) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kv0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= n_kv) s[qb][r] = -__builtin_inff();
    }
  };

  // Transposing V reads: group g = lane/16 covers keys 4*(g/2) + 0..3 (+8 for the
  // second read) and dims 16*(g%2) + 0..15 of each 32-wide dim block.
  const int grp = lane >> 4, gl = lane & 15;
  const int v_off = (4 * (grp >> 1) + (gl >> 2)) * LDV + 16 * (grp & 1) + 4 * (gl & 3);
  f32x16 acc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x16{};
  // V^T operand of the MFMA for 16-key chunk ch and 32-wide dim block db of a V tile.
  auto v_frag = [&](const uint16_t* vt, int ch, int db) {
    const uint16_t* vp = vt + 16 * ch * LDV + 32 * db + v_off;
    const v4i16 lo = ds_read_tr16(vp);
    const v4i16 hi4 = ds_read_tr16(vp + 8 * LDV);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.f;
  }
  const float c = a.scale_log2;

  // Prologue: K(t0..t0+2) and V(t0) in LDS, S of tile t0; registers hold the first
  // pair's staging tiles K(t0+3), K(t0+4), V(t0+1), V(t0+2).
  u32x4 kr[2][NCH], vr[2][NCH];
  gload(kr[0], krs, t0 * BN);
  gload(kr[1], krs, (t0 + 1) * BN);
  gload(vr[0], vrs, t0 * BN);
  sstore(ks(0), k_lds, kr[0]);
  sstore(ks(1), k_lds, kr[1]);
  sstore(vs(0), v_lds, vr[0]);
  gload(kr[0], krs, (t0 + 2) * BN);
  sstore(ks(2), k_lds, kr[0]);
  __syncthreads();
  gload(kr[0], krs, (t0 + 3) * BN);
  gload(kr[1], krs, (t0 + 4) * BN);
  gload(vr[0], vrs, (t0 + 1) * BN);
  gload(vr[1], vrs, (t0 + 2) * BN);
  f32x16 s_cur[QB];
  qk(ks(0), s_cur);
  mask_tail(s_cur, t0 * BN);
  __syncthreads();  // every wave is done with K(t0) before K(t0+4) overwrites it

  bf16x8 p_prev[QB][2];
  // Iteration t: the softmax of tile t on the VALU, interleaved with the MFMA work
  // PV(t-1) and QK(t+1).  Staging and the barrier come once per pair of iterations
  // (pair_end below); a slot is rewritten only after the barrier that follows its
  // last read.
  auto iteration = [&](long t, auto has_prev, auto has_next, auto may_mask) {
    const int r4 = static_cast<int>((t - t0) & 3);
    // LDS reads of this iteration's MFMA operands go out first, so that their
    // latency is covered by the softmax.
    const uint16_t* kt = ks((r4 + 1) & 3);  // K(t+1)
    const uint16_t* vt = vs((r4 + 3) & 3);  // V(t-1)
    bf16x8 kf[NM];
    bf16x8 vf[2][NDB];
    if constexpr (decltype(has_next)::value) {
#pragma unroll
      for (int m = 0; m < NM; ++m) kf[m] = k_frag(kt, m);
    }
    if constexpr (decltype(has_prev)::value) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int db = 0; db < NDB; ++db) vf[ch][db] = v_frag(vt, ch, db);
    }

    bf16x8 pf[QB][2];
    bool upd[QB];
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float cand = mx * c;
      upd[qb] = cand > m_run[qb] + kLazyMax;
      const float m_new = upd[qb] ? cand : m_run[qb];
      alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s_cur[qb][r], c, -m_new));
        psum += p;
        pf[qb][r >> 3][r & 7] = static_cast<__bf16>(p);
      }
      l_run[qb] = fmaf(l_run[qb], alpha[qb], psum);
      // Keep the softmax in this block: its results are consumed only in the next
      // iteration, and left alone the compiler sinks it past the barrier, where it
      // can no longer overlap the MFMAs below.  (An empty asm that reads them.)
      const u32x4 p0 = __builtin_bit_cast(u32x4, pf[qb][0]), p1 = __builtin_bit_cast(u32x4, pf[qb][1]);
      asm volatile("" ::"v"(p0[0]), "v"(p0[1]), "v"(p0[2]), "v"(p0[3]), "v"(p1[0]), "v"(p1[1]),
                   "v"(p1[2]), "v"(p1[3]), "v"(l_run[qb]), "v"(alpha[qb]));
    }
    f32x16 s_next[QB];
    if constexpr (decltype(has_prev)::value) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ch][db], p_prev[qb][ch], acc[qb][db], 0, 0, 0);
    }
    if constexpr (decltype(has_next)::value) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s_next[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[m], qf[qb][m], m == 0 ? f32x16{} : s_next[qb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Only the last key tile of the cache can be partial (bidirectional), so only the
    // iterations whose next tile may be it carry the masking code; frame-causal
    // limits can fall in any tile.
    if constexpr (CAUSAL) {
      if constexpr (decltype(has_next)::value) mask_tail(s_next, (t + 1) * BN);
    } else if constexpr (decltype(may_mask)::value) {
      mask_tail(s_next, (t + 1) * BN);
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if constexpr (decltype(has_next)::value) s_cur[qb] = s_next[qb];
      p_prev[qb][0] = pf[qb][0];
      p_prev[qb][1] = pf[qb][1];
      // O now holds tiles < t (PV(t-1) was issued above) at the old max: bring it
      // to the new one before PV(t) is added in the next iteration.
      if (__ballot(upd[qb])) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha[qb];
      }
    }
  };

  // After the second iteration of each pair (t, t+1): stage K(t+3), K(t+4), V(t+1),
  // V(t+2) into the slots last read in the previous pair, one barrier, then fetch the
  // next pair's staging tiles (two iterations of latency to cover).  The next pair
  // reads K(t+3), K(t+4), V(t+1), V(t+2): published by this barrier.
  auto pair_end = [&](long t) {
    const int r4 = static_cast<int>((t - t0) & 3);
    sstore(ks((r4 + 3) & 3), k_lds, kr[0]);
    sstore(ks(r4), k_lds, kr[1]);
    sstore(vs((r4 + 1) & 3), v_lds, vr[0]);
    sstore(vs((r4 + 2) & 3), v_lds, vr[1]);
    __syncthreads();
    gload(kr[0], krs, (t + 5) * BN);
    gload(kr[1], krs, (t + 6) * BN);
    gload(vr[0], vrs, (t + 3) * BN);
    gload(vr[1], vrs, (t + 4) * BN);
  };
  // Iteration flags: the first has no PV, the last no QK; only the one before the
  // last may meet a partial tile (bidirectional).  Iterations t0 + i with i odd end a
  // pair; the last one ends a pair too when i is odd, so that V(t1-1) is staged.
  const long nt = t1 - t0;
  if (nt == 1) {
    iteration(t0, Flag<false>{}, Flag<false>{}, Flag<false>{});
  } else {
    iteration(t0, Flag<false>{}, Flag<true>{}, Flag<true>{});
    long i = 1;
    for (; i + 4 <= nt; i += 2) {  // iterations i and i+1 <= nt-3
      iteration(t0 + i, Flag<true>{}, Flag<true>{}, Flag<false>{});
      pair_end(t0 + i - 1);
      iteration(t0 + i + 1, Flag<true>{}, Flag<true>{}, Flag<false>{});
    }
    // the remaining one to three iterations i .. nt-1
    if (i == nt - 3) {
      iteration(t0 + i, Flag<true>{}, Flag<true>{}, Flag<false>{});
      if (i & 1) pair_end(t0 + i - 1);
      ++i;
    }
    if (i == nt - 2) {
      iteration(t0 + i, Flag<true>{}, Flag<true>{}, Flag<true>{});
      if (i & 1) pair_end(t0 + i - 1);
      ++i;
    }
    iteration(t0 + i, Flag<true>{}, Flag<false>{}, Flag<false>{});
    if (i & 1) pair_end(t0 + i - 1);
  }
  {
    const uint16_t* vt = vs((t1 - 1 - t0) & 3);
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 vfr = v_frag(vt, ch, db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr, p_prev[qb][ch], acc[qb][db], 0, 0, 0);
      }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const int blk = wave * QB + qb;
    if (part) {
      float* pw = part + static_cast<long>(blk) * (NDB * 16 * 64);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) pw[(db * 16 + r) * 64 + lane] = acc[qb][db][r];
      float* ml = part + attn_blocks<HD>() * 64L * NDB * 16;
      ml[blk * 64 + lane] = m_run[qb];
      ml[attn_blocks<HD>() * 64 + blk * 64 + lane] = l_tot;
      continue;
    }
    const long qrow = qrow0 + 32 * qb;
    if (qrow < a.n_q) {
      const float inv = 1.0f / l_tot;
      const long orow = a.out_rows ? static_cast<long>(a.out_rows[qrow]) : qrow;
      uint16_t* op = a.out + orow * D + head * HD + 4 * hi;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 val{pack_bf16x2(acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv),
                          pack_bf16x2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + db * 32 + g * 8) = val;
        }
      if (a.lse && hi == 0) a.lse[head * a.n_q + qrow] = (m_run[qb] + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

template <int HD, bool BIG>
__global__ __launch_bounds__(64 * attn_waves<HD>(), attn_min_blocks<HD>()) void attention_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t ks[4 * kAttnBN * (HD + 8)];
  __shared__ __align__(16) uint16_t vs[4 * kAttnBN * (HD + 32)];
  const long n_qt = (a.n_q + attn_rows<HD>() - 1) / attn_rows<HD>();
  const long tile = xcd_remap(blockIdx.x, n_qt * a.heads);
  attend_segment<HD, false, BIG>(a, ks, vs, tile, 0, (a.n_kv + kAttnBN - 1) / kAttnBN, nullptr);
}

// Frame-causal variant: one workgroup per query tile, over the key tiles its
// queries can see.  Queries usually come in token order, so later query tiles
// see more keys.  Blocks take the tiles latest-first, all heads of one query
// tile before the next: the long tiles start first on every XCD and the short
// ones fill in behind them (a longest-first schedule; with the XCD-contiguous
// order of the bidirectional kernel one XCD got far more work than another).
template <int HD, bool BIG>
__global__ __launch_bounds__(64 * attn_waves<HD>(), attn_min_blocks<HD>()) void attention_causal_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t ks[4 * kAttnBN * (HD + 8)];
  __shared__ __align__(16) uint16_t vs[4 * kAttnBN * (HD + 32)];
  const long n_qt = (a.n_q + attn_rows<HD>() - 1) / attn_rows<HD>();
  const long b = blockIdx.x;
  const long tile = (b % a.heads) * n_qt + (n_qt - 1 - b / a.heads);
  attend_segment<HD, true, BIG>(a, ks, vs, tile, 0, (a.n_kv + kAttnBN - 1) / kAttnBN, nullptr);
}

// Split schedule for the last, partly filled round of query tiles.  With C
// resident workgroups and T tiles, the first R = floor(T / C) * C tiles run
// whole, one workgroup each, as in attention_kernel.  Each of the r = T - R
// remaining tiles is cut into kp key ranges (pieces) run by workgroups of their
// own, which write fp32 partials (unnormalised O, shift, sum) to the workspace;
// attention_merge_kernel combines them.  Pieces are numbered key-range-major
// and dealt to XCDs in contiguous runs, so the workgroups resident on one XCD
// at a time read the same key range of the same head and share its L2.
template <int HD, bool BIG>
__global__ __launch_bounds__(64 * attn_waves<HD>(), attn_min_blocks<HD>()) void attention_split_kernel(AttnArgs a, float* ws,
                                                                                   long full, long tail,
                                                                                   int kp) {
  __shared__ __align__(16) uint16_t ks[4 * kAttnBN * (HD + 8)];
  __shared__ __align__(16) uint16_t vs[4 * kAttnBN * (HD + 32)];
  const long n_t = (a.n_kv + kAttnBN - 1) / kAttnBN;
  const long b = blockIdx.x;
  if (b < full) {
    attend_segment<HD, false, BIG>(a, ks, vs, xcd_remap(b, full), 0, n_t, nullptr);
    return;
  }
  const long p = xcd_remap(b - full, tail * kp);
  const long j = p / tail, i = p - j * tail;
  attend_segment<HD, false, BIG>(a, ks, vs, full + i, j * n_t / kp, (j + 1) * n_t / kp,
                                 ws + (i * kp + j) * attn_piece_floats<HD>());
}

// One workgroup per cut tile: O = sum_j w_j O_j / sum_j w_j l_j with
// w_j = 2^(m_j - max_j m_j); bf16 rows (+ LSE) written as attention_kernel does.
template <int HD>
__global__ __launch_bounds__(64 * attn_blocks<HD>()) void attention_merge_kernel(AttnArgs a, const float* ws,
                                                                                 long full, int kp) {
  constexpr int NDB = HD / 32;
  constexpr int NW = attn_blocks<HD>();  // one wave per 32-query block
  constexpr long piece = attn_piece_floats<HD>();
  const long n_qt = (a.n_q + 32 * NW - 1) / (32 * NW);
  const long tile = full + blockIdx.x;
  const int head = static_cast<int>(tile / n_qt);
  const long qt = tile - static_cast<long>(head) * n_qt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const long qrow = qt * 32 * NW + wave * 32 + l32;
  if (qrow >= a.n_q) return;
  const float* p0 = ws + static_cast<long>(blockIdx.x) * kp * piece;
  const long mo = NW * 64L * NDB * 16;  // offset of the shifts; the sums follow
  const int ml = wave * 64 + lane;
  float m = -__builtin_inff();
  for (int j = 0; j < kp; ++j) m = fmaxf(m, p0[j * piece + mo + ml]);
  float l = 0.f;
  for (int j = 0; j < kp; ++j)
    l = fmaf(p0[j * piece + mo + NW * 64 + ml], __builtin_amdgcn_exp2f(p0[j * piece + mo + ml] - m), l);
  const float inv = 1.0f / l;
  const long D = static_cast<long>(a.heads) * HD;
  const long orow = a.out_rows ? static_cast<long>(a.out_rows[qrow]) : qrow;
  uint16_t* op = a.out + orow * D + head * HD + 4 * hi;
  const float* acc = p0 + static_cast<long>(wave) * (NDB * 16 * 64) + lane;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float o[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < kp; ++j) {
        const float w = __builtin_amdgcn_exp2f(p0[j * piece + mo + ml] - m);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(acc[j * piece + (db * 16 + 4 * g + e) * 64], w, o[e]);
      }
      *reinterpret_cast<u32x2*>(op + db * 32 + g * 8) =
          u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    }
  if (a.lse && hi == 0) a.lse[head * a.n_q + qrow] = (m + __log2f(l)) * 0.69314718055994531f;
}

namespace {

// Workgroups of attention_split_kernel resident at once on the current device:
// compute units times resident workgroups per unit.  Cached per device.
template <int HD>
long resident_ctas() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attention_split_kernel<HD, false>,
                                                   64 * attn_waves<HD>(), 0) != hipSuccess)
    return 0;
  const int c = cus * (per_cu > 0 ? per_cu : 1);
  if (dev < kMaxDevices) cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

template <int HD>
long query_tiles(long n_q, int heads) {
  constexpr long bm = attn_rows<HD>();
  return (n_q + bm - 1) / bm * heads;
}

struct SplitPlan {
  long full = 0;  // tiles run whole
  long tail = 0;  // tiles cut into pieces
  int kp = 1;     // pieces per cut tile (1: no split)
};

// Cost model, in key-tile steps of one workgroup at full load.  Whole tiles in a
// partly filled last round run faster than at full load (measured on MI355X:
// about 0.79 + 0.1 x the full-load time with a fraction x of the workgroup slots
// busy), so that round costs n_t (0.79 + 0.1 r / C).  Split, it costs rounds of
// pieces of n_t / k steps plus about 3 steps of pipeline fill each, at the
// full-load rate.  The split is taken only when it saves at least 7%.
template <int HD>
SplitPlan split_plan(long n_q, long n_kv, int heads) {
  SplitPlan sp;
  const long c = resident_ctas<HD>();
  const long tiles = query_tiles<HD>(n_q, heads);
  const long n_t = (n_kv + kAttnBN - 1) / kAttnBN;
  if (c < 1) return sp;
  const long r = tiles % c;
  if (r == 0) return sp;
  const double whole = static_cast<double>(n_t) * (0.79 + 0.1 * static_cast<double>(r) / c);
  double best = whole;
  int best_k = 1;
  for (int k = 2; k <= kMaxPieces && static_cast<long>(k) * kMinPieceTiles <= n_t &&
                  r * k <= kMaxPieceSlots * c;
       ++k) {
    const double cost = static_cast<double>((r * k + c - 1) / c) * (static_cast<double>(n_t) / k + 3.0);
    if (cost < best) {
      best = cost;
      best_k = k;
    }
  }
  if (best_k == 1 || best > 0.93 * whole) return sp;
  sp.full = tiles - r;
  sp.tail = r;
  sp.kp = best_k;
  return sp;
}

template <int HD>
size_t split_bytes(const SplitPlan& sp) {
  return static_cast<size_t>(sp.tail) * sp.kp * attn_piece_floats<HD>() * sizeof(float);
}

// K/V of one head span more bytes than one buffer resource addresses.
bool big_kv(const AttnArgs& a, int hd) {
  return ((a.n_kv - 1) * a.heads * static_cast<long>(hd) + hd) * 2 > kMaxRangeBytes;
}

template <int HD, bool BIG>
hipError_t launch_hd(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  const SplitPlan sp = ws ? split_plan<HD>(a.n_q, a.n_kv, a.heads) : SplitPlan{};
  const dim3 block(64 * attn_waves<HD>());
  if (sp.kp == 1) {
    hipLaunchKernelGGL((attention_kernel<HD, BIG>), dim3(static_cast<unsigned>(query_tiles<HD>(a.n_q, a.heads))),
                       block, 0, s, a);
    return hipGetLastError();
  }
  if (ws_bytes < split_bytes<HD>(sp)) return hipErrorInvalidValue;
  float* w = static_cast<float*>(ws);
  hipLaunchKernelGGL((attention_split_kernel<HD, BIG>), dim3(static_cast<unsigned>(sp.full + sp.tail * sp.kp)),
                     block, 0, s, a, w, sp.full, sp.tail, sp.kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attention_merge_kernel<HD>, dim3(static_cast<unsigned>(sp.tail)), dim3(64 * attn_blocks<HD>()), 0, s, a,
                     static_cast<const float*>(w), sp.full, sp.kp);
  return hipGetLastError();
}

}  // namespace

size_t attention_workspace_bytes(long n_q, long n_kv, int heads, int head_dim) {
  return head_dim == 128 ? split_bytes<128>(split_plan<128>(n_q, n_kv, heads))
                         : split_bytes<64>(split_plan<64>(n_q, n_kv, heads));
}

hipError_t launch_attention_causal(const uint16_t* q, const uint16_t* k, const uint16_t* v, long n_q,
                                   long n_kv, int heads, int head_dim, float scale, const int* q_tokens,
                                   long frame_tokens, uint16_t* out, const int* out_rows, float* lse,
                                   hipStream_t s) {
  AttnArgs a{};
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
  a.q_tokens = q_tokens;
  a.frame_tokens = frame_tokens;
  const bool big = big_kv(a, head_dim);
  const dim3 grid128(static_cast<unsigned>(query_tiles<128>(n_q, heads))), block128(64 * attn_waves<128>());
  const dim3 grid64(static_cast<unsigned>(query_tiles<64>(n_q, heads))), block64(64 * attn_waves<64>());
  if (head_dim == 128 && big)
    hipLaunchKernelGGL((attention_causal_kernel<128, true>), grid128, block128, 0, s, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL((attention_causal_kernel<128, false>), grid128, block128, 0, s, a);
  else if (big)
    hipLaunchKernelGGL((attention_causal_kernel<64, true>), grid64, block64, 0, s, a);
  else
    hipLaunchKernelGGL((attention_causal_kernel<64, false>), grid64, block64, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, long n_q,
                            long n_kv, int heads, int head_dim, float scale, uint16_t* out,
                            const int* out_rows, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t s) {
  AttnArgs a{};
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
  if (big_kv(a, head_dim))
    return head_dim == 128 ? launch_hd<128, true>(a, ws, ws_bytes, s) : launch_hd<64, true>(a, ws, ws_bytes, s);
  return head_dim == 128 ? launch_hd<128, false>(a, ws, ws_bytes, s) : launch_hd<64, false>(a, ws, ws_bytes, s);
}

}  // namespace tsa
