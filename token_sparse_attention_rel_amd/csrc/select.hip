// a1-a3: token change scores, active-set selection and compaction.
//
// Scores: per-token (relative) L1 change against a reference row -- HSA page
// §2.1 (dynamic token selection ranks tokens by the relative L1 change of
// each token) and LIPAR page §2.B (L1 difference of a latent patch against
// the same spatial location in the previous frame, pruned below a threshold).
//
// Selection + compaction run in one workgroup of 1024 threads, each owning a
// run of 32 consecutive tokens per 32768-token chunk (the first chunk's scores
// stay in registers): an exact radix select (four 8-bit digit passes over
// order-preserving fp32 keys) finds the k-th largest score, then one ordered
// pass decides every token (ties at the k-th score go to the lowest token
// indices) and writes the ascending active and pruned index lists, positions
// from two workgroup prefix scans per chunk.
// The result is deterministic and does not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace tsa {

// ------------------------------------------------------------------ scores

template <typename T>
struct RowLoad;

template <>
struct RowLoad<uint16_t> {  // bf16: 8 elements per 16-byte load
  static constexpr int kVec = 8;
  __device__ static void load(const uint16_t* p, float* f) {
    unpack8(*reinterpret_cast<const u32x4*>(p), f);
  }
};

template <>
struct RowLoad<float> {  // fp32: 4 elements per 16-byte load
  static constexpr int kVec = 4;
  __device__ static void load(const float* p, float* f) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
    f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
  }
};

// One wave per token row: each lane accumulates sum|x - r| and sum|r| over
// its 16-byte slices, then a butterfly reduction.  The slices of a lane are
// loaded in batches of B, all loads of a batch issued before any is used, so a
// wave keeps 2*B 16-byte loads in flight.  Nontemporal loads: each row is read
// once (33 against 36 us for 2 x 32760 rows of 1536 bf16 with a flushed MALL).
// Fixed order: deterministic.
template <typename T, int B>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ x_cur,
                                                    const T* __restrict__ ref,
                                                    long ref_off, long n_rows, long dim,
                                                    int relative, float* __restrict__ scores) {
  constexpr int V = RowLoad<T>::kVec;
  const int lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const long rr = row - ref_off;
  if (rr < 0 || rr >= n_rows) {
    if (lane == 0) scores[row] = __builtin_inff();
    return;
  }
  const u32x4* a = reinterpret_cast<const u32x4*>(x_cur + row * dim);
  const u32x4* b = reinterpret_cast<const u32x4*>(ref + rr * dim);
  const long nsl = dim / V;
  float num = 0.f, den = 0.f;
  for (long c0 = 0; c0 < nsl; c0 += 64 * B) {
    u32x4 ra[B], rb[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const long c = c0 + lane + 64 * j;
      ra[j] = c < nsl ? __builtin_nontemporal_load(a + c) : u32x4{0u, 0u, 0u, 0u};
      rb[j] = c < nsl ? __builtin_nontemporal_load(b + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      float fa[V], fb[V];
      RowLoad<T>::load(reinterpret_cast<const T*>(&ra[j]), fa);
      RowLoad<T>::load(reinterpret_cast<const T*>(&rb[j]), fb);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        num += fabsf(fa[i] - fb[i]);
        den += fabsf(fb[i]);
      }
    }
  }
  num = wave_sum(num);
  den = wave_sum(den);
  if (lane == 0) {
    float s;
    if (!relative) {
      s = num;
    } else if (den == 0.f) {
      s = (num == 0.f) ? 0.f : __builtin_inff();
    } else {
      s = num / den;
    }
    scores[row] = s;
  }
}

// ---------------------------------------------------------- select/compact

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelRun = 32;                        // consecutive tokens per thread and chunk
constexpr int kSelChunk = kSelThreads * kSelRun;   // tokens per chunk

// Larger float -> larger key (total order on non-NaN values; -0 folded to +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.f) f = 0.f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SelShared {
  union {
    uint32_t hist[256];                  // radix passes: digit histogram
    int stage[kSelWaves][kSelRun * 64];  // compaction: a wave's index lists before the copy out
  };
  int scan[2][kSelWaves];
  uint32_t range[2][kSelWaves];  // per-wave min and max key
  uint32_t digit;
  int krem;
  uint8_t due[256];  // schedule mode: period p is due at this step
};

// A NaN whose order key is 0, the smallest key: fills the run past the last token.
constexpr uint32_t kPadBits = 0xFFFFFFFFu;

// Exclusive prefix of v over the workgroup (thread order); also returns the total.
// Alternates between two LDS slots so one barrier per call suffices.
__device__ __forceinline__ int block_excl_scan(int v, int& total, SelShared& sh, int& parity) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  int* slot = sh.scan[parity];
  parity ^= 1;
  if (lane == 63) slot[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = slot[w];
    before += (w < wave) ? t : 0;
    tot += t;
  }
  total = tot;
  return before + incl - v;
}

// The kSelRun scores of tokens i0 .. i0+kSelRun-1 as raw bits (kPadBits past n); all
// loads issued together.
__device__ __forceinline__ void load_run(const float* __restrict__ scores, long n, long i0,
                                         uint32_t (&v)[kSelRun]) {
  if (i0 + kSelRun <= n) {
    const u32x4* p = reinterpret_cast<const u32x4*>(scores + i0);
    u32x4 q[kSelRun / 4];
#pragma unroll
    for (int j = 0; j < kSelRun / 4; ++j) q[j] = p[j];
#pragma unroll
    for (int j = 0; j < kSelRun / 4; ++j) {
      v[4 * j] = q[j][0];
      v[4 * j + 1] = q[j][1];
      v[4 * j + 2] = q[j][2];
      v[4 * j + 3] = q[j][3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kSelRun; ++e) v[e] = (i0 + e < n) ? __float_as_uint(scores[i0 + e]) : kPadBits;
  }
}

enum SelKind { kByKey = 0, kNone = 1, kAll = 2, kThreshold = 3, kMask = 4, kSchedule = 5 };

// 32 bytes of 0/1 flags from the bits of m, as eight words (byte e = bit e).
__device__ __forceinline__ void bits_to_bytes(uint32_t m, uint32_t (&w)[kSelRun / 4]) {
#pragma unroll
  for (int j = 0; j < kSelRun / 4; ++j) {
    const uint32_t b = m >> (4 * j);
    w[j] = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
  }
}

// Thread t owns the run of kSelRun consecutive tokens starting at c*kSelChunk +
// t*kSelRun in chunk c (wave w the 2048 tokens from c*kSelChunk + 2048*w); the
// scores of chunk 0 stay in registers for all passes, as order keys when ranking.
__global__ __launch_bounds__(kSelThreads) void select_compact_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ aux, int n, int mode, int k,
    float tau, long step, uint8_t* __restrict__ mask_out, int* __restrict__ idx_out,
    int* __restrict__ pidx_out, int* __restrict__ n_active_out, uint8_t* __restrict__ group_accum,
    int accum_first) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long nl = n;
  const long n_chunks = (nl + kSelChunk - 1) / kSelChunk;

  int kind;
  if (mode == kSelectTopk) {
    kind = (k == 0) ? kNone : (k == n ? kAll : kByKey);
  } else if (mode == kSelectThreshold) {
    kind = kThreshold;
  } else if (mode == kSelectMask) {
    kind = kMask;
  } else {
    kind = kSchedule;
  }
  const bool scored = kind == kByKey || kind == kThreshold;
  if (kind == kSchedule) {
    if (tid < 256) sh.due[tid] = tid != 0 && step % tid == 0;
    __syncthreads();
  }

  // chunk 0: score bits, replaced by order keys when ranking
  uint32_t v0[kSelRun];
  const long r0 = static_cast<long>(tid) * kSelRun;
  if (scored) load_run(scores, nl, r0, v0);
  if (kind == kByKey) {
#pragma unroll
    for (int e = 0; e < kSelRun; ++e) v0[e] = order_key(__uint_as_float(v0[e]));
  }

  // ---- exact radix select of the k-th largest key (kByKey only)
  uint32_t thr = 0;
  int take_eq = 0;
  if (kind == kByKey) {
    // Smallest and largest key: the digits they share are shared by every key, so
    // ranking starts at the first digit where they differ (scores of one magnitude
    // skip the top digit).
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    auto range_run = [&](const uint32_t (&key)[kSelRun], long i0) {
      const long rem = nl - i0;
      const int nv = rem <= 0 ? 0 : (rem >= kSelRun ? kSelRun : static_cast<int>(rem));
#pragma unroll
      for (int e = 0; e < kSelRun; ++e) {
        if (e < nv) {
          kmin = key[e] < kmin ? key[e] : kmin;
          kmax = key[e] > kmax ? key[e] : kmax;
        }
      }
    };
    range_run(v0, r0);
    // tokens past the first chunk: four consecutive tokens per thread and step, the
    // scores read again from memory in every pass
    const long end = n_chunks * kSelChunk;
    auto stream_keys = [&](long i, uint32_t (&key)[4]) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(scores + (i + 4 <= nl ? i : 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b = i + 4 <= nl ? q[e] : (i + e < nl ? __float_as_uint(scores[i + e]) : kPadBits);
        key[e] = order_key(__uint_as_float(b));
      }
    };
    for (long i = kSelChunk + 4L * tid; i < nl; i += 4L * kSelThreads) {
      uint32_t key[4];
      stream_keys(i, key);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i + e < nl) {
          kmin = key[e] < kmin ? key[e] : kmin;
          kmax = key[e] > kmax ? key[e] : kmax;
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t a = __shfl_xor(kmin, off, 64), b = __shfl_xor(kmax, off, 64);
      kmin = a < kmin ? a : kmin;
      kmax = b > kmax ? b : kmax;
    }
    if (lane == 0) {
      sh.range[0][wave] = kmin;
      sh.range[1][wave] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      kmin = sh.range[0][w] < kmin ? sh.range[0][w] : kmin;
      kmax = sh.range[1][w] > kmax ? sh.range[1][w] : kmax;
    }
    const uint32_t diff = kmin ^ kmax;
    // first digit to rank: the one holding the highest differing bit (-8: all keys equal)
    const int start = diff == 0 ? -8 : ((31 - __clz(diff)) & ~7);
    // bits above digit `start` (all bits when every key is equal)
    uint32_t pmask = start < 0 ? 0xFFFFFFFFu : (start >= 24 ? 0u : ~((2u << (start + 7)) - 1u));
    uint32_t prefix = kmin & pmask;
    int krem = k;
    // Pad entries past n carry key 0; they are taken out of bin 0 while the prefix is 0.
    const uint32_t n_pad = static_cast<uint32_t>(n_chunks * kSelChunk - nl);
    // Histogram of digit `shift` over the keys that match the prefix.  In the first
    // pass every key takes part and a thread's keys are consecutive tokens: equal
    // digits in a row are added as one count (scores of similar size share their
    // leading digits), so fewer lanes contend for one bin.  Later passes count the
    // few keys under the prefix with one increment each.
    uint32_t run_d = 0, run_n = 0;
    auto count_key = [&](uint32_t key, int shift, bool merge) {
      if ((key & pmask) != prefix) return;
      const uint32_t d = (key >> shift) & 255u;
      if (!merge) {
        atomicAdd(&sh.hist[d], 1u);
      } else if (d != run_d) {
        if (run_n) atomicAdd(&sh.hist[run_d], run_n);
        run_d = d;
        run_n = 1;
      } else {
        ++run_n;
      }
    };
    for (int shift = start; shift >= 0; shift -= 8) {
      if (tid < 256) sh.hist[tid] = 0;
      __syncthreads();
      const bool merge = shift == start;
      if (merge) {
#pragma unroll
        for (int e = 0; e < kSelRun; ++e) count_key(v0[e], shift, true);
      } else {
#pragma unroll
        for (int e = 0; e < kSelRun; ++e) count_key(v0[e], shift, false);
      }
      for (long i = kSelChunk + 4L * tid; i < end; i += 4L * kSelThreads) {
        uint32_t key[4];
        stream_keys(i, key);  // pads past n carry key 0 like those of the first chunk
#pragma unroll
        for (int e = 0; e < 4; ++e) count_key(key[e], shift, merge);
      }
      if (run_n) atomicAdd(&sh.hist[run_d], run_n);
      run_n = 0;
      __syncthreads();
      if (wave == 0) {
        // lane owns bins 4*lane .. 4*lane+3; find the bin where the running count
        // from the top reaches krem
        uint32_t cnt[4];
        uint32_t lsum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t t = sh.hist[4 * lane + j];
          if (lane == 0 && j == 0 && prefix == 0) t -= n_pad;
          cnt[j] = t;
          lsum += t;
        }
        uint32_t suf = lsum;  // inclusive suffix over lanes >= lane
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t t = __shfl_down(suf, off, 64);
          if (lane + off < 64) suf += t;
        }
        uint32_t above = suf - lsum;  // count in bins of higher lanes
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          const uint32_t incl = above + cnt[j];
          if (above < static_cast<uint32_t>(krem) && incl >= static_cast<uint32_t>(krem)) {
            sh.digit = 4 * lane + j;
            sh.krem = krem - static_cast<int>(above);
          }
          above = incl;
        }
      }
      __syncthreads();
      prefix |= sh.digit << shift;
      pmask |= 255u << shift;
      krem = sh.krem;
    }
    thr = prefix;
    take_eq = krem;
  }

  // ---- ordered decision + compaction, one run per thread and chunk.  The index
  // lists of a wave's 2048 tokens are staged in LDS and copied out contiguously.
  int parity = 0;
  int run_active = 0, run_eq = 0;
  const bool mask_vec = (reinterpret_cast<uintptr_t>(mask_out) & 15u) == 0;
  const bool accum_vec = (reinterpret_cast<uintptr_t>(group_accum) & 15u) == 0;
  auto decide_run = [&](const uint32_t (&v)[kSelRun], long i0, long wave_tok0) {
    const long rem = nl - i0;
    const int nv = rem <= 0 ? 0 : (rem >= kSelRun ? kSelRun : static_cast<int>(rem));
    const uint32_t vm = nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u);  // bit e: token i0 + e exists
    uint32_t actm = 0, eqm = 0;
    if (kind == kByKey) {
#pragma unroll
      for (int e = 0; e < kSelRun; ++e) {
        actm |= (v[e] > thr ? 1u : 0u) << e;
        eqm |= (v[e] == thr ? 1u : 0u) << e;
      }
    } else if (kind == kThreshold) {
#pragma unroll
      for (int e = 0; e < kSelRun; ++e) actm |= (__uint_as_float(v[e]) >= tau ? 1u : 0u) << e;
    } else if (kind == kAll) {
      actm = 0xFFFFFFFFu;
    } else if (kind == kMask || kind == kSchedule) {
#pragma unroll
      for (int e = 0; e < kSelRun; ++e) {
        if (e < nv) {
          const uint8_t p = aux[i0 + e];
          const bool a = kind == kMask ? p != 0 : sh.due[p] != 0;
          actm |= (a ? 1u : 0u) << e;
        }
      }
    }
    actm &= vm;
    eqm &= vm;
    if (kind == kByKey) {
      // ties at the k-th key: the lowest token indices are taken first
      int tot_eq;
      const int r = run_eq + block_excl_scan(__popc(eqm), tot_eq, sh, parity);
      run_eq += tot_eq;
      const int take = take_eq - r;  // eq tokens of this run that are taken
      uint32_t m = eqm;
      for (int t = 0; t < take && m; ++t) {
        actm |= m & (~m + 1u);  // lowest remaining eq token
        m &= m - 1u;
      }
    }
    int tot_act;
    const int cact = __popc(actm);
    const int pos = run_active + block_excl_scan(cact, tot_act, sh, parity);
    run_active += tot_act;

    if (group_accum) {
      // rank-group mode: count the boundaries each token falls behind
      if (nv == kSelRun && accum_vec) {
        uint32_t w[kSelRun / 4];
        bits_to_bytes(~actm, w);
        u32x4* g = reinterpret_cast<u32x4*>(group_accum + i0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 o{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
          if (!accum_first) o += g[h];  // bytes stay below 256: at most 16 groups
          g[h] = o;
        }
      } else {
        for (int e = 0; e < nv; ++e) {
          const uint8_t behind = ((actm >> e) & 1u) ? 0 : 1;
          group_accum[i0 + e] = accum_first ? behind : static_cast<uint8_t>(group_accum[i0 + e] + behind);
        }
      }
      return;
    }
    if (nv == kSelRun && mask_vec) {
      uint32_t w[kSelRun / 4];
      bits_to_bytes(actm, w);
      u32x4* mp = reinterpret_cast<u32x4*>(mask_out + i0);
      mp[0] = u32x4{w[0], w[1], w[2], w[3]};
      mp[1] = u32x4{w[4], w[5], w[6], w[7]};
    } else {
      for (int e = 0; e < nv; ++e) mask_out[i0 + e] = (actm >> e) & 1u;
    }
    // wave-local list positions: actives first, then the pruned tokens
    const int pos0 = __builtin_amdgcn_readfirstlane(pos);
    const int a_w = __builtin_amdgcn_readlane(pos + cact, 63) - pos0;
    const long wrem = nl - wave_tok0;
    const int n_w = wrem <= 0 ? 0 : (wrem >= kSelRun * 64 ? kSelRun * 64 : static_cast<int>(wrem));
    int la = pos - pos0;               // next active slot of this thread
    int lp = a_w + kSelRun * lane - (pos - pos0);  // next pruned slot
    int* st = sh.stage[wave];
    // slot j lives at j ^ (j/32 mod 32): a lane's run of slots and a wave's 64
    // consecutive slots both spread over the LDS banks
    auto sw = [](int j) { return j ^ ((j >> 5) & 31); };
    for (int e = 0; e < nv; ++e) {
      const int i = static_cast<int>(i0 + e);
      if ((actm >> e) & 1u)
        st[sw(la++)] = i;
      else
        st[sw(lp++)] = i;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int j = lane; j < a_w; j += 64) idx_out[pos0 + j] = st[sw(j)];
    if (pidx_out) {
      const long p0 = wave_tok0 - pos0;  // pruned-list position of the wave's first pruned token
      for (int j = lane; j < n_w - a_w; j += 64) pidx_out[p0 + j] = st[sw(a_w + j)];
    }
  };
  decide_run(v0, r0, static_cast<long>(wave) * kSelRun * 64);
  for (long c = 1; c < n_chunks; ++c) {
    uint32_t v[kSelRun];
    const long i0 = c * kSelChunk + r0;
    if (scored) load_run(scores, nl, i0, v);
    if (kind == kByKey) {
#pragma unroll
      for (int e = 0; e < kSelRun; ++e) v[e] = order_key(__uint_as_float(v[e]));
    }
    decide_run(v, i0, c * kSelChunk + static_cast<long>(wave) * kSelRun * 64);
  }
  if (tid == 0 && n_active_out) *n_active_out = run_active;
}

__global__ void map_groups_kernel(const uint8_t* __restrict__ group, int n, GroupPeriods table,
                                  uint8_t* __restrict__ period_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) period_out[i] = table.p[group ? group[i] : 0];
}

// ------------------------------------------------------------------ launch

template <typename T, int B>
void launch_scores_t(const void* x_cur, const void* x_ref, long ref_off, long n_rows, long dim,
                     int relative, float* scores, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((n_rows + 3) / 4));
  hipLaunchKernelGGL((score_kernel<T, B>), grid, dim3(256), 0, s, static_cast<const T*>(x_cur),
                     static_cast<const T*>(x_ref ? x_ref : x_cur), ref_off, n_rows, dim, relative, scores);
}

hipError_t launch_scores(const void* x_cur, const void* x_ref, long ref_off, long n_rows,
                         long dim, int dtype, int relative, float* scores, hipStream_t s) {
  // slices per lane: a batch large enough for the whole row up to 64*4 slices
  const long per_lane = (dim / (dtype == kDtypeBf16 ? 8 : 4) + 63) / 64;
  if (dtype == kDtypeBf16) {
    if (per_lane <= 2)
      launch_scores_t<uint16_t, 2>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
    else if (per_lane == 3)
      launch_scores_t<uint16_t, 3>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
    else
      launch_scores_t<uint16_t, 4>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
  } else {
    if (per_lane <= 2)
      launch_scores_t<float, 2>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
    else if (per_lane == 3)
      launch_scores_t<float, 3>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
    else
      launch_scores_t<float, 4>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, const uint8_t* aux, int n, int mode, int k,
                         float tau, long step, uint8_t* mask, int* idx, int* pidx, int* n_active,
                         uint8_t* group_accum, int accum_first, hipStream_t s) {
  hipLaunchKernelGGL(select_compact_kernel, dim3(1), dim3(kSelThreads), 0, s, scores, aux, n,
                     mode, k, tau, step, mask, idx, pidx, n_active, group_accum, accum_first);
  return hipGetLastError();
}

hipError_t launch_map_groups(const uint8_t* group, int n, const GroupPeriods& table,
                             uint8_t* period_out, hipStream_t s) {
  hipLaunchKernelGGL(map_groups_kernel, dim3((n + 255) / 256), dim3(256), 0, s, group, n, table,
                     period_out);
  return hipGetLastError();
}

}  // namespace tsa
