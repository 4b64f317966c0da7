// a1-a3: token change scores, active-set selection and compaction.
//
// Scores: per-token (relative) L1 change against a reference row -- HSA page
// §2.1 (dynamic token selection ranks tokens by the relative L1 change of
// each token) and LIPAR page §2.B (L1 difference of a latent patch against
// the same spatial location in the previous frame, pruned below a threshold).
//
// Selection + compaction run in one workgroup of 1024 threads: an exact
// radix select (four 8-bit digit passes over order-preserving fp32 keys)
// finds the k-th largest score, then one ordered pass decides every token
// (ties at the k-th score go to the lowest token indices) and writes the
// ascending active and pruned index lists with ballot/mbcnt + LDS scans.
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
// wave keeps 2*B 16-byte loads in flight.  Fixed order: deterministic.
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
      ra[j] = c < nsl ? a[c] : u32x4{0u, 0u, 0u, 0u};
      rb[j] = c < nsl ? b[c] : u32x4{0u, 0u, 0u, 0u};
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
constexpr int kSelPer = 4;                      // consecutive tokens per thread per tile
constexpr int kSelTile = kSelThreads * kSelPer;  // tokens per tile

// Larger float -> larger key (total order on non-NaN values; -0 folded to +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.f) f = 0.f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SelShared {
  uint32_t hist[kSelWaves][256];
  int scan[2][kSelWaves];
  uint32_t digit;
  int krem;
};

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

enum SelKind { kByKey = 0, kNone = 1, kAll = 2, kThreshold = 3, kMask = 4, kSchedule = 5 };

__global__ __launch_bounds__(kSelThreads) void select_compact_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ aux, int n, int mode, int k,
    float tau, long step, uint8_t* __restrict__ mask_out, int* __restrict__ idx_out,
    int* __restrict__ pidx_out, int* __restrict__ n_active_out, uint8_t* __restrict__ group_accum,
    int accum_first) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

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

  // ---- exact radix select of the k-th largest key (kByKey only)
  uint32_t thr = 0;
  int take_eq = 0;
  if (kind == kByKey) {
    uint32_t prefix = 0, pmask = 0;
    int krem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0;
      __syncthreads();
      for (int base = 0; base < n; base += kSelTile) {
        const int i0 = base + tid * kSelPer;
        float v[kSelPer];
        if (i0 + kSelPer <= n) {
          const f32x4 q = *reinterpret_cast<const f32x4*>(scores + i0);
          v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
        } else {
#pragma unroll
          for (int e = 0; e < kSelPer; ++e) v[e] = (i0 + e < n) ? scores[i0 + e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < kSelPer; ++e) {
          const uint32_t key = order_key(v[e]);
          const bool has = (i0 + e < n) && ((key & pmask) == prefix);
          const uint32_t d = (key >> shift) & 255u;
          // Wave-aggregated increment when every participating lane has the same digit
          // (the common case for the high digits), plain LDS atomics otherwise.
          const uint64_t act = __ballot(has);
          if (act) {
            const int first = __builtin_ctzll(act);
            const uint32_t d0 = __shfl(d, first, 64);
            const uint64_t same = __ballot(has && d == d0);
            if (same == act) {
              if (lane == first) atomicAdd(&sh.hist[wave][d0], static_cast<uint32_t>(__popcll(act)));
            } else if (has) {
              atomicAdd(&sh.hist[wave][d], 1u);
            }
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        // lane owns bins 4*lane .. 4*lane+3; find the bin where the running count
        // from the top reaches krem
        uint32_t c[4];
        uint32_t lsum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t t = 0;
#pragma unroll
          for (int w = 0; w < kSelWaves; ++w) t += sh.hist[w][4 * lane + j];
          c[j] = t;
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
          const uint32_t incl = above + c[j];
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

  // ---- ordered decision + compaction
  int parity = 0;
  int run_active = 0, run_eq = 0;
  for (int base = 0; base < n; base += kSelTile) {
    const int i0 = base + tid * kSelPer;
    bool valid[kSelPer], act[kSelPer], eq[kSelPer];
    int ceq = 0;
    if (kind == kByKey || kind == kThreshold) {
      float v[kSelPer];
      if (i0 + kSelPer <= n) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(scores + i0);
        v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
      } else {
#pragma unroll
        for (int e = 0; e < kSelPer; ++e) v[e] = (i0 + e < n) ? scores[i0 + e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < kSelPer; ++e) {
        valid[e] = i0 + e < n;
        if (kind == kByKey) {
          const uint32_t key = order_key(v[e]);
          act[e] = valid[e] && key > thr;
          eq[e] = valid[e] && key == thr;
        } else {
          act[e] = valid[e] && (v[e] >= tau);
          eq[e] = false;
        }
        ceq += eq[e] ? 1 : 0;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kSelPer; ++e) {
        valid[e] = i0 + e < n;
        eq[e] = false;
        bool a = false;
        if (valid[e]) {
          if (kind == kAll) {
            a = true;
          } else if (kind == kMask) {
            a = aux[i0 + e] != 0;
          } else if (kind == kSchedule) {
            const long p = aux[i0 + e];
            a = (p != 0) && (step % p == 0);
          }
        }
        act[e] = a;
      }
    }
    if (kind == kByKey) {
      int tot_eq;
      int r = run_eq + block_excl_scan(ceq, tot_eq, sh, parity);
      run_eq += tot_eq;
#pragma unroll
      for (int e = 0; e < kSelPer; ++e) {
        if (eq[e]) {
          act[e] = r < take_eq;
          ++r;
        }
      }
    }
    int cact = 0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) cact += act[e] ? 1 : 0;
    int tot_act;
    int pos = run_active + block_excl_scan(cact, tot_act, sh, parity);
    run_active += tot_act;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
      if (!valid[e]) continue;
      const int i = i0 + e;
      if (group_accum) {
        // rank-group mode: count the boundaries this token falls behind
        const uint8_t behind = act[e] ? 0 : 1;
        group_accum[i] = accum_first ? behind : static_cast<uint8_t>(group_accum[i] + behind);
        continue;
      }
      mask_out[i] = act[e] ? 1 : 0;
      if (act[e]) {
        idx_out[pos] = i;
        ++pos;
      } else if (pidx_out) {
        pidx_out[i - pos] = i;
      }
    }
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
    else
      launch_scores_t<uint16_t, 4>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
  } else {
    if (per_lane <= 2)
      launch_scores_t<float, 2>(x_cur, x_ref, ref_off, n_rows, dim, relative, scores, s);
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
