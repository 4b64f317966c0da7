// Steps beside the pruned layer: the cached Euler update of the sampler, the
// long/short-term inter-frame pruning mask and the restoration of pruned frames.
//
// Euler (HSA page §2.3): after every global step all N tokens advance by the
// same increment dt = sigma_{i+1} - sigma_i along their cached velocity, one
// elementwise pass: x <- x + dt * v_hat.  HBM-bound.
//
// Pruning mask (LIPAR page §2.B): each latent token is compared with the same
// spatial location one frame earlier (short-term change) and in the most
// recent frame where that location was kept (long-term change); it is pruned
// only when both are below their thresholds.  The long-term reference depends
// on the decisions of earlier frames, so each location is scanned frame by
// frame by one workgroup that keeps the previous and the reference row in
// registers, with the next frames' rows in flight: every latent row is read once.
//
// Restoration (Dutch LIPAR page §2.D): after denoising, a pruned token takes
// the value of the same location in the previous frame -- a forward fill along
// the frame axis.  One thread per 16-byte slice of a location's row carries
// the last kept slice down the frames: kept rows are read once, pruned rows
// written once.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace tsa {

// ------------------------------------------------------------------ Euler

// x (fp32 or bf16) += dt * v (bf16), 8 elements per thread.
// fp32: fmaf rounds the exact value once; bf16: that fp32 result is rounded to
// nearest even.
template <typename T>
__global__ __launch_bounds__(256) void euler_kernel(T* __restrict__ x, const uint16_t* __restrict__ v,
                                                    long n8, float dt) {
  const long c = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (c < n8) {
    float fv[8];
    unpack8(reinterpret_cast<const u32x4*>(v)[c], fv);
    if constexpr (sizeof(T) == 4) {
      f32x4* xp = reinterpret_cast<f32x4*>(x) + 2 * c;
      f32x4 a = xp[0], b = xp[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = fmaf(dt, fv[i], a[i]);
        b[i] = fmaf(dt, fv[4 + i], b[i]);
      }
      xp[0] = a;
      xp[1] = b;
    } else {
      u32x4* xp = reinterpret_cast<u32x4*>(x) + c;
      float fx[8];
      unpack8(*xp, fx);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(fmaf(dt, fv[2 * i], fx[2 * i]), fmaf(dt, fv[2 * i + 1], fx[2 * i + 1]));
      *xp = o;
    }
  }
}

hipError_t launch_euler(void* x, int x_dtype, const uint16_t* v, long n_elems, float dt, hipStream_t s) {
  const long n8 = n_elems / 8;
  const dim3 grid(static_cast<unsigned>((n8 + 255) / 256));
  if (x_dtype == kDtypeF32)
    hipLaunchKernelGGL(euler_kernel<float>, grid, dim3(256), 0, s, static_cast<float*>(x), v, n8, dt);
  else
    hipLaunchKernelGGL(euler_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<uint16_t*>(x), v, n8, dt);
  return hipGetLastError();
}

// ------------------------------------------------------- pruning mask

constexpr int kLifThreads = 256;
constexpr int kLifAhead = 4;  // frames whose rows are in flight while one is reduced

template <typename T>
struct Slice;  // one 16-byte slice of a row, unpacked to fp32

template <>
struct Slice<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static void unpack(const u32x4 r, float* f) { unpack8(r, f); }
};

template <>
struct Slice<float> {
  static constexpr int kVec = 4;
  __device__ static void unpack(const u32x4 r, float* f) {
    f[0] = __uint_as_float(r[0]); f[1] = __uint_as_float(r[1]);
    f[2] = __uint_as_float(r[2]); f[3] = __uint_as_float(r[3]);
  }
};

// Sum four values over the workgroup in a fixed order (wave butterflies, then
// the four wave partials in wave order): deterministic.  part alternates between
// two halves from call to call, so one barrier per call suffices.
__device__ __forceinline__ void block_sum4(float v[4], float (*part)[kLifThreads / 64][4], int& parity) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = wave_sum(v[i]);
  float (*pp)[4] = part[parity];
  parity ^= 1;
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pp[wave][i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (pp[0][i] + pp[1][i]) + (pp[2][i] + pp[3][i]);
}

__device__ __forceinline__ float l1_score(float num, float den, int relative) {
  if (!relative) return num;
  if (den == 0.f) return num == 0.f ? 0.f : __builtin_inff();
  return num / den;
}

// One workgroup per spatial location; CPT 16-byte slices per thread and row.  The
// rows of the next kLifAhead frames stay in flight (raw, in a register ring) while
// the current one is reduced.
template <typename T, int CPT>
__global__ __launch_bounds__(kLifThreads) void lif_mask_kernel(const T* __restrict__ x, long frames, long hw,
                                                               long dim, int relative, float tau_s,
                                                               float tau_l, uint8_t* __restrict__ mask,
                                                               float* __restrict__ short_out,
                                                               float* __restrict__ long_out) {
  constexpr int V = Slice<T>::kVec;
  __shared__ float part[2][kLifThreads / 64][4];
  const long loc = blockIdx.x;
  const long n_sl = dim / V;
  auto load_raw = [&](u32x4 (&dst)[CPT], long f) {
    const T* row = x + (f * hw + loc) * dim;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const long sl = threadIdx.x + static_cast<long>(kLifThreads) * j;
      dst[j] = sl < n_sl ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + sl * V))
                         : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto unpack_row = [&](const u32x4 (&r)[CPT], float (*dst)[V]) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) Slice<T>::unpack(r[j], dst[j]);
  };
  float prev[CPT][V], ref[CPT][V], cur[CPT][V];
  u32x4 ring[kLifAhead][CPT];
  load_raw(ring[0], 0);
#pragma unroll
  for (int p = 1; p < kLifAhead; ++p)
    if (p < frames) load_raw(ring[p], p);
  unpack_row(ring[0], prev);
  if (kLifAhead < frames) load_raw(ring[0], kLifAhead);
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < V; ++e) ref[j][e] = prev[j][e];
  if (threadIdx.x == 0) {
    mask[loc] = 1;
    if (short_out) short_out[loc] = __builtin_inff();
    if (long_out) long_out[loc] = __builtin_inff();
  }
  int parity = 0;
  // Frame f's row lives in ring slot f % kLifAhead; the slot is a compile-time
  // index (the frame loop is unrolled by kLifAhead), so no register is copied
  // while its load may still be in flight.
  auto step = [&](long f, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    unpack_row(ring[slot], cur);
    // the slot is free again: fetch the frame kLifAhead ahead into it
    if (f + kLifAhead < frames) load_raw(ring[slot], f + kLifAhead);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};  // short num, short den, long num, long den
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        acc[0] += fabsf(cur[j][e] - prev[j][e]);
        acc[1] += fabsf(prev[j][e]);
        acc[2] += fabsf(cur[j][e] - ref[j][e]);
        acc[3] += fabsf(ref[j][e]);
      }
    block_sum4(acc, part, parity);
    const float ss = l1_score(acc[0], acc[1], relative);
    const float ls = l1_score(acc[2], acc[3], relative);
    const bool keep = !((ss < tau_s) && (ls < tau_l));
    const long t = f * hw + loc;
    if (threadIdx.x == 0) {
      mask[t] = keep ? 1 : 0;
      if (short_out) short_out[t] = ss;
      if (long_out) long_out[t] = ls;
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (keep) ref[j][e] = cur[j][e];
        prev[j][e] = cur[j][e];
      }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  static_assert(kLifAhead == 4, "the unrolled frame loop below has four slots");
  long f = 1;
  for (; f + 3 < frames; f += 4) {
    step(f, S1{});
    step(f + 1, S2{});
    step(f + 2, S3{});
    step(f + 3, S0{});
  }
  if (f < frames) step(f, S1{});
  if (f + 1 < frames) step(f + 1, S2{});
  if (f + 2 < frames) step(f + 2, S3{});
}

// Rows of up to 64 * kLifWaveMaxCpt slices: one wave per spatial location (four per
// 256-thread workgroup).  Lane l holds slices l + 64 j (j < CPT) of each row as raw
// 16-byte slices: frame f sits in ring slot f mod 3, so the previous frame is the slot
// before it and the frame two ahead is fetched into the previous frame's slot once it is
// used; the last kept row and the sums of magnitudes of the previous and the kept row
// (the denominators of the relative scores) are carried along.  Sums cross the wave by
// DPP moves and four lane reads in a fixed order: no LDS, no barrier between frames.
constexpr int kLifWaveMaxCpt = 6;

template <typename T, int CPT>
__global__ __launch_bounds__(256) void lif_mask_wave_kernel(const T* __restrict__ x, long frames, long hw,
                                                            long dim, int relative, float tau_s, float tau_l,
                                                            uint8_t* __restrict__ mask,
                                                            float* __restrict__ short_out,
                                                            float* __restrict__ long_out) {
  constexpr int V = Slice<T>::kVec;
  const long loc = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (loc >= hw) return;  // a whole wave
  const int lane = threadIdx.x & 63;
  const long n_sl = dim / V;
  // slices past the row end read the last slice (no branch around the load) and count as zero
  auto load_raw = [&](u32x4 (&dst)[CPT], long f) {
    const T* row = x + (f * hw + loc) * dim;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const long sl = lane + 64L * j;
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + (sl < n_sl ? sl : n_sl - 1) * V));
      dst[j] = sl < n_sl ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 ring[3][CPT], ref[CPT];
  load_raw(ring[0], 0);
  if (1 < frames) load_raw(ring[1], 1);
  if (2 < frames) load_raw(ring[2], 2);
  float den_prev = 0.f;  // sum |x| of the previous row
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    float p[V];
    Slice<T>::unpack(ring[0][j], p);
#pragma unroll
    for (int e = 0; e < V; ++e) den_prev += fabsf(p[e]);
    ref[j] = ring[0][j];
  }
  den_prev = wave_sum_dpp(den_prev);
  float den_ref = den_prev;  // sum |x| of the last kept row
  if (lane == 0) {
    mask[loc] = 1;
    if (short_out) short_out[loc] = __builtin_inff();
    if (long_out) long_out[loc] = __builtin_inff();
  }
  auto step = [&](long f, auto cur_c, auto tail_c) {
    constexpr int sc = decltype(cur_c)::value, sp = (sc + 2) % 3;  // slots of frames f and f - 1
    float num_s = 0.f, num_l = 0.f, den_c = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float c[V], p[V], r[V];
      // unpack the previous row again rather than keep last step's fp32 copy of it live
      // (an empty asm hides that the two are equal): three raw rows fit the registers,
      // three fp32 rows do not
      u32x4 pr = ring[sp][j], rr = ref[j];
      asm volatile("" : "+v"(pr), "+v"(rr));
      Slice<T>::unpack(ring[sc][j], c);
      Slice<T>::unpack(pr, p);
      Slice<T>::unpack(rr, r);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        num_s += fabsf(c[e] - p[e]);
        num_l += fabsf(c[e] - r[e]);
        den_c += fabsf(c[e]);
      }
      __builtin_amdgcn_sched_barrier(0);  // one slice at a time
    }
    // frame f - 1 is no longer needed: fetch frame f + 2 into its slot (inside the main
    // loop it always exists; a conditional fetch there would keep the old row live too)
    if (!decltype(tail_c)::value || f + 2 < frames) load_raw(ring[sp], f + 2);
    num_s = wave_sum_dpp(num_s);
    num_l = wave_sum_dpp(num_l);
    den_c = wave_sum_dpp(den_c);
    const float ss = l1_score(num_s, den_prev, relative);
    const float ls = l1_score(num_l, den_ref, relative);
    // the sums are wave-uniform, so is the decision: say so, and the row update is a branch
    const bool keep = __builtin_amdgcn_readfirstlane(!((ss < tau_s) && (ls < tau_l)) ? 1 : 0) != 0;
    const long t = f * hw + loc;
    if (lane == 0) {
      mask[t] = keep ? 1 : 0;
      if (short_out) short_out[t] = ss;
      if (long_out) long_out[t] = ls;
    }
    if (keep) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) ref[j] = ring[sc][j];
      den_ref = den_c;
    }
    den_prev = den_c;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using Main = std::false_type;
  using Tail = std::true_type;
  long f = 1;
  for (; f + 4 < frames; f += 3) {  // fetches up to frame f + 4
    step(f, S1{}, Main{});
    step(f + 1, S2{}, Main{});
    step(f + 2, S0{}, Main{});
  }
  // at most four frames left
  if (f < frames) step(f, S1{}, Tail{});
  if (f + 1 < frames) step(f + 1, S2{}, Tail{});
  if (f + 2 < frames) step(f + 2, S0{}, Tail{});
  if (f + 3 < frames) step(f + 3, S1{}, Tail{});
}

template <typename T>
hipError_t launch_lif_t(const T* x, long frames, long hw, long dim, int relative, float tau_s, float tau_l,
                        uint8_t* mask, float* so, float* lo, hipStream_t s) {
  const long n_sl = dim / Slice<T>::kVec;
  const long wcpt = (n_sl + 63) / 64;  // slices per lane with one wave per location
  if (wcpt <= kLifWaveMaxCpt) {
    const dim3 wgrid(static_cast<unsigned>((hw + 3) / 4)), wblock(256);
    switch (wcpt <= 2 ? wcpt : (wcpt <= 4 ? 4 : kLifWaveMaxCpt)) {
      case 1: hipLaunchKernelGGL((lif_mask_wave_kernel<T, 1>), wgrid, wblock, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
      case 2: hipLaunchKernelGGL((lif_mask_wave_kernel<T, 2>), wgrid, wblock, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
      case 4: hipLaunchKernelGGL((lif_mask_wave_kernel<T, 4>), wgrid, wblock, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
      default: hipLaunchKernelGGL((lif_mask_wave_kernel<T, kLifWaveMaxCpt>), wgrid, wblock, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
    }
    return hipGetLastError();
  }
  // longer rows: one workgroup per location
  const long cpt = (n_sl + kLifThreads - 1) / kLifThreads;
  const dim3 grid(static_cast<unsigned>(hw)), block(kLifThreads);
  switch (cpt) {
    case 1: hipLaunchKernelGGL((lif_mask_kernel<T, 1>), grid, block, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
    case 2: hipLaunchKernelGGL((lif_mask_kernel<T, 2>), grid, block, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
    case 3: hipLaunchKernelGGL((lif_mask_kernel<T, 3>), grid, block, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
    case 4: hipLaunchKernelGGL((lif_mask_kernel<T, 4>), grid, block, 0, s, x, frames, hw, dim, relative, tau_s, tau_l, mask, so, lo); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

long lif_max_dim(int dtype) { return (dtype == kDtypeF32 ? 4L : 8L) * kLifThreads * 4; }

hipError_t launch_lif_mask(const void* x, int dtype, long frames, long hw, long dim, int relative, float tau_s,
                           float tau_l, uint8_t* mask, float* short_out, float* long_out, hipStream_t s) {
  if (dtype == kDtypeF32)
    return launch_lif_t(static_cast<const float*>(x), frames, hw, dim, relative, tau_s, tau_l, mask, short_out,
                        long_out, s);
  return launch_lif_t(static_cast<const uint16_t*>(x), frames, hw, dim, relative, tau_s, tau_l, mask, short_out,
                      long_out, s);
}

// ----------------------------------------------------------- restoration

// Thread = (location, 16-byte slice); rows of row_bytes bytes.  The kept
// slices of up to 8 frames are loaded together, then the pruned ones written.
__global__ __launch_bounds__(256) void restore_kernel(u32x4* __restrict__ buf, const uint8_t* __restrict__ mask,
                                                      long frames, long hw, long slices) {
  constexpr int kF = 8;
  const long id = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= hw * slices) return;
  const long loc = id / slices, sl = id - loc * slices;
  u32x4 carry = buf[loc * slices + sl];
  for (long f0 = 1; f0 < frames; f0 += kF) {
    bool kept[kF];
    u32x4 r[kF];
#pragma unroll
    for (int i = 0; i < kF; ++i) {
      const long f = f0 + i;
      kept[i] = f < frames && mask[f * hw + loc];
      if (kept[i]) r[i] = __builtin_nontemporal_load(buf + (f * hw + loc) * slices + sl);
    }
#pragma unroll
    for (int i = 0; i < kF; ++i) {
      const long f = f0 + i;
      if (f >= frames) break;
      if (kept[i])
        carry = r[i];
      else
        buf[(f * hw + loc) * slices + sl] = carry;
    }
  }
}

hipError_t launch_restore(void* buf, const uint8_t* mask, long frames, long hw, long row_bytes, hipStream_t s) {
  const long slices = row_bytes / 16;
  const long threads = hw * slices;
  hipLaunchKernelGGL(restore_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s,
                     static_cast<u32x4*>(buf), mask, frames, hw, slices);
  return hipGetLastError();
}

}  // namespace tsa
