// Device helpers shared by the tsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Unpack 8 bf16 held in a 16-byte vector into fp32.
__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// LIPAR recovery of 8 bf16 elements: bf16((1 - s) * clean + s * noise), the
// products and sum in fp32 (one fused multiply-add), rounded to nearest even.
__device__ __forceinline__ u32x4 recover8(const u32x4 clean, const u32x4 noise, float one_m_s, float s) {
  float c[8], e[8];
  unpack8(clean, c);
  unpack8(noise, e);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = fmaf(one_m_s, c[2 * i], s * e[2 * i]);
    const float b = fmaf(one_m_s, c[2 * i + 1], s * e[2 * i + 1]);
    r[i] = pack_bf16x2(a, b);
  }
  return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Data-parallel-primitive moves inside a row of 16 lanes (quad_perm 1,0,3,2 and
// 2,3,0,1, half-row mirror, row mirror): summing a value with each in turn leaves
// every lane of an aligned group of 4, 8 or 16 lanes holding the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(L == 4 || L == 8 || L == 16, "lane groups of 4, 8 or 16");
  v += dpp_move<0xB1>(v);  // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  if constexpr (L >= 8) v += dpp_move<0x141>(v);   // row_half_mirror: lane i <-> 7 - i
  if constexpr (L >= 16) v += dpp_move<0x140>(v);  // row_mirror: lane i <-> 15 - i
  return v;
}

// Sum over the 64 lanes of a wave in a fixed order without LDS: the four rows of
// 16 lanes by DPP moves, then the row sums (lanes 0, 16, 32, 48) read out and added
// in row order.  The result is wave-uniform.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = lane_group_sum<16>(v);
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// Number of set lanes of a 64-bit ballot below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(ballot), 0));
}

}  // namespace tsa

namespace tsa {

// Workgroups of a 1-D grid are dispatched round-robin over the 8 XCDs of the
// chip (block b runs on XCD b % 8).  Remap block ids so that each XCD works on
// one contiguous range of logical tiles: tiles that share inputs (e.g. the
// query tiles of one head, which all stream that head's K/V) then share the
// XCD's L2.  The mapping is a bijection on [0, total).
__device__ __forceinline__ long xcd_remap(long b, long total) {
  constexpr long kXcd = 8;
  const long q = total / kXcd, r = total % kXcd;
  const long xcd = b % kXcd, slot = b / kXcd;
  return xcd * q + (xcd < r ? xcd : r) + slot;
}

}  // namespace tsa
