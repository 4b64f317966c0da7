// a4 / a6 / a8: row movers (HBM-bound).
//
// gather: dst[r] = row source of token rows[r] (plain copy, or the LIPAR
//   recovery row (1 - sigma) * x[t - off] + sigma * eps[t], LIPAR page §2.C).
// copy_rows2: dst[rows[r]] = src[r] for one or two buffers -- the KV-cache
//   overwrite of HSA page §2.2 item 2 and the scatter back to token order.
//
// One wave moves one row in 16-byte lanes; a 256-thread block handles four
// rows.  All loads of a row (up to J slices per lane, J sized to the row) are
// issued before its stores.
#include "common.h"
#include "kernels.h"

namespace tsa {

constexpr int kRowsPerBlock = 4;

template <bool RECOVER, int J>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          long n_x_rows,
                                                          const int* __restrict__ rows,
                                                          const uint16_t* __restrict__ eps,
                                                          long src_off, float sigma, long n,
                                                          long dim, uint16_t* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const long r = static_cast<long>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= n) return;
  const long t = rows ? rows[r] : r;
  const long chunks = dim / 8;
  u32x4* out = reinterpret_cast<u32x4*>(dst + r * dim);
  if (!RECOVER) {
    const u32x4* in = reinterpret_cast<const u32x4*>(x + t * dim);
    for (long c0 = 0; c0 < chunks; c0 += 64 * J) {
      u32x4 buf[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (c < chunks) buf[j] = __builtin_nontemporal_load(in + c);
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (c < chunks) out[c] = buf[j];
      }
    }
  } else {
    const long src = t - src_off;
    const bool has_clean = src >= 0 && src < n_x_rows;
    const u32x4* in = reinterpret_cast<const u32x4*>(x + (has_clean ? src : 0) * dim);
    const u32x4* ne = reinterpret_cast<const u32x4*>(eps + t * dim);
    const float one_m_s = 1.0f - sigma;
    for (long c0 = 0; c0 < chunks; c0 += 64 * J) {
      u32x4 bc[J], be[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (c < chunks) {
          bc[j] = has_clean ? in[c] : u32x4{0u, 0u, 0u, 0u};
          be[j] = ne[c];
        }
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (c < chunks) out[c] = recover8(bc[j], be[j], one_m_s, sigma);
      }
    }
  }
}

// dst_a[rows[r]] = a[r] (and dst_b[rows[r]] = b[r] when b is given).
template <bool TWO, int J>
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint16_t* __restrict__ a,
                                                        const uint16_t* __restrict__ b,
                                                        const int* __restrict__ rows, long n,
                                                        uint16_t* __restrict__ da,
                                                        uint16_t* __restrict__ db, long dim) {
  const int lane = threadIdx.x & 63;
  const long r = static_cast<long>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= n) return;
  const long t = rows[r];
  const long chunks = dim / 8;
  const u32x4* sa = reinterpret_cast<const u32x4*>(a + r * dim);
  const u32x4* sb = reinterpret_cast<const u32x4*>(TWO ? b + r * dim : a);
  u32x4* oa = reinterpret_cast<u32x4*>(da + t * dim);
  u32x4* ob = reinterpret_cast<u32x4*>(TWO ? db + t * dim : da);
  for (long c0 = 0; c0 < chunks; c0 += 64 * J) {
    u32x4 va[J], vb[TWO ? J : 1];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const long c = c0 + lane + 64 * j;
      if (c < chunks) {
        va[j] = __builtin_nontemporal_load(sa + c);
        if (TWO) vb[j] = __builtin_nontemporal_load(sb + c);
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const long c = c0 + lane + 64 * j;
      if (c < chunks) {
        oa[c] = va[j];
        if (TWO) ob[c] = vb[j];
      }
    }
  }
}

// Slices per lane and pass: enough for the whole row up to 8 (4096 bf16 columns).
static int slices_per_lane(long dim) {
  const long per_lane = (dim / 8 + 63) / 64;
  return per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : 8;
}

template <int J>
static void gather_j(const RowSource& src, long n, long dim, uint16_t* dst, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((n + kRowsPerBlock - 1) / kRowsPerBlock));
  const uint16_t* x = static_cast<const uint16_t*>(src.x);
  if (src.eps)
    hipLaunchKernelGGL((gather_rows_kernel<true, J>), grid, dim3(256), 0, s, x, src.n_x_rows, src.rows,
                       src.eps, src.src_off, src.sigma, n, dim, dst);
  else
    hipLaunchKernelGGL((gather_rows_kernel<false, J>), grid, dim3(256), 0, s, x, src.n_x_rows, src.rows,
                       src.eps, src.src_off, src.sigma, n, dim, dst);
}

hipError_t launch_gather_rows(const RowSource& src, long n, long dim, uint16_t* dst,
                              hipStream_t s) {
  switch (slices_per_lane(dim)) {
    case 2: gather_j<2>(src, n, dim, dst, s); break;
    case 4: gather_j<4>(src, n, dim, dst, s); break;
    default: gather_j<8>(src, n, dim, dst, s); break;
  }
  return hipGetLastError();
}

template <int J>
static void copy_j(const uint16_t* a, const uint16_t* b, const int* rows, long n, uint16_t* da,
                   uint16_t* db, long dim, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((n + kRowsPerBlock - 1) / kRowsPerBlock));
  if (b)
    hipLaunchKernelGGL((copy_rows_kernel<true, J>), grid, dim3(256), 0, s, a, b, rows, n, da, db, dim);
  else
    hipLaunchKernelGGL((copy_rows_kernel<false, J>), grid, dim3(256), 0, s, a, b, rows, n, da, db, dim);
}

hipError_t launch_copy_rows2(const uint16_t* a, const uint16_t* b, const int* rows, long n,
                             uint16_t* da, uint16_t* db, long dim, hipStream_t s) {
  switch (slices_per_lane(dim)) {
    case 2: copy_j<2>(a, b, rows, n, da, db, dim, s); break;
    case 4: copy_j<4>(a, b, rows, n, da, db, dim, s); break;
    default: copy_j<8>(a, b, rows, n, da, db, dim, s); break;
  }
  return hipGetLastError();
}

}  // namespace tsa
