// a4 / a6 / a8: row movers (HBM-bound).
//
// gather: dst[r] = row source of token rows[r] (plain copy, or the LIPAR
//   recovery row (1 - sigma) * x[t - off] + sigma * eps[t], LIPAR page §2.C).
// copy_rows2: dst[rows[r]] = src[r] for one or two buffers -- the KV-cache
//   overwrite of HSA page §2.2 item 2 and the scatter back to token order.
//
// One wave moves R rows in 16-byte lanes (a 256-thread block: 4R rows).  All
// loads of a pass (up to J slices per lane of each of the R rows, J sized to the
// row) are issued before its stores.  Copies of rows that fit one pass of 4
// slices per lane go two to a wave, so twice the bytes are in flight (gather and
// scatter of 9828 rows of 1536 bf16 with a flushed MALL: 14 against 17 us; the
// two-buffer cache sync 21.6 against 22.4 us over back-to-back launches on
// rotated inputs).  Copied sources are read with nontemporal loads (they are not
// read again); the plain gather also stores nontemporally (11.8 against 12.5 us;
// neutral for the scatter, slower for the two-buffer copy).
#include "common.h"
#include "kernels.h"

namespace tsa {

constexpr int kWavesPerBlock = 4;

template <bool RECOVER, int J, int R>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          long n_x_rows,
                                                          const int* __restrict__ rows,
                                                          const uint16_t* __restrict__ eps,
                                                          long src_off, float sigma, long n,
                                                          long dim, uint16_t* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const long r0 = (static_cast<long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6)) * R;
  if (r0 >= n) return;
  const long chunks = dim / 8;
  const float one_m_s = 1.0f - sigma;
  const u32x4* in[R];
  const u32x4* ne[R];
  u32x4* out[R];
  bool live[R], has_clean[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const long r = r0 + q;
    live[q] = r < n;
    const long t = !live[q] ? 0 : rows ? rows[r] : r;
    const long src = RECOVER ? t - src_off : t;
    has_clean[q] = !RECOVER || (src >= 0 && src < n_x_rows);
    in[q] = reinterpret_cast<const u32x4*>(x + (has_clean[q] ? src : 0) * dim);
    ne[q] = reinterpret_cast<const u32x4*>(RECOVER ? eps + t * dim : x);
    out[q] = reinterpret_cast<u32x4*>(dst + (live[q] ? r : 0) * dim);
  }
  for (long c0 = 0; c0 < chunks; c0 += 64 * J) {
    u32x4 bc[R][J], be[R][RECOVER ? J : 1];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (live[q] && c < chunks) {
          if (RECOVER) {  // plain loads: measured faster here than nontemporal ones
            bc[q][j] = has_clean[q] ? in[q][c] : u32x4{0u, 0u, 0u, 0u};
            be[q][j] = ne[q][c];
          } else {
            bc[q][j] = __builtin_nontemporal_load(in[q] + c);
          }
        }
      }
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (live[q] && c < chunks) {
          if (RECOVER)
            out[q][c] = recover8(bc[q][j], be[q][RECOVER ? j : 0], one_m_s, sigma);
          else
            __builtin_nontemporal_store(bc[q][j], out[q] + c);
        }
      }
  }
}

// dst_a[rows[r]] = a[r] (and dst_b[rows[r]] = b[r] when b is given).
template <bool TWO, int J, int R>
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint16_t* __restrict__ a,
                                                        const uint16_t* __restrict__ b,
                                                        const int* __restrict__ rows, long n,
                                                        uint16_t* __restrict__ da,
                                                        uint16_t* __restrict__ db, long dim) {
  const int lane = threadIdx.x & 63;
  const long r0 = (static_cast<long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6)) * R;
  if (r0 >= n) return;
  const long chunks = dim / 8;
  const u32x4* sa[R];
  const u32x4* sb[R];
  u32x4* oa[R];
  u32x4* ob[R];
  bool live[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const long r = r0 + q;
    live[q] = r < n;
    const long rr = live[q] ? r : 0;
    const long t = live[q] ? rows[r] : 0;
    sa[q] = reinterpret_cast<const u32x4*>(a + rr * dim);
    sb[q] = reinterpret_cast<const u32x4*>(TWO ? b + rr * dim : a);
    oa[q] = reinterpret_cast<u32x4*>(da + t * dim);
    ob[q] = reinterpret_cast<u32x4*>(TWO ? db + t * dim : da);
  }
  for (long c0 = 0; c0 < chunks; c0 += 64 * J) {
    u32x4 va[R][J], vb[R][TWO ? J : 1];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (live[q] && c < chunks) {
          va[q][j] = __builtin_nontemporal_load(sa[q] + c);
          if (TWO) vb[q][j] = __builtin_nontemporal_load(sb[q] + c);
        }
      }
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const long c = c0 + lane + 64 * j;
        if (live[q] && c < chunks) {
          oa[q][c] = va[q][j];
          if (TWO) ob[q][c] = vb[q][TWO ? j : 0];
        }
      }
  }
}

// Slices per lane and pass: enough for the whole row up to 8 (4096 bf16 columns).
static int slices_per_lane(long dim) {
  const long per_lane = (dim / 8 + 63) / 64;
  return per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : 8;
}

// The recovery rows (two sources, fp32 blend) keep one row per wave: two were
// measured slower there (24.2 against 22.5 us for 9828 rows of 1536).
template <int J, int R>
static void gather_j(const RowSource& src, long n, long dim, uint16_t* dst, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(src.x);
  if (src.eps) {
    const dim3 grid(static_cast<unsigned>((n + kWavesPerBlock - 1) / kWavesPerBlock));
    hipLaunchKernelGGL((gather_rows_kernel<true, J, 1>), grid, dim3(256), 0, s, x, src.n_x_rows, src.rows,
                       src.eps, src.src_off, src.sigma, n, dim, dst);
  } else {
    constexpr long rows_per_block = kWavesPerBlock * R;
    const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((gather_rows_kernel<false, J, R>), grid, dim3(256), 0, s, x, src.n_x_rows, src.rows,
                       src.eps, src.src_off, src.sigma, n, dim, dst);
  }
}

hipError_t launch_gather_rows(const RowSource& src, long n, long dim, uint16_t* dst,
                              hipStream_t s) {
  switch (slices_per_lane(dim)) {
    case 2: gather_j<2, 2>(src, n, dim, dst, s); break;
    case 4: gather_j<4, 2>(src, n, dim, dst, s); break;
    default: gather_j<8, 1>(src, n, dim, dst, s); break;
  }
  return hipGetLastError();
}

template <int J, int R>
static void copy_j(const uint16_t* a, const uint16_t* b, const int* rows, long n, uint16_t* da,
                   uint16_t* db, long dim, hipStream_t s) {
  // two buffers (the cache sync): R rows of each per wave as well
  if (b) {
    constexpr long rows_per_block = kWavesPerBlock * R;
    const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((copy_rows_kernel<true, J, R>), grid, dim3(256), 0, s, a, b, rows, n, da, db, dim);
  } else {
    constexpr long rows_per_block = kWavesPerBlock * R;
    const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((copy_rows_kernel<false, J, R>), grid, dim3(256), 0, s, a, b, rows, n, da, db, dim);
  }
}

hipError_t launch_copy_rows2(const uint16_t* a, const uint16_t* b, const int* rows, long n,
                             uint16_t* da, uint16_t* db, long dim, hipStream_t s) {
  switch (slices_per_lane(dim)) {
    case 2: copy_j<2, 2>(a, b, rows, n, da, db, dim, s); break;
    case 4: copy_j<4, 2>(a, b, rows, n, da, db, dim, s); break;
    default: copy_j<8, 1>(a, b, rows, n, da, db, dim, s); break;
  }
  return hipGetLastError();
}

}  // namespace tsa
