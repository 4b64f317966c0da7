// f4: Timeripple partial-score reuse on Q or K (Timeripple page, Metodología §1-§2).
//
// A head's channels form the three rotary groups time / height / width (sizes
// d - 4*(d/6), 2*(d/6), 2*(d/6)).  Moving along one axis leaves the rotary phase
// of the other two groups unchanged, so those channels of neighbouring tokens
// tend to agree.  For every token, head and axis:
//
//   delta[n,h,a] = ||v[n,h,C_a] - v[nb_a(n),h,C_a]|| / ||v[n,h,C_a]||
//
// over C_a = the channels of the two groups axis a does not rotate, nb_a the
// token one step back along a (one frame, row or column); no neighbour: +inf.
// Group g of the token then reuses the partial scores of the neighbour along the
// first axis a != g (order time, height, width) whose delta is below theta_a,
// which is the same as taking the group's channels from that neighbour's own
// (resolved) vector.  The attention of the resulting effective vectors is the
// attention with reused partial scores.
//
// Three kernels, each a flat pass:
//   delta_src: L = d/8 lanes per (token, head), 16-byte slices, sums by DPP lane moves;
//   resolve:   one thread per (token, head, group) follows the sources back to the
//              token that computes the group itself (every step moves back along
//              an axis, so a chain is at most frame + row + column steps long);
//   copy:      one wave per token writes its effective row in 16-byte chunks.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace tsa {

struct ReuseGeom {
  long n;
  int heads;
  long hw;     // tokens per frame
  long width;  // tokens per row
  int d_t;     // channels of the time group; the height group follows with d_s, then width
  int d_s;
};

__device__ __forceinline__ int channel_group(const ReuseGeom& g, int c) {
  return c < g.d_t ? 0 : (c < g.d_t + g.d_s ? 1 : 2);
}

// The tokens one step back along each axis (time, height, width), -1 where there is
// none.  Token indices fit 31 bits (the ABI checks), so the divisions are 32-bit ones.
__device__ __forceinline__ void axis_back3(const ReuseGeom& g, uint32_t t, long nb[3]) {
  const uint32_t hw = static_cast<uint32_t>(g.hw), w = static_cast<uint32_t>(g.width);
  const uint32_t in_frame = t % hw;
  nb[0] = t >= hw ? static_cast<long>(t - hw) : -1;
  nb[1] = in_frame >= w ? static_cast<long>(t - w) : -1;
  nb[2] = in_frame % w ? static_cast<long>(t) - 1 : -1;
}

template <int HD>
__global__ __launch_bounds__(256) void reuse_delta_src_kernel(const uint16_t* __restrict__ v, ReuseGeom geo,
                                                              float th0, float th1, float th2,
                                                              int* __restrict__ src, int* __restrict__ src_copy,
                                                              float* __restrict__ delta_out) {
  constexpr int L = HD / 8;  // lanes per (token, head), 8 channels each
  // (token, head) pairs fit 31 bits: n * heads * 3 < 2^31 (the ABI checks); the thread
  // index itself may not, so the pair is formed from the block index in 64 bits
  const uint32_t pair = static_cast<uint32_t>(static_cast<uint64_t>(blockIdx.x) * (256 / L) + threadIdx.x / L);
  const int sub = threadIdx.x % L;
  const uint32_t heads = static_cast<uint32_t>(geo.heads);
  const bool live = pair < static_cast<uint32_t>(geo.n * geo.heads);
  const uint32_t t = live ? pair / heads : 0u;
  const int h = live ? static_cast<int>(pair - t * heads) : 0;  // dead lanes read row 0, head 0
  const long dim = static_cast<long>(geo.heads) * HD;
  const long col = static_cast<long>(h) * HD + 8 * sub;
  const long tl = t;

  long nb[3];
  axis_back3(geo, t, nb);
  if (!live) nb[0] = nb[1] = nb[2] = -1;
  // all four rows in flight before any is used
  u32x4 raw[4];
  raw[0] = *reinterpret_cast<const u32x4*>(v + tl * dim + col);
#pragma unroll
  for (int a = 0; a < 3; ++a) raw[1 + a] = *reinterpret_cast<const u32x4*>(v + (nb[a] >= 0 ? nb[a] : tl) * dim + col);
  float own[8];
  unpack8(raw[0], own);
  int grp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) grp[e] = channel_group(geo, 8 * sub + e);

  float num[3], den[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    float w[8];
    unpack8(raw[1 + a], w);
    float s_num = 0.f, s_den = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (grp[e] != a) {
        const float dv = own[e] - w[e];
        s_num = fmaf(dv, dv, s_num);
        s_den = fmaf(own[e], own[e], s_den);
      }
    }
    // sum over the L lanes of this (token, head)
    static_assert(L == 8 || L == 16, "lane groups of 8 or 16");
    num[a] = lane_group_sum<L>(s_num);
    den[a] = lane_group_sum<L>(s_den);
  }
  if (!live || sub != 0) return;
  const float theta[3] = {th0, th1, th2};
  float delta[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    if (nb[a] < 0)
      delta[a] = __builtin_inff();
    else if (den[a] == 0.f)
      delta[a] = num[a] == 0.f ? 0.f : __builtin_inff();
    else
      delta[a] = sqrtf(num[a]) / sqrtf(den[a]);
  }
  const long base = static_cast<long>(pair) * 3;
#pragma unroll
  for (int gi = 0; gi < 3; ++gi) {
    long from = tl;
#pragma unroll
    for (int a = 2; a >= 0; --a)  // the first qualifying axis in time, height, width order wins
      if (a != gi && delta[a] < theta[a]) from = nb[a];
    src[base + gi] = static_cast<int>(from);
    if (src_copy) src_copy[base + gi] = static_cast<int>(from);
    if (delta_out) delta_out[base + gi] = delta[gi];
  }
}

// root[(t*heads + h)*3 + g] = the token whose own channels group g of token t ends up with.
__global__ __launch_bounds__(256) void reuse_resolve_kernel(const int* __restrict__ src, long n_entries,
                                                            int heads, int* __restrict__ root) {
  // entries fit 31 bits (the ABI checks n * heads * 3 < 2^31)
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= static_cast<uint64_t>(n_entries)) return;
  const uint32_t per_token = 3u * static_cast<uint32_t>(heads);
  const uint32_t s0 = i / per_token;
  const uint32_t hg = i - s0 * per_token;  // (head, group) part of the entry index
  uint32_t s = s0;
  uint32_t nx = static_cast<uint32_t>(src[i]);
  // sources strictly precede their tokens: at most s0 steps
  for (uint32_t it = 0; nx != s && it <= s0; ++it) {
    s = nx;
    nx = static_cast<uint32_t>(src[s * per_token + hg]);
  }
  root[i] = static_cast<int>(s);
}

// eff[t, chunk c] = the 8 channels of chunk c, each taken from the resolved token of
// its group.  One wave per token, 16-byte chunks; a chunk crosses at most one group
// bound (groups are at least 20 channels wide), and bounds are even, so a chunk
// that straddles one is blended from two rows in 4-byte channel pairs.
template <int HD>
__global__ __launch_bounds__(256) void reuse_copy_kernel(const u32x4* __restrict__ v, const int* __restrict__ root,
                                                         ReuseGeom geo, u32x4* __restrict__ eff) {
  constexpr int CPH = HD / 8;  // chunks per head
  const long t = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= geo.n) return;
  const int lane = threadIdx.x & 63;
  const int chunks = geo.heads * CPH;
  const int* rt = root + t * geo.heads * 3;
  for (int c = lane; c < chunks; c += 64) {
    const int h = c / CPH;
    const int c0 = 8 * (c - h * CPH);  // first channel of the chunk within its head
    const int g0 = channel_group(geo, c0), g1 = channel_group(geo, c0 + 7);
    const long r0 = rt[h * 3 + g0];
    u32x4 val = v[r0 * chunks + c];
    if (g1 != g0) {
      const long r1 = rt[h * 3 + g1];
      if (r1 != r0) {
        const u32x4 w = v[r1 * chunks + c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (channel_group(geo, c0 + 2 * i) == g1) val[i] = w[i];
      }
    }
    eff[t * chunks + c] = val;
  }
}

hipError_t launch_reuse(const uint16_t* v, long n, int heads, int head_dim, long height, long width,
                        const float theta[3], uint16_t* eff, int* src_out, float* delta_out, int* ws_src,
                        int* ws_root, hipStream_t s) {
  ReuseGeom geo;
  geo.n = n;
  geo.heads = heads;
  geo.hw = height * width;
  geo.width = width;
  geo.d_s = 2 * (head_dim / 6);
  geo.d_t = head_dim - 2 * geo.d_s;
  const long pairs = n * heads;
  if (head_dim == 128) {
    const long threads = pairs * 16;
    hipLaunchKernelGGL(reuse_delta_src_kernel<128>, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256),
                       0, s, v, geo, theta[0], theta[1], theta[2], ws_src, src_out, delta_out);
  } else {
    const long threads = pairs * 8;
    hipLaunchKernelGGL(reuse_delta_src_kernel<64>, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256),
                       0, s, v, geo, theta[0], theta[1], theta[2], ws_src, src_out, delta_out);
  }
  const long entries = pairs * 3;
  hipLaunchKernelGGL(reuse_resolve_kernel, dim3(static_cast<unsigned>((entries + 255) / 256)), dim3(256), 0, s,
                     ws_src, entries, heads, ws_root);
  const dim3 copy_grid(static_cast<unsigned>((n + 3) / 4));
  if (head_dim == 128)
    hipLaunchKernelGGL(reuse_copy_kernel<128>, copy_grid, dim3(256), 0, s, reinterpret_cast<const u32x4*>(v), ws_root,
                       geo, reinterpret_cast<u32x4*>(eff));
  else
    hipLaunchKernelGGL(reuse_copy_kernel<64>, copy_grid, dim3(256), 0, s, reinterpret_cast<const u32x4*>(v), ws_root,
                       geo, reinterpret_cast<u32x4*>(eff));
  return hipGetLastError();
}

}  // namespace tsa
