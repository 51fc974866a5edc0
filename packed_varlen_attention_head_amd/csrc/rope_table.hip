// Packed 3D rotary table: token positions from per-segment (T, H, W) grids
// and fp64 angles, rounded once to fp32 cos/sin.
//
// The DiT's position grid is fp64 because it feeds the rotary (vllm.cpp PR
// #26, opening commit), and its 3D rotary is plain NeoX rotate-half fed by a
// per-row cos/sin cache with angles from the t, h and w axes (same PR,
// description, "The device-resident forward (W2b)").  The table is
// step-invariant: it is built once per request.
//
// Four ways to get a token's per-axis coordinate p_a from its grid index i_a
// (extent n_a) -- the table modes of include/h3a.h:
//   grid         p = i
//   linspace     p = i * step_a + start_a, step_a = (stop_a - start_a) / n_a
//                (numpy.linspace(endpoint=False) order, which the DiT's fp64
//                grid follows bit for bit: PR #26 description, "Correctness
//                gates")
//   normalized   p = 2 pi (2 ((i + 0.5) / n) - 1); tokens past T*H*W (the
//                ViT3D decoder's register and cls suffix) get angle 0
//                (video-VAE decoder commit, "3D ROPE DETAIL")
//   interleaved  p = i on the axis the host assigned to each angle
//                (M-RoPE's [t h w t h w ...]; encoder-tower commit)
// and angle j = p_axis(j) * inv_freq[j], with the frequency ladder and the
// axis of each angle set on the host.  Floating-point contraction is off so
// the fp64 positions are the exact IEEE results of those expressions.
//
// One thread per (token, angle).  Segment descriptors travel in the kernel
// arguments, kMaxSegs per launch (an argument block under 1 KiB), so no
// device staging buffer is needed.
#include <cstdint>

#include "common.h"

namespace h3a {
namespace {

constexpr int kMaxSegs = 16;
constexpr int kMaxHalf = 64;  // R/2 <= D/2 <= 64

struct RopeArgs {
  int32_t nseg;
  int32_t half;           // R / 2 angles per token
  int64_t S;              // rows of the cos and sin blocks
  int32_t mode;           // RopeMode
  int32_t start[kMaxSegs];
  int32_t len[kMaxSegs];
  int32_t gt[kMaxSegs];   // grid T
  int32_t gh[kMaxSegs];   // grid H
  int32_t gw[kMaxSegs];   // grid W
  double lin_start[3];
  double lin_stop[3];
  double inv_freq[kMaxHalf];
  int8_t axis[kMaxHalf];  // 0 = t, 1 = h, 2 = w
};
static_assert(sizeof(RopeArgs) <= 1024, "kernel argument block");

__global__ void __launch_bounds__(256) rope_table_kernel(RopeArgs a, float* __restrict__ cos_sin,
                                                          int32_t first_token, int32_t ntok) {
#pragma clang fp contract(off)
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(ntok) * a.half) return;
  // 32-bit division where the index fits (every practical table)
  int32_t tl, j;
  if (idx <= int64_t(INT32_MAX)) {
    tl = int32_t(idx) / a.half;
    j = int32_t(idx) - tl * a.half;
  } else {
    tl = int32_t(idx / a.half);
    j = int32_t(idx % a.half);
  }
  const int32_t token = first_token + tl;
  int s = 0;
  while (s + 1 < a.nseg && token >= a.start[s + 1]) ++s;
  const int32_t n = token - a.start[s];
  const int32_t hw = a.gh[s] * a.gw[s];
  const int ax = a.axis[j];
  const int32_t ext = ax == 0 ? a.gt[s] : (ax == 1 ? a.gh[s] : a.gw[s]);
  const int32_t i = ax == 0 ? n / hw : (ax == 1 ? (n / a.gw[s]) % a.gh[s] : n % a.gw[s]);
  double p;
  if (a.mode == kRopeLinspace) {
    // numpy.linspace's step, (stop - start) / n; IEEE division and product.
    const double step = (a.lin_stop[ax] - a.lin_start[ax]) / double(ext);
    p = double(i) * step + a.lin_start[ax];
  } else if (a.mode == kRopeNormalized) {
    p = (((double(i) + 0.5) / double(ext)) * 2.0 - 1.0) * (2.0 * 3.141592653589793);
    if (n >= a.gt[s] * hw) p = 0.0;  // suffix token: identity
  } else {
    p = double(i);
  }
  const double theta = p * a.inv_freq[j];
  const int64_t o = int64_t(token) * a.half + j;
  double sn, cs;
  sincos(theta, &sn, &cs);  // one shared range reduction
  cos_sin[o] = float(cs);
  cos_sin[a.S * a.half + o] = float(sn);
}

}  // namespace

hipError_t launch_rope_table(const RopeTableSpec& spec, const int32_t* segments, const int32_t* starts,
                             int32_t nseg, float* cos_sin, int64_t S, hipStream_t stream) {
  const int32_t half = spec.half;
  if (half <= 0 || half > kMaxHalf) return hipErrorInvalidValue;
  RopeArgs a{};
  a.half = half;
  a.S = S;
  a.mode = spec.mode;
  for (int i = 0; i < half; ++i) {
    a.inv_freq[i] = spec.inv_freq[i];
    a.axis[i] = int8_t(spec.axis_of[i]);
  }
  for (int ax = 0; ax < 3; ++ax) {
    a.lin_start[ax] = spec.lin_start[ax];
    a.lin_stop[ax] = spec.lin_stop[ax];
  }
  for (int32_t s0 = 0; s0 < nseg; s0 += kMaxSegs) {
    const int32_t n = nseg - s0 < kMaxSegs ? nseg - s0 : kMaxSegs;
    a.nseg = n;
    for (int i = 0; i < n; ++i) {
      const int32_t* g = segments + 4 * int64_t(s0 + i);
      a.start[i] = starts[s0 + i];
      a.gt[i] = g[0];
      a.gh[i] = g[1];
      a.gw[i] = g[2];
      a.len[i] = g[3];
    }
    const int32_t first = starts[s0];
    const int32_t ntok = starts[s0 + n - 1] + a.len[n - 1] - first;
    if (ntok == 0) continue;
    const int64_t threads = int64_t(ntok) * half;
    const unsigned blocks = unsigned((threads + 255) / 256);
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, stream, a, cos_sin, first,
                       ntok);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace h3a
