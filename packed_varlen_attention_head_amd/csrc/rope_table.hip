// Packed 3D rotary table: token positions from per-segment (T, H, W) grids
// and fp64 angles, rounded once to fp32 cos/sin.
//
// The DiT's position grid is fp64 because it feeds the rotary (vllm.cpp PR
// #26, opening commit), and its 3D rotary is plain NeoX rotate-half fed by a
// per-row cos/sin cache with angles from the t, h and w axes (same PR,
// description, "The device-resident forward (W2b)").  The table is
// step-invariant: it is built once per request.
//
// One thread per (token, angle).  Segment descriptors travel in the kernel
// arguments, kMaxSegs per launch, so no device staging buffer is needed.
#include <cstdint>

#include "common.h"

namespace h3a {
namespace {

constexpr int kMaxSegs = 32;
constexpr int kMaxHalf = 64;  // R/2 <= D/2 <= 64

struct RopeArgs {
  int32_t nseg;
  int32_t half;           // R / 2 angles per token
  int64_t S;              // rows of the cos and sin blocks
  int32_t start[kMaxSegs];
  int32_t len[kMaxSegs];
  int32_t gh[kMaxSegs];   // grid H
  int32_t gw[kMaxSegs];   // grid W
  double inv_freq[kMaxHalf];
  int32_t axis[kMaxHalf]; // 0 = t, 1 = h, 2 = w
};

__global__ void __launch_bounds__(256) rope_table_kernel(RopeArgs a, float* __restrict__ cos_sin,
                                                          int32_t first_token, int32_t ntok) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(ntok) * a.half) return;
  const int32_t token = first_token + int32_t(idx / a.half);
  const int32_t j = int32_t(idx % a.half);
  int s = 0;
  while (s + 1 < a.nseg && token >= a.start[s + 1]) ++s;
  const int32_t n = token - a.start[s];
  const int32_t hw = a.gh[s] * a.gw[s];
  const int32_t pos_t = n / hw;
  const int32_t pos_h = (n / a.gw[s]) % a.gh[s];
  const int32_t pos_w = n % a.gw[s];
  const int ax = a.axis[j];
  const int32_t p = ax == 0 ? pos_t : (ax == 1 ? pos_h : pos_w);
  const double theta = double(p) * a.inv_freq[j];
  const int64_t o = int64_t(token) * a.half + j;
  cos_sin[o] = float(cos(theta));
  cos_sin[a.S * a.half + o] = float(sin(theta));
}

}  // namespace

hipError_t launch_rope_table(const int32_t* segments, const int32_t* starts, int32_t nseg,
                             const double* inv_freq, const int32_t* axis_of, int32_t half,
                             float* cos_sin, int64_t S, hipStream_t stream) {
  if (half <= 0 || half > kMaxHalf) return hipErrorInvalidValue;
  RopeArgs a{};
  a.half = half;
  a.S = S;
  for (int i = 0; i < half; ++i) {
    a.inv_freq[i] = inv_freq[i];
    a.axis[i] = axis_of[i];
  }
  for (int32_t s0 = 0; s0 < nseg; s0 += kMaxSegs) {
    const int32_t n = nseg - s0 < kMaxSegs ? nseg - s0 : kMaxSegs;
    a.nseg = n;
    for (int i = 0; i < n; ++i) {
      a.start[i] = starts[s0 + i];
      a.len[i] = segments[4 * (s0 + i) + 3];
      a.gh[i] = segments[4 * (s0 + i) + 1];
      a.gw[i] = segments[4 * (s0 + i) + 2];
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
