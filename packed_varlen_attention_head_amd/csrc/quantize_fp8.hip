// bf16 -> OCP FP8 E4M3 ("fn") codes, round to nearest even, saturating at
// +-448: the operands of the low-precision attention's score product (the
// pages' GB10 builds quantise Q and K for SageAttention / Comfy Kitchen's
// INT8 attention; h3-spark model card, runtime options).
//
// HBM-bound elementwise pass: each thread converts 8 consecutive elements
// (16 bytes in, 8 bytes out) with the hardware packed conversion, after
// clamping to the largest finite value so nothing overflows to NaN.
#include <cstdint>

#include "common.h"

namespace h3a {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
quantize_e4m3_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ y, int64_t S, int32_t row_vecs,
                     int64_t sx, int64_t sy) {
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= S * row_vecs) return;
  const int64_t token = idx / row_vecs;
  const int32_t vec = int32_t(idx % row_vecs);
  const uint4 r = *reinterpret_cast<const uint4*>(x + token * sx + vec * 8);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  uint32_t out[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float f[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f[2 * j] = __uint_as_float(w[2 * i + j] << 16);
      f[2 * j + 1] = __uint_as_float(w[2 * i + j] & 0xffff0000u);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = fminf(fmaxf(f[e], -448.0f), 448.0f);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], packed, true);
    out[i] = uint32_t(packed);
  }
  *reinterpret_cast<uint2*>(y + token * sy + vec * 8) = make_uint2(out[0], out[1]);
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* x, void* y, int64_t S, int32_t row_elems, int64_t sx, int64_t sy,
                                hipStream_t stream) {
  if (S <= 0) return hipSuccess;
  const int32_t row_vecs = row_elems / 8;
  const int64_t n = S * row_vecs;
  const unsigned blocks = unsigned((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<uint8_t*>(y), S, row_vecs, sx, sy);
  return hipGetLastError();
}

}  // namespace h3a
