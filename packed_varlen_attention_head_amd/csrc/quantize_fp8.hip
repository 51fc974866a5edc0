// bf16 -> OCP FP8 E4M3 ("fn") codes, round to nearest even, saturating at
// +-448: the operands of the low-precision attention's score product (the
// pages' GB10 builds quantise Q and K for SageAttention / Comfy Kitchen's
// INT8 attention; h3-spark model card, runtime options).
//
// HBM-bound elementwise pass: each thread converts 8 consecutive elements
// (16 bytes in, 8 bytes out) with the hardware packed conversion, after
// clamping finite and infinite values to the largest finite magnitude so
// nothing overflows to NaN; a NaN input stays NaN (an E4M3 NaN code).
#include <cstdint>

#include "common.h"

namespace h3a {
namespace {

constexpr int kThreads = 256;

// Saturate to +-448 before the E4M3 conversion; NaN passes through unchanged
// (fminf/fmaxf alone would turn it into -448).
__device__ __forceinline__ float e4m3_sat(float x) { return x != x ? x : fminf(fmaxf(x, -448.0f), 448.0f); }

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
    for (int e = 0; e < 4; ++e) f[e] = e4m3_sat(f[e]);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], packed, true);
    out[i] = uint32_t(packed);
  }
  *reinterpret_cast<uint2*>(y + token * sy + vec * 8) = make_uint2(out[0], out[1]);
}

// ---- V as transposed E4M3 tiles -------------------------------------------
// vt[h][d][col] (one byte per code, row stride vt_cols): column col0(s) + i
// holds key i of segment s, where every segment is padded to whole 64-key
// tiles (col0 = the padded lengths of the earlier segments) and padding
// columns hold code 0.  A workgroup transposes one 64-column tile of one
// head through LDS: each thread converts 8 dims x 4 tokens and stores them
// as 8 dwords (4 tokens per dword); rows are padded to 68 bytes so the 16
// chunk-lanes of a store land on different banks.
constexpr int kVtMaxSegs = 64;
constexpr int kVtPitch = 68;

struct VtArgs {
  int32_t nseg;
  int32_t tile0;                 // first column tile of this launch
  int32_t start[kVtMaxSegs];     // token index of the segment's first key
  int32_t len[kVtMaxSegs];
  int32_t tiles[kVtMaxSegs + 1]; // prefix sums of the segments' tile counts (from tile0)
};

template <int D>
__global__ void __launch_bounds__(kThreads)
prepare_vt_e4m3_kernel(VtArgs a, const uint16_t* __restrict__ v, int64_t sv, uint8_t* __restrict__ vt,
                       int64_t vt_cols) {
  static_assert(D / 8 * 16 == kThreads || D / 8 * 16 == kThreads / 2, "one (chunk, 4-token group) per thread");
  __shared__ uint32_t tile[D * kVtPitch / 4];
  const int tau = blockIdx.x;  // tile within this launch
  const int h = blockIdx.y;
  int s = 0;
  while (s + 1 < a.nseg && tau >= a.tiles[s + 1]) ++s;
  const int key0 = (tau - a.tiles[s]) * kVtTile;
  const int t = threadIdx.x;
  constexpr int CH = D / 8;  // 8-dim chunks per row
  for (int u = t; u < CH * 16; u += kThreads) {
    const int c = u % CH, g = u / CH;  // chunk of dims, group of 4 tokens
    uint32_t w[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 4 * g + i;
      uint4 r = make_uint4(0, 0, 0, 0);
      if (key < a.len[s]) r = *reinterpret_cast<const uint4*>(v + int64_t(a.start[s] + key) * sv + h * D + c * 8);
      w[i][0] = r.x; w[i][1] = r.y; w[i][2] = r.z; w[i][3] = r.w;
    }
    // dim 8c + e of the 4 tokens -> one dword (byte i = token 4g + i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = w[i][e / 2];
        f[i] = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
        f[i] = e4m3_sat(f[i]);
      }
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], packed, true);
      tile[((8 * c + e) * kVtPitch) / 4 + g] = uint32_t(packed);
    }
  }
  __syncthreads();
  const int64_t col = int64_t(a.tile0 + tau) * kVtTile;
  for (int u = t; u < D * 4; u += kThreads) {
    const int row = u / 4, part = u % 4;  // 16-byte part of the 64-byte row
    const uint32_t* src = tile + (row * kVtPitch) / 4 + part * 4;
    *reinterpret_cast<uint4*>(vt + (int64_t(h) * D + row) * vt_cols + col + part * 16) =
        make_uint4(src[0], src[1], src[2], src[3]);
  }
}

}  // namespace

int64_t vt_e4m3_columns(const int32_t* cu, int32_t nseg) {
  int64_t cols = 0;
  for (int32_t s = 0; s < nseg; ++s) cols += (int64_t(cu[s + 1] - cu[s]) + kVtTile - 1) / kVtTile * kVtTile;
  return cols;
}

hipError_t launch_prepare_vt_e4m3(const void* v, int64_t sv, const int32_t* cu, int32_t nseg, int32_t H, int32_t D,
                                  void* vt, int64_t vt_cols, hipStream_t stream) {
  int32_t tile0 = 0;
  for (int32_t s0 = 0; s0 < nseg; s0 += kVtMaxSegs) {
    const int32_t n = nseg - s0 < kVtMaxSegs ? nseg - s0 : kVtMaxSegs;
    VtArgs a{};
    a.nseg = n;
    a.tile0 = tile0;
    a.tiles[0] = 0;
    for (int32_t i = 0; i < n; ++i) {
      a.start[i] = cu[s0 + i];
      a.len[i] = cu[s0 + i + 1] - cu[s0 + i];
      a.tiles[i + 1] = a.tiles[i] + (a.len[i] + kVtTile - 1) / kVtTile;
    }
    const int32_t ntiles = a.tiles[n];
    if (ntiles > 0) {
      const dim3 grid{unsigned(ntiles), unsigned(H), 1u};
      if (D == 128)
        hipLaunchKernelGGL(prepare_vt_e4m3_kernel<128>, grid, dim3(kThreads), 0, stream, a,
                           static_cast<const uint16_t*>(v), sv, static_cast<uint8_t*>(vt), vt_cols);
      else if (D == 64)
        hipLaunchKernelGGL(prepare_vt_e4m3_kernel<64>, grid, dim3(kThreads), 0, stream, a,
                           static_cast<const uint16_t*>(v), sv, static_cast<uint8_t*>(vt), vt_cols);
      else
        return hipErrorInvalidValue;
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    tile0 += ntiles;
  }
  return hipSuccess;
}

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
