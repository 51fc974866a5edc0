// bf16 -> OCP FP8 E4M3 ("fn") codes with one power-of-two scale per block of
// 32 elements along the contraction (mx_scale.h): the operands of the
// low-precision attention (the pages' GB10 builds quantise Q, K and V per
// block for SageAttention / Comfy Kitchen's INT8 attention; h3-spark model
// card, runtime options and "What this config does").
//
// HBM-bound elementwise pass: each thread converts 8 consecutive elements
// (16 bytes in, 8 bytes out) with the hardware packed conversion, four lanes
// sharing a block's largest magnitude through two lane exchanges.  Scaled
// values never exceed 448; infinities saturate to +-448 * 2^X and a NaN
// input stays NaN (an E4M3 NaN code).
#include <cstdint>

#include "common.h"
#include "mx_scale.h"

namespace h3a {
namespace {

constexpr int kThreads = 256;

// row_vecs (8-element vectors per token) is a multiple of 4, so the four
// lanes of a block are consecutive and exit together at the end.  Scales are
// head-major: ys[h][token][b] for block b of head h (d32 blocks per head).
__global__ void __launch_bounds__(kThreads)
quantize_e4m3_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ y, uint8_t* __restrict__ ys,
                     int64_t S, int32_t row_vecs, int32_t d32, int64_t sx, int64_t sy) {
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= S * row_vecs) return;
  const int64_t token = idx / row_vecs;
  const int32_t vec = int32_t(idx % row_vecs);
  const uint4 r = *reinterpret_cast<const uint4*>(x + token * sx + vec * 8);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  float f[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    amax = abs_max(abs_max(amax, f[2 * i]), f[2 * i + 1]);
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int X = mx_exponent(amax);
  const float inv = mx_inv_scale(X);
  uint32_t out[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(f[4 * i] * inv), e4m3_sat(f[4 * i + 1] * inv), 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(f[4 * i + 2] * inv), e4m3_sat(f[4 * i + 3] * inv), packed, true);
    out[i] = uint32_t(packed);
  }
  *reinterpret_cast<uint2*>(y + token * sy + vec * 8) = make_uint2(out[0], out[1]);
  if ((vec & 3) == 0) {
    const int32_t blk = vec / 4, h = blk / d32;
    ys[(int64_t(h) * S + token) * d32 + blk % d32] = uint8_t(X + 127);
  }
}

// ---- V as transposed E4M3 tiles -------------------------------------------
// vt[h][d][col] (one byte per code, row stride vt_cols): column col0(s) + i
// holds key i of segment s, where every segment is padded to whole 64-key
// tiles (col0 = the padded lengths of the earlier segments) and padding
// columns hold code 0.  Each head dim's 32-key blocks (two per tile, aligned
// at the segment start) share one scale; vs[h][tile][j][r][b] holds the E8M0
// code of dim 32 b + r, key block j of that tile, so the attention's lane
// (r, j) reads its D / 32 scales as one word.  A workgroup transposes one
// 64-column tile of one head through LDS: each thread loads 8 dims x 4
// tokens, the block maxima meet in LDS (an atomic max on the non-negative
// fp32 bits), then each thread converts its values and stores them as 8
// dwords (4 tokens per dword); rows are padded to 68 bytes so the 16
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
                       uint8_t* __restrict__ vs, int64_t vt_cols) {
  static_assert(D / 8 * 16 == kThreads || D / 8 * 16 == kThreads / 2, "one (chunk, 4-token group) per thread");
  __shared__ uint32_t tile[D * kVtPitch / 4];
  __shared__ uint32_t amax_bits[D * 2];  // [dim][key block]
  const int tau = blockIdx.x;  // tile within this launch
  const int h = blockIdx.y;
  int s = 0;
  while (s + 1 < a.nseg && tau >= a.tiles[s + 1]) ++s;
  const int key0 = (tau - a.tiles[s]) * kVtTile;
  const int t = threadIdx.x;
  constexpr int CH = D / 8;  // 8-dim chunks per row
  for (int u = t; u < D * 2; u += kThreads) amax_bits[u] = 0u;
  // one (chunk of 8 dims, group of 4 tokens) per thread, at most
  const bool has = t < CH * 16;
  const int c = t % CH, g = t / CH;
  float f[8][4];
  if (has) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 4 * g + i;
      uint4 r = make_uint4(0, 0, 0, 0);
      if (key < a.len[s]) r = *reinterpret_cast<const uint4*>(v + int64_t(a.start[s] + key) * sv + h * D + c * 8);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e][i] = __uint_as_float((e & 1) ? (w[e / 2] & 0xffff0000u) : (w[e / 2] << 16));
    }
  }
  __syncthreads();  // amax_bits cleared
  if (has)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float m = abs_max(abs_max(abs_max(abs_max(0.f, f[e][0]), f[e][1]), f[e][2]), f[e][3]);
      atomicMax(&amax_bits[(8 * c + e) * 2 + g / 8], __float_as_uint(m));
    }
  __syncthreads();
  if (has)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dim 8c + e of the 4 tokens -> one dword (byte i = token 4g + i)
      const float inv = mx_inv_scale(mx_exponent(__uint_as_float(amax_bits[(8 * c + e) * 2 + g / 8])));
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(f[e][0] * inv), e4m3_sat(f[e][1] * inv), 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(f[e][2] * inv), e4m3_sat(f[e][3] * inv), packed, true);
      tile[((8 * c + e) * kVtPitch) / 4 + g] = uint32_t(packed);
    }
  // scales: thread (j, r) writes the D / 32 codes of dims r, 32 + r, ...
  const int64_t gtile = int64_t(a.tile0 + tau);
  if (t < 64) {
    const int j = t / 32, r = t % 32;
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
      word |= uint32_t(mx_exponent(__uint_as_float(amax_bits[(32 * b + r) * 2 + j])) + 127) << (8 * b);
    uint8_t* dst = vs + ((int64_t(h) * (vt_cols / kVtTile) + gtile) * 64 + t) * (D / 32);
    if constexpr (D == 128) *reinterpret_cast<uint32_t*>(dst) = word;
    else *reinterpret_cast<uint16_t*>(dst) = uint16_t(word);
  }
  __syncthreads();
  const int64_t col = gtile * kVtTile;
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
                                  void* vt, void* vs, int64_t vt_cols, hipStream_t stream) {
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
                           static_cast<const uint16_t*>(v), sv, static_cast<uint8_t*>(vt),
                           static_cast<uint8_t*>(vs), vt_cols);
      else if (D == 64)
        hipLaunchKernelGGL(prepare_vt_e4m3_kernel<64>, grid, dim3(kThreads), 0, stream, a,
                           static_cast<const uint16_t*>(v), sv, static_cast<uint8_t*>(vt),
                           static_cast<uint8_t*>(vs), vt_cols);
      else
        return hipErrorInvalidValue;
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    tile0 += ntiles;
  }
  return hipSuccess;
}

hipError_t launch_quantize_e4m3(const void* x, void* y, void* ys, int64_t S, int32_t H, int32_t D, int64_t sx,
                                int64_t sy, hipStream_t stream) {
  if (S <= 0) return hipSuccess;
  if (D % 32 != 0 || H < 1) return hipErrorInvalidValue;
  const int32_t row_elems = H * D;
  const int32_t row_vecs = row_elems / 8;
  const int64_t n = S * row_vecs;
  const unsigned blocks = unsigned((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<uint8_t*>(y), static_cast<uint8_t*>(ys), S,
                     row_vecs, D / 32, sx, sy);
  return hipGetLastError();
}

}  // namespace h3a
