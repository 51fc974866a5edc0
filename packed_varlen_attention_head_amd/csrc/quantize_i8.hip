// bf16 -> INT8 codes with fp32 scales for the INT8 score product: q with one
// scale per token and head, k with one per block of 64 keys of a segment and
// head (the pages' GB10 image runs INT8 Q/K attention -- Comfy Kitchen's
// kernel, a Sol-Attn INT8 QK switch, the fused "Sage Q-INT8" tail of the Q
// norm + rotary pass; H3 Blackwell Runtime README, attention backends;
// h3-spark model card, "What this config does").
//
// With amax a block's largest magnitude (fp32): scale = amax / 127 and code =
// rint(x * (127 / amax)) clamped to [-127, 127], both divisions correctly
// rounded, the product a plain fp32 multiply.  A zero block has scale 0 and
// codes 0.  amax is NaN when the block holds a NaN and infinite when it holds
// an infinity; then every code of the block is 0 and its scale NaN or
// infinite, so the scores the block enters become NaN.
//
// HBM-bound elementwise passes: a token row is read once (16 bytes a lane)
// and its codes written once (8 bytes a lane).
//
// Centred keys (SageAttention's K smoothing, among the same backends): the
// key quantiser can subtract each segment's mean key (per head and dim, fp32)
// first; within a softmax every score then moves by the same q . mean, which
// the softmax cancels.  The means come from two deterministic passes: sums of
// 256-key chunks (aligned at each segment's start) in a fixed order, then each
// segment's chunk sums in chunk order, divided by its length.
#include <cstdint>

#include "common.h"

namespace h3a {
namespace {

constexpr int kThreads = 256;

// The larger magnitude of a and b, a NaN kept (fmaxf would drop it):
// magnitudes compare as their bit patterns with the sign cleared, every NaN
// above +inf, with no branch.
__device__ __forceinline__ float nan_max(float a, float b) {
  return __uint_as_float(max(__float_as_uint(a) & 0x7fffffffu, __float_as_uint(b) & 0x7fffffffu));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight codes rint(f[e] * inv), as two dwords (byte e = element e).  With
// |f| <= amax and inv = 127 / amax correctly rounded, every product is at
// most 127 * (1 + 2^-24)^2 < 127.5 in magnitude: no clamp.  Adding
// 1.5 * 2^23 rounds the product to the nearest integer (ties to even) in the
// low mantissa bits, whose low byte is the code in two's complement; three
// byte permutes gather four codes.  When the block maximum is NaN or
// infinite, or 127 / amax overflows, every product is NaN, infinite or 0,
// and every code is 0.
__device__ __forceinline__ uint2 i8_codes(const float (&f)[8], float inv, float amax) {
  uint32_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // the product rounded on its own (kept out of an FMA with the add)
    float r = f[e] * inv;
    asm volatile("" : "+v"(r));
    t[e] = __float_as_uint(r + 12582912.0f);
  }
  const bool ok = __builtin_isfinite(amax) && __builtin_isfinite(inv);
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = __builtin_amdgcn_perm(t[4 * h + 1], t[4 * h], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(t[4 * h + 3], t[4 * h + 2], 0x0c0c0400u);
    w[h] = ok ? __builtin_amdgcn_perm(hi, lo, 0x05040100u) : 0u;
  }
  return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ float inv_of(float amax) { return amax == 0.f ? 0.f : __fdiv_rn(127.0f, amax); }

// One (token, head) row of D dims per D / 8 consecutive lanes (8 dims each).
template <int D>
__global__ void __launch_bounds__(kThreads)
quantize_i8_rows_kernel(const uint16_t* __restrict__ x, int8_t* __restrict__ y, float* __restrict__ ys, int64_t S,
                        int32_t H, int64_t sx, int64_t sy) {
  constexpr int G = D / 8;  // lanes per row (a power of two dividing 64)
  const int64_t row = (int64_t(blockIdx.x) * kThreads + threadIdx.x) / G;
  const int c = int(threadIdx.x % G);
  const bool in = row < S * H;  // the group of a row exits together
  const int64_t token = in ? row / H : 0;
  const int h = in ? int(row % H) : 0;
  float f[8];
  float amax = 0.f;
  if (in) {
    const uint4 r = *reinterpret_cast<const uint4*>(x + token * sx + h * D + c * 8);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
      amax = nan_max(nan_max(amax, __builtin_fabsf(f[2 * i])), __builtin_fabsf(f[2 * i + 1]));
    }
  }
#pragma unroll
  for (int m = 1; m < G; m <<= 1) amax = nan_max(amax, __shfl_xor(amax, m, 64));
  if (!in) return;
  *reinterpret_cast<uint2*>(y + token * sy + h * D + c * 8) = i8_codes(f, inv_of(amax), amax);
  if (c == 0) ys[int64_t(h) * S + token] = __fdiv_rn(amax, 127.0f);
}

// One block of 64 keys of one head per workgroup: the block's maximum meets in
// LDS, then each thread writes the codes of its rows.  Segments of this
// launch: key 0 at start[s], len[s] keys, first block blocks[s] (from block0).
constexpr int kKeyMaxSegs = 64;

struct KeyBlockArgs {
  int32_t nseg;
  int32_t seg0;    // first segment of this launch
  int32_t block0;  // first block of this launch
  int32_t start[kKeyMaxSegs];
  int32_t len[kKeyMaxSegs];
  int32_t blocks[kKeyMaxSegs + 1];  // prefix sums of the segments' block counts
};

template <int D>
__global__ void __launch_bounds__(kThreads)
quantize_i8_keys_kernel(KeyBlockArgs a, const uint16_t* __restrict__ x, int8_t* __restrict__ y,
                        float* __restrict__ ys, int64_t n_blocks, int64_t sx, int64_t sy,
                        const float* __restrict__ mu) {
  constexpr int CH = D / 8;               // 8-dim chunks per key
  constexpr int KPP = kThreads / CH;      // keys per pass
  constexpr int NP = kVtTile / KPP;       // passes over the block's 64 keys
  __shared__ float wave_max[kThreads / 64];
  const int tau = blockIdx.x;
  const int h = blockIdx.y;
  int s = 0;
  while (s + 1 < a.nseg && tau >= a.blocks[s + 1]) ++s;
  const int key0 = (tau - a.blocks[s]) * kVtTile;
  const int c = int(threadIdx.x % CH), kr = int(threadIdx.x / CH);
  // centred keys: the segment's mean for this lane's 8 dims (0 without)
  float mk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mu != nullptr) {
    const float4* mp = reinterpret_cast<const float4*>(mu + (int64_t(a.seg0 + s) * gridDim.y + h) * D + c * 8);
    const float4 m0 = mp[0], m1 = mp[1];
    mk[0] = m0.x; mk[1] = m0.y; mk[2] = m0.z; mk[3] = m0.w; mk[4] = m1.x; mk[5] = m1.y; mk[6] = m1.z; mk[7] = m1.w;
  }
  float f[NP][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int key = key0 + p * KPP + kr;
    uint4 r = make_uint4(0, 0, 0, 0);  // keys past the segment: zeros, not stored
    if (key < a.len[s]) r = *reinterpret_cast<const uint4*>(x + int64_t(a.start[s] + key) * sx + h * D + c * 8);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[p][2 * i] = bf16_lo(w[i]) - mk[2 * i];
      f[p][2 * i + 1] = bf16_hi(w[i]) - mk[2 * i + 1];
      if (key < a.len[s])  // keys past the segment take no part in the maximum
        amax = nan_max(nan_max(amax, __builtin_fabsf(f[p][2 * i])), __builtin_fabsf(f[p][2 * i + 1]));
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = nan_max(amax, __shfl_xor(amax, m, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x / 64] = amax;
  __syncthreads();
  amax = wave_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) amax = nan_max(amax, wave_max[w]);
  const float inv = inv_of(amax);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int key = key0 + p * KPP + kr;
    if (key < a.len[s])
      *reinterpret_cast<uint2*>(y + int64_t(a.start[s] + key) * sy + h * D + c * 8) = i8_codes(f[p], inv, amax);
  }
  if (threadIdx.x == 0) ys[int64_t(h) * n_blocks + a.block0 + tau] = __fdiv_rn(amax, 127.0f);
}

// Segment means of the keys.  Segments of one launch: key 0 at start[s],
// len[s] keys, chunks[s] .. chunks[s + 1] its 256-key chunks (from chunk0).
constexpr int kMeanChunk = 256;

struct KeyChunkArgs {
  int32_t nseg;
  int32_t seg0;    // first segment of this launch
  int32_t chunk0;  // first chunk of this launch
  int32_t start[kKeyMaxSegs];
  int32_t len[kKeyMaxSegs];
  int32_t chunks[kKeyMaxSegs + 1];
};

// One 256-key chunk of one head per workgroup: each thread sums 8 dims of
// every (kThreads / (D / 8))-th key, then the rows of partial sums meet in LDS
// in row order; part [chunks][H][D].
template <int D>
__global__ void __launch_bounds__(kThreads)
key_chunk_sums_kernel(KeyChunkArgs a, const uint16_t* __restrict__ x, float* __restrict__ part, int64_t sx) {
  constexpr int CH = D / 8;           // 8-dim pieces per key
  constexpr int RPP = kThreads / CH;  // keys per pass
  __shared__ float rows[RPP][D];
  const int tau = blockIdx.x;
  const int h = blockIdx.y;
  int s = 0;
  while (s + 1 < a.nseg && tau >= a.chunks[s + 1]) ++s;
  const int key0 = (tau - a.chunks[s]) * kMeanChunk;
  const int c = int(threadIdx.x % CH), kr = int(threadIdx.x / CH);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int p = 0; p < kMeanChunk / RPP; ++p) {
    const int key = key0 + p * RPP + kr;
    if (key < a.len[s]) {
      const uint4 r = *reinterpret_cast<const uint4*>(x + int64_t(a.start[s] + key) * sx + h * D + c * 8);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_lo(w[i]);
        acc[2 * i + 1] += bf16_hi(w[i]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) rows[kr][c * 8 + e] = acc[e];
  __syncthreads();
  if (int(threadIdx.x) < D) {
    float t = 0.f;
    for (int r = 0; r < RPP; ++r) t += rows[r][threadIdx.x];
    part[(int64_t(a.chunk0 + tau) * gridDim.y + h) * D + threadIdx.x] = t;
  }
}

// One segment and head per workgroup, one dim per thread: the segment's chunk
// sums in chunk order, divided by its length (0 for an empty segment).
template <int D>
__global__ void __launch_bounds__(D)
key_means_kernel(KeyChunkArgs a, const float* __restrict__ part, float* __restrict__ mu) {
  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  float t = 0.f;
  for (int ci = a.chunks[s]; ci < a.chunks[s + 1]; ++ci) t += part[(int64_t(a.chunk0 + ci) * gridDim.y + h) * D + d];
  mu[(int64_t(a.seg0 + s) * gridDim.y + h) * D + d] = a.len[s] > 0 ? __fdiv_rn(t, float(a.len[s])) : 0.f;
}

}  // namespace

int64_t key_mean_chunks(const int32_t* cu, int32_t nseg) {
  int64_t n = 0;
  for (int32_t s = 0; s < nseg; ++s) n += (int64_t(cu[s + 1]) - cu[s] + kMeanChunk - 1) / kMeanChunk;
  return n;
}

hipError_t launch_segment_key_means(const void* x, void* part, void* mu, const int32_t* cu, int32_t nseg, int32_t H,
                                    int32_t D, int64_t sx, int64_t n_chunks, hipStream_t stream) {
  if (D != 128 && D != 64) return hipErrorInvalidValue;
  int32_t chunk0 = 0;
  for (int32_t s0 = 0; s0 < nseg; s0 += kKeyMaxSegs) {
    const int32_t n = nseg - s0 < kKeyMaxSegs ? nseg - s0 : kKeyMaxSegs;
    KeyChunkArgs a{};
    a.nseg = n;
    a.seg0 = s0;
    a.chunk0 = chunk0;
    a.chunks[0] = 0;
    for (int32_t i = 0; i < n; ++i) {
      a.start[i] = cu[s0 + i];
      a.len[i] = cu[s0 + i + 1] - cu[s0 + i];
      a.chunks[i + 1] = a.chunks[i] + (a.len[i] + kMeanChunk - 1) / kMeanChunk;
    }
    const int32_t nc = a.chunks[n];
    if (int64_t(chunk0) + nc > n_chunks) return hipErrorInvalidValue;
    if (nc > 0) {
      const dim3 grid{unsigned(nc), unsigned(H), 1u};
      if (D == 128)
        hipLaunchKernelGGL(key_chunk_sums_kernel<128>, grid, dim3(kThreads), 0, stream, a,
                           static_cast<const uint16_t*>(x), static_cast<float*>(part), sx);
      else
        hipLaunchKernelGGL(key_chunk_sums_kernel<64>, grid, dim3(kThreads), 0, stream, a,
                           static_cast<const uint16_t*>(x), static_cast<float*>(part), sx);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const dim3 grid{unsigned(n), unsigned(H), 1u};
    if (D == 128)
      hipLaunchKernelGGL(key_means_kernel<128>, grid, dim3(128), 0, stream, a, static_cast<const float*>(part),
                         static_cast<float*>(mu));
    else
      hipLaunchKernelGGL(key_means_kernel<64>, grid, dim3(64), 0, stream, a, static_cast<const float*>(part),
                         static_cast<float*>(mu));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    chunk0 += nc;
  }
  return hipSuccess;
}

hipError_t launch_quantize_i8_rows(const void* x, void* y, void* ys, int64_t S, int32_t H, int32_t D, int64_t sx,
                                   int64_t sy, hipStream_t stream) {
  if (S <= 0) return hipSuccess;
  if (H < 1) return hipErrorInvalidValue;
  const int64_t lanes = S * H * (D / 8);
  const unsigned blocks = unsigned((lanes + kThreads - 1) / kThreads);
  if (D == 128)
    hipLaunchKernelGGL(quantize_i8_rows_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<int8_t*>(y), static_cast<float*>(ys), S, H, sx, sy);
  else if (D == 64)
    hipLaunchKernelGGL(quantize_i8_rows_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<int8_t*>(y), static_cast<float*>(ys), S, H, sx, sy);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quantize_i8_keys(const void* x, void* y, void* ys, const int32_t* cu, int32_t nseg, int32_t H,
                                   int32_t D, int64_t sx, int64_t sy, int64_t n_blocks, hipStream_t stream,
                                   const float* mu) {
  if (D != 128 && D != 64) return hipErrorInvalidValue;
  int32_t block0 = 0;
  for (int32_t s0 = 0; s0 < nseg; s0 += kKeyMaxSegs) {
    const int32_t n = nseg - s0 < kKeyMaxSegs ? nseg - s0 : kKeyMaxSegs;
    KeyBlockArgs a{};
    a.nseg = n;
    a.seg0 = s0;
    a.block0 = block0;
    a.blocks[0] = 0;
    for (int32_t i = 0; i < n; ++i) {
      a.start[i] = cu[s0 + i];
      a.len[i] = cu[s0 + i + 1] - cu[s0 + i];
      a.blocks[i + 1] = a.blocks[i] + (a.len[i] + kVtTile - 1) / kVtTile;
    }
    const int32_t nb = a.blocks[n];
    if (nb > 0) {
      if (int64_t(block0) + nb > n_blocks) return hipErrorInvalidValue;
      const dim3 grid{unsigned(nb), unsigned(H), 1u};
      if (D == 128)
        hipLaunchKernelGGL(quantize_i8_keys_kernel<128>, grid, dim3(kThreads), 0, stream, a,
                           static_cast<const uint16_t*>(x), static_cast<int8_t*>(y), static_cast<float*>(ys), n_blocks,
                           sx, sy, mu);
      else
        hipLaunchKernelGGL(quantize_i8_keys_kernel<64>, grid, dim3(kThreads), 0, stream, a,
                           static_cast<const uint16_t*>(x), static_cast<int8_t*>(y), static_cast<float*>(ys), n_blocks,
                           sx, sy, mu);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    block0 += nb;
  }
  return hipSuccess;
}

}  // namespace h3a
