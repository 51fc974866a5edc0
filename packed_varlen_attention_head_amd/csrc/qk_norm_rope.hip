// Fused per-head RMSNorm + NeoX rotary of Q and K (one HBM pass).
//
// The GB10 serving build fuses "Q RMSNorm + rot96 RoPE" into one kernel,
// byte-exact on default and non-default streams (h3-spark model card, "What
// this config does"); RmsNorm reduces in f32 (vllm.cpp PR #26, description,
// "The device-resident forward (W2b)"), and the rotary is NeoX rotate-half
// from a per-row cos/sin cache (same section).
//
// Mapping (HBM-bound; designed for 16-byte coalesced loads):
//   * one wavefront per token, four tokens per 256-thread workgroup;
//   * a head vector of D elements is split over LPV = D / V lanes, each lane
//     owning one 16-byte vector of V elements (V = 8 bf16 or 4 fp32), so a
//     wave touches G = 64 / LPV head vectors per instruction;
//   * a lane's cos/sin (and gains) depend only on its dims, so they are loaded
//     once per token and reused for every head of q and k;
//   * the rotary partner of element i (i +- R/2) lives in the lane R/(2V)
//     positions away, same slot, and is fetched with a lane shuffle;
//   * all loads of a head batch are issued before its stores, so in-place
//     calls are safe (each token is owned by a single wave); the stores are
//     non-temporal (streaming), as nothing in the pass reads them back;
//   * k may have fewer heads than q (grouped K/V heads of causal GQA);
//   * optionally (F8OUT) the bf16 results are written as OCP FP8 E4M3 codes
//     instead, one byte per element: the Q RMSNorm + rotary pass fused with
//     the quantisation that the low-precision attention consumes (h3-spark
//     model card, "What this config does": the Q RMSNorm + rot96 RoPE fused
//     into SageAttention's Q quantisation).  Each value is rounded to bf16
//     first and every block of 32 head dims shares one power-of-two scale
//     (mx_scale.h; the four lanes of a block exchange their maxima), so the
//     codes and scales equal those of the bf16 pass followed by the separate
//     quantiser;
//   * or (I8) the q results are written as INT8 codes with one fp32 scale per
//     token and head (the fused "Sage Q-INT8" tail of the same model card
//     section), k as plain bf16 for the key-block quantiser: rounded to bf16
//     first, the row maximum met over the row's lanes, so codes and scales
//     equal the bf16 pass followed by the row quantiser.
#include <cstdint>

#include "common.h"
#include "mx_scale.h"

namespace h3a {
namespace {

// The larger magnitude of a and b, a NaN kept (fmaxf would drop it):
// magnitudes compare as their bit patterns with the sign cleared, every NaN
// above +inf, with no branch.
__device__ __forceinline__ float nan_max(float a, float b) {
  return __uint_as_float(max(__float_as_uint(a) & 0x7fffffffu, __float_as_uint(b) & 0x7fffffffu));
}

// INT8 codes rint(b[e] * inv) of eight values, byte e of the pair = code e.
// With |b| <= amax and inv = 127 / amax correctly rounded, every product is
// at most 127 * (1 + 2^-24)^2 < 127.5 in magnitude: no clamp.  Adding
// 1.5 * 2^23 rounds the product to the nearest integer (ties to even) in the
// low mantissa bits, whose low byte is the code in two's complement; three
// byte permutes gather four codes.  `ok` false (a NaN or infinite maximum,
// or 127 / amax overflowing): every product is NaN, infinite or 0, so every
// code is 0.
__device__ __forceinline__ uint2 i8_pack8(const float* b, float inv, bool ok) {
  uint32_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // the product rounded on its own (kept out of an FMA with the add)
    float r = b[e] * inv;
    asm volatile("" : "+v"(r));
    t[e] = __float_as_uint(r + 12582912.0f);
  }
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = __builtin_amdgcn_perm(t[4 * h + 1], t[4 * h], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(t[4 * h + 3], t[4 * h + 2], 0x0c0c0400u);
    w[h] = ok ? __builtin_amdgcn_perm(hi, lo, 0x05040100u) : 0u;
  }
  return make_uint2(w[0], w[1]);
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int V = 4;
  __device__ static void unpack(const uint4& r, float* x) {
    x[0] = __uint_as_float(r.x);
    x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z);
    x[3] = __uint_as_float(r.w);
  }
  __device__ static uint4 pack(const float* y) {
    return make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                      __float_as_uint(y[3]));
  }
};

struct Bf16Tag;
template <>
struct Elem<Bf16Tag> {
  static constexpr int V = 8;
  __device__ static void unpack(const uint4& r, float* x) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  // fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
  __device__ static uint32_t pack2(float lo, float hi) {
    const __bf16 a = __bf16(lo);
    const __bf16 b = __bf16(hi);
    return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
  }
  __device__ static uint4 pack(const float* y) {
    return make_uint4(pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7]));
  }
  // bf16 rounding, then E4M3 codes of the values times 2^-X, X the scale
  // exponent of the lane's 32-dim block (shared with its three neighbours);
  // returns the codes and leaves X in *X.
  __device__ static uint2 pack_e4m3(const float* y, int* X) {
    float b[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = float(__bf16(y[e]));
      amax = abs_max(amax, b[e]);
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    *X = mx_exponent(amax);
    const float inv = mx_inv_scale(*X);
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = e4m3_sat(b[e] * inv);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(b[0], b[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(b[2], b[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(b[4], b[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(b[6], b[7], w1, true);
    return make_uint2(uint32_t(w0), uint32_t(w1));
  }
  // bf16 rounding, then INT8 codes rint(b * 127 / amax) of a row whose LPV
  // lanes (consecutive, an aligned group) share amax; a NaN maximum is kept,
  // so a row holding a NaN or an infinity has a non-finite scale and codes 0.
  // Returns the codes and leaves the row's scale amax / 127 in *scale.
  template <int LPV>
  __device__ static uint2 pack_i8(const float* y, float* scale) {
    float b[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = float(__bf16(y[e]));
      amax = nan_max(amax, __builtin_fabsf(b[e]));
    }
#pragma unroll
    for (int off = LPV / 2; off >= 1; off >>= 1) amax = nan_max(amax, __shfl_xor(amax, off, 64));
    const float inv = amax == 0.f ? 0.f : __fdiv_rn(127.0f, amax);
    *scale = __fdiv_rn(amax, 127.0f);
    return i8_pack8(b, inv, __builtin_isfinite(amax) && __builtin_isfinite(inv));
  }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;
constexpr int kBatch = 8;  // head vectors a lane keeps in flight

// Output forms of one tensor: plain (the input type), E4M3 codes with
// dst_scale [H][S][D / 32] E8M0 codes (head-major: a head's tokens are
// contiguous, the order the attention reads a tile's keys in), or INT8 codes
// with dst_scale [H][S] fp32.
constexpr int kOutPlain = 0, kOutE4M3 = 1, kOutI8 = 2;

template <typename T, int D, int OUT>
__device__ __forceinline__ void norm_rope_one(const char* __restrict__ src, char* dst, void* dst_scale,
                                              int64_t stride_b, int64_t stride_ob, int32_t token, int32_t S,
                                              int32_t H,
                                              const float* g, const float* c, const float* s, int role,
                                              int partner, float eps, int lane) {
  constexpr int V = Elem<T>::V;
  constexpr int LPV = D / V;
  constexpr int G = 64 / LPV;
  constexpr int esz = 16 / V;
  const int sub = lane % LPV;
  const int grp = lane / LPV;
  const char* row = src + int64_t(token) * stride_b + sub * 16;
  char* orow = dst + int64_t(token) * stride_ob + sub * (OUT != kOutPlain ? V : 16);
  for (int h0 = 0; h0 < H; h0 += G * kBatch) {
    uint4 raw[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int h = h0 + b * G + grp;
      raw[b] = h < H ? *reinterpret_cast<const uint4*>(row + int64_t(h) * D * esz) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (h0 + b * G >= H) break;  // wave-uniform
      float x[V];
      Elem<T>::unpack(raw[b], x);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
      for (int off = LPV / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
      const float r = 1.0f / sqrtf(ss * (1.0f / float(D)) + eps);
      float y[V], out[V];
#pragma unroll
      for (int e = 0; e < V; ++e) y[e] = x[e] * r * g[e];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float py = __shfl(y[e], partner, 64);
        out[e] = role == 0 ? fmaf(y[e], c[e], -py * s[e]) : (role == 1 ? fmaf(y[e], c[e], py * s[e]) : y[e]);
      }
      const int h = h0 + b * G + grp;
      if (h < H) {
        // Streaming (non-temporal) stores: the outputs are not re-read by
        // this pass; measured 14% faster than ordinary stores at S = 20,423.
        if constexpr (OUT == kOutE4M3) {
          int X = 0;
          const uint2 pk = Elem<T>::pack_e4m3(out, &X);
          __builtin_nontemporal_store(u32x2{pk.x, pk.y}, reinterpret_cast<u32x2*>(orow + int64_t(h) * D));
          if ((sub & 3) == 0)
            static_cast<uint8_t*>(dst_scale)[(int64_t(h) * S + token) * (D / 32) + sub / 4] = uint8_t(X + 127);
        } else if constexpr (OUT == kOutI8) {
          float sc = 0.f;
          const uint2 pk = Elem<T>::template pack_i8<LPV>(out, &sc);
          __builtin_nontemporal_store(u32x2{pk.x, pk.y}, reinterpret_cast<u32x2*>(orow + int64_t(h) * D));
          if (sub == 0) static_cast<float*>(dst_scale)[int64_t(h) * S + token] = sc;
        } else {
          const uint4 pk = Elem<T>::pack(out);
          __builtin_nontemporal_store(u32x4{pk.x, pk.y, pk.z, pk.w},
                                      reinterpret_cast<u32x4*>(orow + int64_t(h) * D * esz));
        }
      }
    }
  }
}

template <typename T, int D, int QOUT = kOutPlain, int KOUT = QOUT>
__global__ void __launch_bounds__(64 * kWavesPerBlock)
qk_norm_rope_kernel(const char* q, const char* k, char* qo, char* ko, void* qos, void* kos, int64_t sq_b,
                    int64_t sk_b, int64_t sqo_b, int64_t sko_b, int32_t S, int32_t H, int32_t Hk,
                    const float* __restrict__ gq, const float* __restrict__ gk, float eps,
                    const float* __restrict__ cos_sin, int32_t rot_dim) {
  constexpr int V = Elem<T>::V;
  constexpr int LPV = D / V;
  const int lane = threadIdx.x & 63;
  const int32_t token = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (token >= S) return;
  const int sub = lane % LPV;
  const int d0 = sub * V;
  const int half = rot_dim >> 1;
  const int po = half / V;  // partner distance in lanes
  const int role = d0 < half ? 0 : (d0 < rot_dim ? 1 : 2);
  const int partner = role == 0 ? lane + po : (role == 1 ? lane - po : lane);
  float c[V], s[V], g_q[V], g_k[V];
  if (role != 2) {
    const int j0 = role == 0 ? d0 : d0 - half;
    const float* cp = cos_sin + int64_t(token) * half + j0;
    const float* sp = cp + int64_t(S) * half;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      c[e] = cp[e];
      s[e] = sp[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      c[e] = 1.f;
      s[e] = 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) {
    g_q[e] = gq[d0 + e];
    g_k[e] = gk[d0 + e];
  }
  norm_rope_one<T, D, QOUT>(q, qo, qos, sq_b, sqo_b, token, S, H, g_q, c, s, role, partner, eps, lane);
  norm_rope_one<T, D, KOUT>(k, ko, kos, sk_b, sko_b, token, S, Hk, g_k, c, s, role, partner, eps, lane);
}

// Strides in elements of the input type; for code outputs the output strides
// are in bytes (one per code).
template <typename T, int D, int QOUT = kOutPlain, int KOUT = QOUT>
hipError_t launch(const void* q, const void* k, void* qo, void* ko, int64_t S, int32_t H, int32_t Hk, int64_t sq,
                  int64_t sk, int64_t sqo, int64_t sko, const float* gq, const float* gk, float eps,
                  const float* cos_sin, int32_t rot_dim, hipStream_t stream, void* qos = nullptr,
                  void* kos = nullptr) {
  constexpr int esz = 16 / Elem<T>::V;
  constexpr int qoesz = QOUT != kOutPlain ? 1 : esz, koesz = KOUT != kOutPlain ? 1 : esz;
  const unsigned blocks = unsigned((S + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL((qk_norm_rope_kernel<T, D, QOUT, KOUT>), dim3(blocks), dim3(64 * kWavesPerBlock), 0, stream,
                     static_cast<const char*>(q), static_cast<const char*>(k), static_cast<char*>(qo),
                     static_cast<char*>(ko), qos, kos, sq * esz, sk * esz, sqo * qoesz, sko * koesz, int32_t(S), H,
                     Hk, gq, gk, eps, cos_sin, rot_dim);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_rmsnorm_rope(bool bf16, const void* q, const void* k, void* q_out, void* k_out,
                                  int64_t S, int32_t H, int32_t Hk, int32_t D, int64_t sq, int64_t sk,
                                  int64_t sqo, int64_t sko, const float* gq, const float* gk,
                                  float eps, const float* cos_sin, int32_t rot_dim,
                                  hipStream_t stream) {
  if (bf16) {
    if (D == 128)
      return launch<Bf16Tag, 128>(q, k, q_out, k_out, S, H, Hk, sq, sk, sqo, sko, gq, gk, eps, cos_sin, rot_dim, stream);
    if (D == 64)
      return launch<Bf16Tag, 64>(q, k, q_out, k_out, S, H, Hk, sq, sk, sqo, sko, gq, gk, eps, cos_sin, rot_dim, stream);
  } else {
    if (D == 128)
      return launch<float, 128>(q, k, q_out, k_out, S, H, Hk, sq, sk, sqo, sko, gq, gk, eps, cos_sin, rot_dim, stream);
    if (D == 64)
      return launch<float, 64>(q, k, q_out, k_out, S, H, Hk, sq, sk, sqo, sko, gq, gk, eps, cos_sin, rot_dim, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qk_rmsnorm_rope_e4m3(const void* q, const void* k, void* q8, void* k8, void* q8s, void* k8s,
                                       int64_t S, int32_t H, int32_t Hk, int32_t D, int64_t sq, int64_t sk,
                                       int64_t sq8, int64_t sk8, const float* gq, const float* gk, float eps,
                                       const float* cos_sin, int32_t rot_dim, hipStream_t stream) {
  if (D == 128)
    return launch<Bf16Tag, 128, kOutE4M3>(q, k, q8, k8, S, H, Hk, sq, sk, sq8, sk8, gq, gk, eps, cos_sin, rot_dim,
                                          stream, q8s, k8s);
  if (D == 64)
    return launch<Bf16Tag, 64, kOutE4M3>(q, k, q8, k8, S, H, Hk, sq, sk, sq8, sk8, gq, gk, eps, cos_sin, rot_dim,
                                         stream, q8s, k8s);
  return hipErrorInvalidValue;
}

hipError_t launch_qk_rmsnorm_rope_i8q(const void* q, const void* k, void* q8, void* k_out, void* q8s, int64_t S,
                                      int32_t H, int32_t Hk, int32_t D, int64_t sq, int64_t sk, int64_t sq8,
                                      int64_t sko, const float* gq, const float* gk, float eps,
                                      const float* cos_sin, int32_t rot_dim, hipStream_t stream) {
  if (D == 128)
    return launch<Bf16Tag, 128, kOutI8, kOutPlain>(q, k, q8, k_out, S, H, Hk, sq, sk, sq8, sko, gq, gk, eps, cos_sin,
                                                   rot_dim, stream, q8s, nullptr);
  if (D == 64)
    return launch<Bf16Tag, 64, kOutI8, kOutPlain>(q, k, q8, k_out, S, H, Hk, sq, sk, sq8, sko, gq, gk, eps, cos_sin,
                                                  rot_dim, stream, q8s, nullptr);
  return hipErrorInvalidValue;
}

}  // namespace h3a
