// Varlen bidirectional flash attention, bf16 MFMA with fp32 accumulation,
// for gfx950 (CDNA4, wave64).
//
// What it computes: for every packed segment and head, o_i = sum_j
// softmax_j(scale <q_i, k_j>) v_j over the segment's own keys -- the
// per-document bidirectional cu_seqlens varlen attention of the H3 DiT
// (vllm.cpp PR #26, opening commit).  The softmax is the online recurrence
// with f32 accumulation (same PR, commit on the attention fast path), here
// evaluated per key tile rather than per key.
//
// Design (one workgroup per work item = 128 query rows of one segment and
// head; four waves, each owning 32 query rows):
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = a 32-key x 16-dim slice of K read from
//     LDS, B = the wave's 32 queries x 16 dims held in registers for the whole
//     item.  In the 32x32 accumulator layout a lane then holds one query
//     (lane % 32) and 16 of the 32 keys, so the softmax row statistics of a
//     query live in one lane pair (lane, lane ^ 32): one cross-lane exchange
//     per key tile for the max, none for the sum.
//   * The output is accumulated transposed as well, O^T += V^T P^T: the
//     probabilities leave the score accumulator as the B operand with no data
//     movement (converted to bf16 in place), and the per-query rescale factor
//     is a per-lane scalar.
//   * V^T is produced while staging V into LDS.  The score accumulator hands
//     a lane keys {0-3, 8-11} (lanes 0-31) or {4-7, 12-15} (lanes 32-63) of
//     each 16-key group as its 8 contraction slots, so V^T is stored with bits
//     2 and 3 of the key index swapped, which makes each A operand one
//     contiguous 16-byte LDS read.
//   * K rows and V^T rows are padded by 16 bytes so the 32 rows read by one
//     MFMA operand load fall on distinct LDS banks.
//   * K/V tiles of 64 keys are prefetched into registers one tile ahead.
//   * Keys past the segment end are loaded as zeros and masked to -inf in the
//     last tile only; query rows past the end are computed but not stored.
//   * exp2 with scale * log2(e) folded into one FMA; the accumulator rescale
//     is skipped when no query of the wave raised its running max.
#include <cstdint>

#include "common.h"

namespace h3a {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per work item
constexpr int kBN = 64;           // keys per tile
constexpr int kPad = 8;           // bf16 elements of row padding in LDS
static_assert(kBM == kAttnBlockM_BF16, "plan block size must match the kernel");

template <int D>
struct Smem {
  uint16_t k[kBN][D + kPad];   // K tile, row-major
  uint16_t vt[D][kBN + kPad];  // V tile transposed, key index bits 2 and 3 swapped
};

__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = __bf16(lo);
  const __bf16 b = __bf16(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

template <int D>
__global__ void __launch_bounds__(64 * kWaves, 2)
attn_fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, uint16_t* __restrict__ o, int64_t sq,
                     int64_t sk, int64_t sv, int64_t so, const WorkItem* __restrict__ items,
                     float c) {
  constexpr int KS = D / 16;               // MFMA k-steps over the head dim
  constexpr int DB = D / 32;               // 32-wide output dim blocks
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int KCH = kBN * CH / (64 * kWaves);  // K chunks staged per thread
  constexpr int KPT = kBN * CH / (64 * kWaves);  // V keys staged per thread
  static_assert(KCH >= 1 && KPT >= 2 && (KPT & (KPT - 1)) == 0, "staging layout");

  __shared__ Smem<D> sm;

  const WorkItem it = items[blockIdx.x];
  if (it.seg_len <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int head_off = it.head * D;
  const int qrow0 = it.q_start + wave * 32;
  const bool active = qrow0 < it.seg_len;

  // Q as the B operand: lane holds query (qrow0 + l32), dims ks*16 + hi*8 .. +8.
  bf16x8 qb[KS];
  {
    const int qi = qrow0 + l32;
    const uint16_t* qp = q + int64_t(it.seg_start + qi) * sq + head_off + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qi < it.seg_len) {
        qb[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
      } else {
        qb[ks] = bf16x8{};
      }
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -1e30f;  // running max of scale*log2(e)*score
  float l_run = 0.f;     // this lane's partial row sum (its 16-of-32 keys)

  // Staging assignment.  K: chunk index tid + i*256 -> (row, col chunk).
  // V: column chunk vc, keys vk0 .. vk0 + KPT - 1.
  const int vc = tid % CH;
  const int vk0 = (tid / CH) * KPT;

  uint4 kst[KCH], vst[KPT];
  const int ntiles = (it.seg_len + kBN - 1) / kBN;

  auto load_tile = [&](int t) {
    const int key0 = t * kBN;
    const int kvalid = it.seg_len - key0;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * 64 * kWaves;
      const int row = idx / CH, cc = idx % CH;
      if (row < kvalid) {
        kst[i] = *reinterpret_cast<const uint4*>(k + int64_t(it.seg_start + key0 + row) * sk + head_off + cc * 8);
      } else {
        kst[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int row = vk0 + i;
      if (row < kvalid) {
        vst[i] = *reinterpret_cast<const uint4*>(v + int64_t(it.seg_start + key0 + row) * sv + head_off + vc * 8);
      } else {
        vst[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * 64 * kWaves;
      const int row = idx / CH, cc = idx % CH;
      *reinterpret_cast<uint4*>(&sm.k[row][cc * 8]) = kst[i];
    }
    // Transpose: for each of the 8 dims of chunk vc, the KPT keys form one
    // contiguous run at vt_pos(vk0) (KPT divides 4, so bits 2/3 stay fixed).
    const int pos0 = vt_pos(vk0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t vals[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t w = (&vst[i].x)[e >> 1];
        vals[i] = uint16_t((e & 1) ? (w >> 16) : (w & 0xffffu));
      }
      uint16_t* dst = &sm.vt[vc * 8 + e][pos0];
      if constexpr (KPT == 4) {
        uint2 pk;
        pk.x = uint32_t(vals[0]) | (uint32_t(vals[1]) << 16);
        pk.y = uint32_t(vals[2]) | (uint32_t(vals[3]) << 16);
        *reinterpret_cast<uint2*>(dst) = pk;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = uint32_t(vals[0]) | (uint32_t(vals[1]) << 16);
      }
    }
  };

  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);
    if (!active) continue;

    // ---- S^T = K Q^T --------------------------------------------------------
    f32x16 sacc[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[kb * 32 + l32][ks * 16 + hi * 8]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], sacc[kb], 0, 0, 0);
      }
    }

    // ---- mask keys past the segment end (last tile only) ------------------
    const int kvalid = it.seg_len - t * kBN;
    if (kvalid < kBN) {
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          if (key >= kvalid) sacc[kb][r] = -__builtin_inff();
        }
    }

    // ---- online softmax ---------------------------------------------------
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const bool grow = m_new > m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;

    bf16x8 pb[kBN / 16];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][hh * 8 + i], c, -m_new));
          rs += p[i];
        }
        bf16x8 v8;
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = __bf16(p[i]);
        pb[kb * 2 + hh] = v8;
      }
    }
    l_run = l_run * alpha + rs;
    if (__any(grow)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }

    // ---- O^T += V^T P^T -----------------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kk = 0; kk < kBN / 16; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.vt[db * 32 + l32][kk * 16 + hi * 8]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], oacc[db], 0, 0, 0);
      }
  }

  if (!active) return;
  const int qi = qrow0 + l32;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qi >= it.seg_len) return;
  uint16_t* op = o + int64_t(it.seg_start + qi) * so + head_off + hi * 4;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk;
      pk.x = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      pk.y = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + db * 32 + g * 8) = pk;
    }
}

template <int D>
hipError_t launch(const void* q, const void* k, const void* v, void* o, int64_t sq, int64_t sk,
                  int64_t sv, int64_t so, const WorkItem* items, int64_t n_items, float scale,
                  hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D>), dim3(unsigned(n_items)), dim3(64 * kWaves), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), sq, sk, sv, so, items, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int32_t D,
                                int64_t sq, int64_t sk, int64_t sv, int64_t so,
                                const WorkItem* items, int64_t n_items, float scale,
                                hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  if (D == 128) return launch<128>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, stream);
  if (D == 64) return launch<64>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, stream);
  return hipErrorInvalidValue;
}

}  // namespace h3a
