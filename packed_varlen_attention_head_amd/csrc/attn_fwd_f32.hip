// Varlen bidirectional attention in fp32 (correctness path for fp32 inputs).
//
// Same contract as the bf16 kernel -- per-segment, non-causal softmax
// attention over cu_seqlens (vllm.cpp PR #26, opening commit) with an
// online softmax in f32 (same PR, commit on the attention fast path) -- but
// fp32 end to end with plain FMAs: one lane per query row, 64 query rows per
// workgroup, K/V tiles of 4096/D keys staged in LDS and read as broadcasts.
// Scores of a tile are kept in registers so the running max and the output
// rescale happen once per tile.  The variants of the bf16 kernel are here
// too: K/V heads shared by query-head groups and a causal mask aligned at the
// segment start.
#include <cstdint>

#include "common.h"

namespace h3a {
namespace {

constexpr int kBM = 64;
static_assert(kBM == kAttnBlockM_F32, "plan block size must match the kernel");

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64)
attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, float* __restrict__ o, int64_t sq, int64_t sk,
                    int64_t sv, int64_t so, const WorkItem* __restrict__ items, float scale,
                    int kv_group) {
  constexpr int kBN = 4096 / D;  // 32 KiB of K and V per tile
  __shared__ float ks[kBN][D];
  __shared__ float vs[kBN][D];
  const WorkItem it = items[blockIdx.x];
  if (it.seg_len <= 0) return;
  const int lane = threadIdx.x;
  const int qi = it.q_start + lane;
  const bool valid = qi < it.seg_len;
  const int head_off = it.head * D;
  const int kv_off = (it.head / kv_group) * D;
  // Keys the workgroup needs: the segment, or (causal) up to its last row.
  const int nkeys = CAUSAL ? min(it.seg_len, it.q_start + kBM) : it.seg_len;

  float qv[D], acc[D];
  {
    const float* qp = q + int64_t(it.seg_start + (valid ? qi : 0)) * sq + head_off;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      qv[d] = valid ? qp[d] : 0.f;
      acc[d] = 0.f;
    }
  }
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  for (int key0 = 0; key0 < nkeys; key0 += kBN) {
    const int nk = nkeys - key0 < kBN ? nkeys - key0 : kBN;
    // Last key of the tile this lane may see (tile-relative).
    const int last = CAUSAL ? min(nk - 1, qi - key0) : nk - 1;
    __syncthreads();
    for (int idx = lane; idx < kBN * D; idx += 64) {
      const int r = idx / D, d = idx % D;
      const int64_t row = it.seg_start + key0 + r;
      ks[r][d] = r < nk ? k[row * sk + kv_off + d] : 0.f;
      vs[r][d] = r < nk ? v[row * sv + kv_off + d] : 0.f;
    }
    __syncthreads();

    float s[kBN];
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(qv[d], ks[j][d], dot);
      s[j] = j <= last ? dot * scale : -__builtin_inff();
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);  // finite: tile 0 always holds key 0
    const float alpha = expf(m_run - m_new);  // exp(-inf) = 0 on the first tile
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const float p = expf(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
    }
    m_run = m_new;
  }

  if (!valid) return;
  const float inv = 1.0f / l_run;
  float* op = o + int64_t(it.seg_start + qi) * so + head_off;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, int64_t sq, int64_t sk,
                  int64_t sv, int64_t so, const WorkItem* items, int64_t n_items, float scale,
                  int kv_group, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3(unsigned(n_items)), dim3(64), 0, stream,
                     static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), static_cast<float*>(o), sq, sk, sv, so, items, scale,
                     kv_group);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const void* q, const void* k, const void* v, void* o, int32_t D,
                               int64_t sq, int64_t sk, int64_t sv, int64_t so,
                               const WorkItem* items, int64_t n_items, float scale,
                               int32_t kv_group, bool causal, hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  if (kv_group < 1) return hipErrorInvalidValue;
  if (D == 128)
    return causal ? launch<128, true>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, stream)
                  : launch<128, false>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, stream);
  if (D == 64)
    return causal ? launch<64, true>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, stream)
                  : launch<64, false>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, stream);
  return hipErrorInvalidValue;
}

}  // namespace h3a
