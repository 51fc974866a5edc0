// Internal declarations shared by the h3a host code and its kernel launchers.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

namespace h3a {

// One attention work item: query rows [q_start, q_start + block_m) of one
// segment and one head, against the segment's 64-key tiles [kt0, kt1)
// (kt1 == 0: all of them).  seg_len == 0 marks a padding item (the workgroup
// exits at once).  vt_col0 is the segment's first column in the transposed
// E4M3 V layout, where every segment is padded to whole 64-key tiles (the sum
// of the earlier segments' padded lengths); only the FP8-PV kernel reads it.
// part == 0: the item covers all keys and stores its normalised rows; part
// > 0: it covers one key range of a split item and stores its unnormalised
// rows with their running max and row sum in partial slot part - 1, for the
// merge pass (kt0 is then even, so tile parities match a full item's).
struct WorkItem {
  int32_t seg_start;
  int32_t seg_len;
  int32_t q_start;  // relative to seg_start
  int32_t head;
  int32_t vt_col0;
  int32_t kt0;
  int32_t kt1;
  int32_t part;
};
static_assert(sizeof(WorkItem) == 32, "WorkItem is uploaded as 8 x int32");

// One split item to merge: query rows [q_start, q_start + block_m) of one
// segment and head, whose key ranges wrote partial slots part0 .. part0 +
// nparts - 1 (in key order).
struct MergeItem {
  int32_t seg_start;
  int32_t seg_len;
  int32_t q_start;
  int32_t head;
  int32_t part0;
  int32_t nparts;
  int32_t pad[2];
};
static_assert(sizeof(MergeItem) == 32, "MergeItem is uploaded as 8 x int32");

// Partial results of split items, in device memory: slot p holds block_m rows
// of D fp32 unnormalised outputs at o + p * block_m * D, and per row the
// running max (scale * log2(e) units) and row sum at ml + 2 * (p * block_m + r).
struct SplitArgs {
  float* o;
  float* ml;
};

// Keys per tile of the transposed E4M3 V layout (and of the attention's K/V
// tiles).
constexpr int32_t kVtTile = 64;

// ---- host tile planner (planner.cpp) --------------------------------------
// Items for every (non-empty segment, head, query tile), longest segments
// first, balanced over n_xcd XCDs and interleaved so that workgroup b lands on
// XCD b % n_xcd with that XCD's items in its own longest-first order.
// Causal plans cost an item by the keys up to its last row and put each
// chunk's costliest (last) query tiles first.
std::vector<WorkItem> plan_tiles(const int32_t* cu, int32_t nseg, int32_t heads, int32_t block_m,
                                 int32_t n_xcd, bool causal = false);

// Split policies of plan_tiles_split.
constexpr int32_t kSplitAuto = 0, kSplitNever = 1, kSplitAlways = 2;

// As plan_tiles, but (bidirectional plans) an item's keys may be cut into
// even-tile ranges, each its own item writing a partial slot, so that the
// longest items no longer set the time on `slots` concurrent workgroups:
// kSplitAuto picks the largest part length that minimises a list-scheduling
// estimate of the makespan plus the merge pass; kSplitAlways cuts every item
// of four or more key tiles into parts of about a third (for tests).  Plans
// needing more than 16,384 partial slots stay unsplit.  Fills
// merges (one per split item) and *n_parts (partial slots used).
std::vector<WorkItem> plan_tiles_split(const int32_t* cu, int32_t nseg, int32_t heads, int32_t block_m,
                                       int32_t n_xcd, int32_t slots, bool causal, int32_t policy,
                                       std::vector<MergeItem>* merges, int64_t* n_parts);

// ---- kernel launchers (one per .hip file) ---------------------------------

// Rotary table modes (values of h3a_rope_mode).
constexpr int32_t kRopeGrid = 0, kRopeLinspace = 1, kRopeNormalized = 2, kRopeInterleaved = 3;

// Angle j of a token = p_axis_of[j] * inv_freq[j]; the mode says how the
// coordinate p comes from the grid index (see rope_table.hip).
struct RopeTableSpec {
  int32_t mode;
  int32_t half;             // R / 2 angles per token (<= 64)
  const double* inv_freq;   // [half]
  const int32_t* axis_of;   // [half], 0 = t, 1 = h, 2 = w
  double lin_start[3];      // linspace mode only
  double lin_stop[3];
};

hipError_t launch_rope_table(const RopeTableSpec& spec, const int32_t* segments, const int32_t* starts,
                             int32_t nseg, float* cos_sin, int64_t S, hipStream_t stream);

hipError_t launch_qk_rmsnorm_rope(bool bf16, const void* q, const void* k, void* q_out, void* k_out,
                                  int64_t S, int32_t H, int32_t Hk, int32_t D, int64_t sq, int64_t sk,
                                  int64_t sqo, int64_t sko, const float* gq, const float* gk,
                                  float eps, const float* cos_sin, int32_t rot_dim,
                                  hipStream_t stream);

// Query rows per work item of each attention kernel.
constexpr int kAttnBlockM_BF16 = 128;
constexpr int kAttnBlockM_F32 = 64;

// Query head h reads K/V head h / kv_group; causal: query i of a segment
// sees keys 0..i of it.
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int32_t D,
                                int64_t sq, int64_t sk, int64_t sv, int64_t so,
                                const WorkItem* items, int64_t n_items, float scale,
                                int32_t kv_group, bool causal, hipStream_t stream,
                                const SplitArgs& sp = SplitArgs{});

// Bidirectional bf16 attention that RMS-normalises and rotates the raw q rows
// in its prologue (rot_dim a multiple of 32, at most D); q' is bit-identical
// to launch_qk_rmsnorm_rope's.
hipError_t launch_attn_fwd_bf16_qnorm(const void* q, const void* k, const void* v, void* o, int32_t D,
                                      int64_t sq, int64_t sk, int64_t sv, int64_t so,
                                      const WorkItem* items, int64_t n_items, float scale, int32_t kv_group,
                                      const float* gamma_q, float eps, const float* cos_sin, int64_t S,
                                      int32_t rot_dim, hipStream_t stream,
                                      const SplitArgs& sp = SplitArgs{});

// Attention whose q and k are FP8 E4M3 codes (token strides in bytes) with
// one E8M0 scale per 32 head dims, head-major (q8s [Hq][S][D/32], k8s
// [Hkv][S][D/32]; head strides sqs, sks bytes); the score product runs on the
// scaled FP8 MFMA, the rest as launch_attn_fwd_bf16.
hipError_t launch_attn_fwd_fp8qk(const void* q8, const void* k8, const void* q8s, const void* k8s, const void* v,
                                 void* o, int32_t D, int64_t sq, int64_t sk, int64_t sqs, int64_t sks, int64_t sv,
                                 int64_t so, const WorkItem* items, int64_t n_items, float scale, int32_t kv_group,
                                 bool causal, hipStream_t stream,
                                 const SplitArgs& sp = SplitArgs{});

// Attention whose q and k are INT8 codes (token strides in bytes): q with one
// fp32 scale per token (q_scale [Hq][S], head stride sqs bytes), k with one
// per block of 64 keys of a segment (k_scale [Hkv][blocks], the segment's
// first block at its padded column / 64, head stride sks bytes); the score
// product runs on the INT8 MFMA, the rest as launch_attn_fwd_bf16.
hipError_t launch_attn_fwd_i8qk(const void* q8, const void* k8, const void* q_scale, const void* k_scale,
                                const void* v, void* o, int32_t D, int64_t sq, int64_t sk, int64_t sqs, int64_t sks,
                                int64_t sv, int64_t so, const WorkItem* items, int64_t n_items, float scale,
                                int32_t kv_group, bool causal, hipStream_t stream,
                                const SplitArgs& sp = SplitArgs{});

// INT8 scores (as launch_attn_fwd_i8qk) with FP8 PV on the transposed E4M3
// V layout (as launch_attn_fwd_fp8).
hipError_t launch_attn_fwd_i8qk_fp8pv(const void* q8, const void* k8, const void* vt8, const void* q_scale,
                                     const void* k_scale, const void* vt8s, void* o, int32_t D, int64_t sq, int64_t sk,
                                     int64_t sqs, int64_t sks, int64_t vt_cols, int64_t so, const WorkItem* items,
                                     int64_t n_items, float scale, int32_t kv_group, bool causal, hipStream_t stream,
                                     const SplitArgs& sp);

// bf16 [S, H, D] rows (token stride sx elements) -> INT8 codes (token stride
// sy bytes) with one fp32 scale per token and head (ys [H][S]); and, per
// segment of cu (host array, nseg + 1 entries), with one fp32 scale per block
// of 64 keys of a head (ys [H][blocks], blocks numbered segment by segment).
hipError_t launch_quantize_i8_rows(const void* x, void* y, void* ys, int64_t S, int32_t H, int32_t D, int64_t sx,
                                   int64_t sy, hipStream_t stream);
hipError_t launch_quantize_i8_keys(const void* x, void* y, void* ys, const int32_t* cu, int32_t nseg, int32_t H,
                                   int32_t D, int64_t sx, int64_t sy, int64_t n_blocks, hipStream_t stream,
                                   const float* mu = nullptr);

// Centred keys: the number of 256-key chunks of cu_seqlens (each segment's
// from its start), and the segment means of x [S, H, D] (bf16, token stride
// sx elements) into mu [nseg][H][D] fp32 through the chunk sums part
// [n_chunks][H][D] fp32.
int64_t key_mean_chunks(const int32_t* cu, int32_t nseg);
hipError_t launch_segment_key_means(const void* x, void* part, void* mu, const int32_t* cu, int32_t nseg, int32_t H,
                                    int32_t D, int64_t sx, int64_t n_chunks, hipStream_t stream);

// The bf16 norm + rotary pass writing E4M3 codes of its bf16 results (output
// token strides sq8, sk8 in bytes) with one E8M0 scale per 32 head dims in
// q8s [H][S][D/32], k8s [Hk][S][D/32].
hipError_t launch_qk_rmsnorm_rope_e4m3(const void* q, const void* k, void* q8, void* k8, void* q8s, void* k8s,
                                       int64_t S, int32_t H, int32_t Hk, int32_t D, int64_t sq, int64_t sk,
                                       int64_t sq8, int64_t sk8, const float* gq, const float* gk, float eps,
                                       const float* cos_sin, int32_t rot_dim, hipStream_t stream);

// The bf16 norm + rotary pass writing q as INT8 codes of its bf16 results
// (token stride sq8 in bytes) with one fp32 scale per token and head in
// q8s [H][S], and k as bf16 (token stride sko elements).
hipError_t launch_qk_rmsnorm_rope_i8q(const void* q, const void* k, void* q8, void* k_out, void* q8s, int64_t S,
                                      int32_t H, int32_t Hk, int32_t D, int64_t sq, int64_t sk, int64_t sq8,
                                      int64_t sko, const float* gq, const float* gk, float eps,
                                      const float* cos_sin, int32_t rot_dim, hipStream_t stream);

// Attention with q, k as scaled E4M3 codes (as launch_attn_fwd_fp8qk) and V
// as the transposed E4M3 layout of launch_prepare_vt_e4m3 (row length vt_cols
// bytes, scales vt8s); both products on the scaled FP8 MFMA.
hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, const void* q8s, const void* k8s,
                               const void* vt8s, void* o, int32_t D, int64_t sq, int64_t sk, int64_t sqs, int64_t sks,
                               int64_t vt_cols, int64_t so, const WorkItem* items, int64_t n_items, float scale,
                               int32_t kv_group, bool causal, hipStream_t stream,
                               const SplitArgs& sp = SplitArgs{});

// Merge pass of a split plan: for each of the n_merges split items, the
// softmax-weighted combination of its key ranges' partial rows (sp), written
// as bf16 rows of o [S, H, D] (token stride so elements).
hipError_t launch_attn_merge(const MergeItem* merges, int64_t n_merges, const SplitArgs& sp, void* o, int32_t D,
                             int64_t so, hipStream_t stream);

// Columns of the transposed E4M3 V layout: every segment padded to whole
// kVtTile-key tiles.
int64_t vt_e4m3_columns(const int32_t* cu, int32_t nseg);

// bf16 v [S, H, D] (token stride sv elements) -> vt [H][D][vt_cols] E4M3
// codes, segment s at columns from the padded prefix sum, padding zeroed;
// one E8M0 scale per head dim and 32-key block in vs
// [H][vt_cols / 64][2][32][D / 32] (dim 32 b + r, block j at [j][r][b]).
hipError_t launch_prepare_vt_e4m3(const void* v, int64_t sv, const int32_t* cu, int32_t nseg, int32_t H, int32_t D,
                                  void* vt, void* vs, int64_t vt_cols, hipStream_t stream);

// bf16 [S, H, D] rows (token stride sx elements) -> E4M3 codes (token stride
// sy bytes) with one E8M0 scale per 32 consecutive elements of a head in ys
// [H][S][D / 32]; D a multiple of 32.
hipError_t launch_quantize_e4m3(const void* x, void* y, void* ys, int64_t S, int32_t H, int32_t D, int64_t sx,
                                int64_t sy, hipStream_t stream);

hipError_t launch_attn_fwd_f32(const void* q, const void* k, const void* v, void* o, int32_t D,
                               int64_t sq, int64_t sk, int64_t sv, int64_t so,
                               const WorkItem* items, int64_t n_items, float scale,
                               int32_t kv_group, bool causal, hipStream_t stream);

// ---- allocation-free attention (attn_noalloc.hip) --------------------------
// Largest padded plan (work items) and number of non-empty segments the
// allocation-free entry point takes: 2 MiB of plan storage per GPU, and a
// segment table that fits in the plan kernel's arguments.
constexpr int32_t kNoAllocMaxItems = 1 << 16;
constexpr int32_t kNoAllocMaxSegs = 256;

// Per-segment table of the allocation-free plan: the non-empty segments,
// longest first, and the index of each one's first item in the natural order
// (segment-major, then head, then query tile).
struct NoAllocPlanArgs {
  int32_t nseg;
  int32_t block_m;
  int32_t n_xcd;
  int32_t n_items;   // natural items (sum of query tiles times heads)
  int32_t n_blocks;  // padded launch size: n_xcd * kChunk * ceil(ceil(n_items / 16) / n_xcd)
  int32_t start[kNoAllocMaxSegs];
  int32_t len[kNoAllocMaxSegs];
  int32_t first[kNoAllocMaxSegs];
};

// Expands the table into the file-scope plan array on `stream`, then launches
// the bf16 or fp32 attention kernel on it (after any earlier such launch on
// this device, whatever its stream).
hipError_t launch_attn_noalloc(const NoAllocPlanArgs& plan, bool bf16, const void* q, const void* k, const void* v,
                               void* o, int32_t D, int64_t sq, int64_t sk, int64_t sv, int64_t so, float scale,
                               int32_t kv_group, bool causal, hipStream_t stream);

}  // namespace h3a
