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
//     is a per-lane scalar.  The accumulator hands a lane keys {0-3, 8-11}
//     (lanes 0-31) or {4-7, 12-15} (lanes 32-63) of each 16-key group as its
//     8 contraction slots; the matching V^T operand is two transposing LDS
//     reads (ds_read_b64_tr_b16) of 4 consecutive keys each from row-major V.
//   * K and V tiles of 64 keys go from HBM straight into LDS with 16-byte
//     buffer-to-LDS loads (no staging registers), double-buffered: the next
//     tile's loads are in flight while the current tile is computed, and one
//     barrier per tile separates the two stages' writers and readers.
//   * Each ring slot is its own LDS object: with one array and an index, the
//     compiler cannot tell a load into one slot from reads of another and
//     waits for every outstanding load before each LDS read.
//   * LDS rows are not padded (the LDS-bound loads write 1 KiB runs); bank
//     conflicts are avoided by XOR-swizzling the 16-byte chunks of a row
//     (k_swz, v_swz below: the 16 rows of one K operand read, and the 4 rows
//     x 64 bytes of one transposing V read, each land on distinct bank
//     slots).  All per-lane LDS addresses are computed once; tile, slot and
//     block offsets are immediates (the tile loop is unrolled over the two
//     slots).
//   * Loads go through buffer resources bounded at the segment end, so rows
//     past it read as zeros with no per-lane branches; those keys are masked
//     to -inf in the last tile only, and query rows past the end are computed
//     but not stored.
//   * exp2 with scale * log2(e) folded into one FMA.  The running max is a
//     reference only: it is raised (and the accumulator rescaled, which is
//     exact) when a tile exceeds it by more than 2^8 -- or, in the bf16 steady
//     loop, which takes no per-tile max at all, when a lane's sum of its
//     tile probabilities exceeds 2^13, after which the tile is recomputed.
//   * Optionally (QNORM) the Q rows are RMS-normalised and rotated in the
//     prologue, from raw q, fusing the Q half of the norm + rotary pass into
//     the attention (the GB10 build fuses Q RMSNorm + rot96 RoPE into its
//     attention front end: h3-spark model card, "What this config does").
//     The arithmetic follows the standalone norm + rotary kernel operation
//     for operation (per-16-byte-chunk FMA chains, the same xor-butterfly
//     for the sum of squares, the same rotation FMAs and one RNE rounding),
//     so q' -- and therefore the output -- is bit-identical to the unfused
//     path.
//   * Low-precision variants: F8 >= 1 takes Q and K as FP8 E4M3 codes with
//     one power-of-two (E8M0) scale per 32 head dims of each token, and runs
//     the score product on v_mfma_scale_f32_32x32x64_f8f6f4, which applies
//     those scales inside the instruction (no VALU), at twice the bf16 MFMA
//     rate, with K tiles of half the bytes.  The instruction numbers the 64
//     contraction elements of a step so that byte b of a lane in half h is
//     element 32 (b / 16) + 16 h + b % 16, and takes the scale of the block of
//     32 elements starting at 32 j from the lane in half j: a lane therefore
//     carries dims 16 h .. 16 h + 15 and 32 + 16 h .. +15 of its key (A) and
//     query (B) row per 64-dim step, and supplies the scale of block 2 ks + h.
//     F8 == 2 also runs PV in FP8: V arrives transposed (rows = dims, one
//     64-key tile per segment-padded column block, E4M3) with one scale per
//     dim and 32-key block, so the V^T operand is two plain 16-byte LDS reads
//     (keys 16 h .. +15 and 32 + 16 h .. +15) and one scale word per tile; the
//     probabilities, offset by 2^4 against the running reference (which moves
//     once a tile exceeds it by 2^4) so the weights of the largest scores stay
//     in E4M3's normal range and below 448, leave the score accumulator as the
//     B operand after four lane-half swaps that give each lane the same keys.
//     The row sums are one more FP8 MFMA per tile with an all-ones A operand,
//     so they add exactly the E4M3 weights PV applies; the 2^4 cancels.
//     F8 == 3 takes Q and K as INT8 codes (one fp32 scale per query row, one
//     per 64-key block of a segment) and runs the score product on
//     v_mfma_i32_32x32x32_i8: the accumulator starts from the bits of the
//     float 1.5 * 2^23, so the exact int32 sum reads as a float offset by that
//     constant and the probabilities' existing FMA applies both scales and
//     removes the offset.  F8 == 4 combines those scores with F8 == 2's FP8 PV
//     product (INT8 QK^T, FP8 PV).
//   * Variants: K/V heads shared by groups of query heads (query head h reads
//     K/V head h / kv_group), and a causal mask aligned at the segment start
//     (the encoder text tower's causal GQA; encoder-tower commit).  Causal
//     items stop at their last query row's key tile; with 128-row items on
//     128-aligned starts only the last two key tiles cross the diagonal, and
//     those are always computed in the masked tail of the tile loop, so the
//     steady-state loop is the same code in both variants.
#include <cstdint>
#include <type_traits>

#include "common.h"

namespace h3a {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per work item
[[maybe_unused]] constexpr int kBN = 64;  // keys per tile
[[maybe_unused]] constexpr float kRescaleSlack = 8.0f;  // log2 headroom before the running max moves
[[maybe_unused]] constexpr float kRescaleSlackF8 = 4.0f;  // E4M3 probabilities: 2^(4 + 4) = 256 <= 448
[[maybe_unused]] constexpr float kProbOffsetF8 = 4.0f;    // E4M3 probabilities are 2^4 p
[[maybe_unused]] constexpr float kSumBound = 8192.0f;   // bf16 steady state: bound on a lane's tile sum
static_assert(kBM == kAttnBlockM_BF16, "plan block size must match the kernel");

#define LDS __attribute__((address_space(3)))

// LDS serves 16 lanes x 16 bytes per clock (64 banks of 4 bytes), so the
// rows one operand read touches must land on distinct 16-byte bank slots of
// a 256-byte window.  K operand reads: 16 lanes read one chunk of 16
// consecutive rows.  V transposing reads: 32 lanes read 4 consecutive rows x
// 64 contiguous bytes.  Both swizzles permute the 16-byte chunks of a row.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// FP8 K rows are D bytes (8 or 4 chunks of 16 bytes): two (D = 128) or four
// (D = 64) rows share a 256-byte bank window, so the swizzle takes the
// remaining row bits.
template <int D>
__device__ __forceinline__ int k8_swz(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = __bf16(lo);
  const __bf16 b = __bf16(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Buffer resource over min(rows, max_rows) rows of `stride_bytes` starting at
// `base` (rows <= 0: none): loads past the last row return zeros.  32-bit
// arithmetic (the host bounds max_rows * stride_bytes) and readfirstlane keep
// it a branch-free scalar, so loads need no per-lane waterfall.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows, int max_rows,
                                                            int stride_bytes) {
  // clamp in two scalar steps: as one clamp the compiler picks the vector
  // v_med3 and reads the result back, two instructions per descriptor per tile
  int r = __builtin_amdgcn_readfirstlane(rows);
  r = r < 0 ? 0 : r;
  asm volatile("" : "+s"(r));
  r = r > max_rows ? max_rows : r;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           __builtin_amdgcn_readfirstlane(r * stride_bytes), 0x00020000);
}

// The value held by lane ^ 32 (v_permlane32_swap exchanges the two halves).
__device__ __forceinline__ float other_half(float x, int hi) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, hi ? r[0] : r[1]);
}

// max(x, value of lane ^ 32) in every lane: one v_permlane32_swap of x with
// itself leaves lanes l and l ^ 32 holding (x[l % 32], x[l % 32 + 32]) in its
// two results.  The optimiser takes the two results of swapping a value with
// itself for equal and folds the max away (keeping only the lower half's
// keys in the row max), so the second result passes through an empty asm
// that hides its value.
__device__ __forceinline__ float pair_max(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  int lo = r[0], up = r[1];
  asm volatile("" : "+v"(up));
  // compare and select: no NaN-quieting of the swapped values (fmaxf adds it)
  const float a = __builtin_bit_cast(float, lo), b = __builtin_bit_cast(float, up);
  return a > b ? a : b;
}

template <int N>
using IC = std::integral_constant<int, N>;

// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 x E4M3 with the E8M0 scales in
// byte sel_a of sa (A rows) and byte sel_b of sb (B columns); the selectors
// must be constants, so each value gets its own call.
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int sel_a, uint32_t sa, int sel_b,
                                          uint32_t sb) {
#define H3A_MF8(SA, SB) __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SA, int(sa), SB, int(sb))
  switch (sel_a * 4 + sel_b) {
    case 0: return H3A_MF8(0, 0);
    case 10: return H3A_MF8(2, 2);
    case 4: return H3A_MF8(1, 0);
    case 8: return H3A_MF8(2, 0);
    case 12: return H3A_MF8(3, 0);
    default: return H3A_MF8(0, 0);
  }
#undef H3A_MF8
}

}  // namespace

// Arguments of the fused Q norm + rotary (QNORM variant).
struct QNormArgs {
  const float* gamma;    // [D] fp32 gain of q
  const float* cos_sin;  // [2][S][half] fp32 rotary table
  int64_t S;             // rows of the table
  int32_t half;          // rot_dim / 2
  float eps;
};

// Per-block E8M0 scales of the FP8 operands (F8 >= 1), head-major so a
// tile's rows are contiguous: q [Hq][S][D/32] and k [Hkv][S][D/32] (head
// strides q_head, k_head bytes); F8 == 2 and 4 also v [Hkv][v_tiles][2][32][D/32]
// (dim 32 b + r of 32-key block j of a tile at [j][r][b]).  INT8 (F8 == 3, 4):
// q holds fp32 [Hq][S] and k fp32 [Hkv][key blocks] instead.
struct F8Scales {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  int64_t q_head;
  int64_t k_head;
  int32_t v_tiles;
};

namespace {

// RH: 16-dim blocks per rotary half when QNORM (rot_dim = 32 RH), else 0.
// F8 >= 1: q and k hold E4M3 (F8 1, 2) or INT8 (F8 3, 4) codes (token strides
// sq, sk in bytes).  F8 == 2, 4: v is the transposed E4M3 layout
// [head][dim][column], sv its row length in bytes, each item's segment
// starting at column it.vt_col0.
template <int D, bool CAUSAL, bool QNORM, int RH, int F8>
__global__ void __launch_bounds__(64 * kWaves, 2)
attn_fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, uint16_t* __restrict__ o, int64_t sq,
                     int64_t sk, int64_t sv, int64_t so, const WorkItem* __restrict__ items,
                     float c, int kv_group, QNormArgs qn, F8Scales fs, SplitArgs sp) {
  // The body uses LDS address-space pointers and gfx950-only builtins, which
  // exist only in the device pass; the host pass needs just the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 16;                      // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                      // 32-wide output dim blocks
  constexpr int CH = D / 8;                       // 16-byte chunks per row
  constexpr int ROWB = D * 2;                     // bytes per LDS row
  constexpr int NDMA = kBN * CH / (64 * kWaves);  // 16-byte loads per thread per tile and operand
  static_assert(NDMA >= 1 && CH >= 8, "tile layout");
  constexpr int KESZ = F8 >= 1 ? 1 : 2;            // bytes per K (and Q) element
  constexpr int KROWB = D * KESZ;                  // bytes per K row
  constexpr int KCH = KROWB / 16;                  // 16-byte chunks per K row
  constexpr int NDMAK = kBN * KCH / (64 * kWaves);
  constexpr int KS8 = D / 64;                      // FP8 MFMA k-steps over the head dim
  constexpr int NDMAV8 = D * 4 / (64 * kWaves);    // FP8 V^T tile: D rows x 4 chunks
  constexpr bool kF8K = F8 == 1 || F8 == 2;       // E4M3 q, k with per-32-dim scales
  constexpr bool kI8 = F8 == 3 || F8 == 4;       // INT8 q, k: per-row q, per-64-key-block k scales
  constexpr bool kPV8 = F8 == 2 || F8 == 4;       // E4M3 probabilities and V^T, FP8 PV product
  constexpr bool kPbf = !kPV8;                    // bf16 probabilities and V
  constexpr int KS32 = D / 32;                    // INT8 MFMA k-steps over the head dim
  static_assert(NDMAK >= 1 && NDMAV8 >= 1 && !(F8 && QNORM), "tile layout / variant");

  // One object per ring slot, so alias analysis can tell a load into one slot
  // from reads of another (otherwise every LDS read waits for all loads).
  __shared__ uint16_t k_slot0[kBN * KROWB / 2], k_slot1[kBN * KROWB / 2];
  __shared__ uint16_t v_slot0[kPV8 ? kBN * D / 2 : kBN * D], v_slot1[kPV8 ? kBN * D / 2 : kBN * D];
  // Slot pointers: compile-time choice for IC<> slots, a select otherwise.
  auto kslot = [&](auto slot) -> uint16_t* {
    if constexpr (std::is_integral_v<decltype(slot)>) return slot ? k_slot1 : k_slot0;
    else if constexpr (decltype(slot)::value == 0) return k_slot0;
    else return k_slot1;
  };
  auto vslot = [&](auto slot) -> uint16_t* {
    if constexpr (std::is_integral_v<decltype(slot)>) return slot ? v_slot1 : v_slot0;
    else if constexpr (decltype(slot)::value == 0) return v_slot0;
    else return v_slot1;
  };
  // F8: the block scales of a ring slot's tile, one dword per row (the row's
  // D / 32 bytes, zero-extended: an LDS-bound load narrower than a dword
  // still fills one dword per lane): the K tile's 64 keys (E4M3 scores); with
  // FP8 PV the V^T tile's (key block j, dim 32 b + r) words in lane order
  // 32 j + r.  One wave fetches each with one LDS-bound load, shared by the
  // workgroup like the tile itself.
  constexpr int SCBK = kF8K ? kBN * 4 : 4, SCBV = kPV8 ? kBN * 4 : 4;
  __shared__ __align__(16) uint8_t ks_slot0[SCBK], ks_slot1[SCBK];
  __shared__ __align__(16) uint8_t vs_slot0[SCBV], vs_slot1[SCBV];
  auto kscl = [&](auto slot) -> uint8_t* {
    if constexpr (std::is_integral_v<decltype(slot)>) return slot ? ks_slot1 : ks_slot0;
    else if constexpr (decltype(slot)::value == 0) return ks_slot0;
    else return ks_slot1;
  };
  auto vscl = [&](auto slot) -> uint8_t* {
    if constexpr (std::is_integral_v<decltype(slot)>) return slot ? vs_slot1 : vs_slot0;
    else if constexpr (decltype(slot)::value == 0) return vs_slot0;
    else return vs_slot1;
  };
  // Row `row`'s scale word.
  auto scale_word = [](const uint8_t* p, int row) -> uint32_t {
    return *(const LDS uint32_t*)((const LDS char*)p + row * 4);
  };
  // One LDS-bound load of 64 scale rows (lane i: row i) into `dst`.
  auto load_scales = [](__amdgpu_buffer_rsrc_t r, uint8_t* dst) {
    const int ln = int(threadIdx.x & 63);
    if constexpr (D == 128) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)dst, 4, ln * 4, 0, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)dst, 2, ln * 2, 0, 0, 0);
  };

  // The item is uniform over the workgroup: its fields in scalar registers,
  // so per-tile descriptor arithmetic stays on the scalar unit.
  WorkItem it = items[blockIdx.x];
  it.seg_start = __builtin_amdgcn_readfirstlane(it.seg_start);
  it.seg_len = __builtin_amdgcn_readfirstlane(it.seg_len);
  it.q_start = __builtin_amdgcn_readfirstlane(it.q_start);
  it.head = __builtin_amdgcn_readfirstlane(it.head);
  it.vt_col0 = __builtin_amdgcn_readfirstlane(it.vt_col0);
  it.kt0 = __builtin_amdgcn_readfirstlane(it.kt0);
  it.kt1 = __builtin_amdgcn_readfirstlane(it.kt1);
  it.part = __builtin_amdgcn_readfirstlane(it.part);
  if (it.seg_len <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int head_off = it.head * D;
  const int kv_off = __builtin_amdgcn_readfirstlane(it.head / kv_group) * D;
  const int qrow0 = it.q_start + wave * 32;
  const bool active = qrow0 < it.seg_len;

  // Q as the B operand: lane holds query (qrow0 + l32), dims ks*16 + hi*8 .. +8.
  bf16x8 qb[KS];
  // F8: lane holds query (qrow0 + l32), dims ks8*64 + hi*16 .. +16 and
  // ks8*64 + 32 + hi*16 .. +16; qsc: the row's scales, shifted so that byte
  // 2 ks8 is block 2 ks8 + hi.
  [[maybe_unused]] i32x8 qb8[kF8K ? KS8 : 1];
  [[maybe_unused]] uint32_t qsc = 0;
  // kI8: lane holds query (qrow0 + l32), dims ks*32 + hi*16 .. +16, and the
  // score multiplier c times the row's scale.
  [[maybe_unused]] i32x4 qi8[kI8 ? KS32 : 1];
  [[maybe_unused]] float cq = c;
  const int kv_head = __builtin_amdgcn_readfirstlane(it.head / kv_group);
  if constexpr (F8 == 0) {
    const auto rq = rows_rsrc(q + (int64_t(it.seg_start) + qrow0) * sq + head_off, it.seg_len - qrow0, 32, int(sq) * 2);
    const int off = (l32 * int(sq) + hi * 8) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off + ks * 32, 0, 0));
  } else if constexpr (kI8) {
    const uint8_t* q8 = reinterpret_cast<const uint8_t*>(q);
    const auto rq = rows_rsrc(q8 + (int64_t(it.seg_start) + qrow0) * sq + head_off, it.seg_len - qrow0, 32, int(sq));
    const int off = l32 * int(sq) + hi * 16;
#pragma unroll
    for (int ks = 0; ks < KS32; ++ks)
      qi8[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off + ks * 32, 0, 0));
    // the row's fp32 scale ([head][token]); rows past the segment end read 0
    const auto rqs = rows_rsrc(fs.q + it.head * fs.q_head + (int64_t(it.seg_start) + qrow0) * 4, it.seg_len - qrow0,
                               32, 4);
    cq = c * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rqs, l32 * 4, 0, 0));
  } else {
    const uint8_t* q8 = reinterpret_cast<const uint8_t*>(q);
    const auto rq = rows_rsrc(q8 + (int64_t(it.seg_start) + qrow0) * sq + head_off, it.seg_len - qrow0, 32, int(sq));
    const int off = l32 * int(sq) + hi * 16;
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      const auto lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off + ks * 64, 0, 0);
      const auto up = __builtin_amdgcn_raw_buffer_load_b128(rq, off + ks * 64 + 32, 0, 0);
      qb8[ks] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(up[0]), int(up[1]), int(up[2]), int(up[3])};
    }
    // rows past the segment end read scale code 0 (their codes are 0 too)
    const auto rqs = rows_rsrc(fs.q + it.head * fs.q_head + (int64_t(it.seg_start) + qrow0) * (D / 32),
                               it.seg_len - qrow0, 32, D / 32);
    const uint32_t w = D == 128 ? __builtin_amdgcn_raw_buffer_load_b32(rqs, l32 * 4, 0, 0)
                                : uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rqs, l32 * 2, 0, 0));
    qsc = w >> (8 * hi);
  }
  // QNORM operands (the gain of each of the lane's dims, cos/sin of its
  // rotated pairs) load together with Q, so their latency overlaps; the
  // arithmetic (qnorm_apply) runs once the first K/V tiles are in flight.
  // The lane holds 16-byte chunks 2 ks + hi (dims (2 ks + hi) * 8 .. +7) of
  // its query row, half the row; the other half is in lane ^ 32.  Chunk
  // 2 ks + hi (ks < RH) pairs with chunk 2 (ks + RH) + hi: the partner dim is
  // i + rot_dim / 2, in the same lane.
  static_assert(2 * RH <= KS, "rotary dims exceed the head");
  [[maybe_unused]] float qg[QNORM ? KS : 1][8];
  [[maybe_unused]] float qc[RH > 0 ? RH : 1][8];
  [[maybe_unused]] float qs[RH > 0 ? RH : 1][8];
  if constexpr (QNORM) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4* gp = reinterpret_cast<const float4*>(qn.gamma + (2 * ks + hi) * 8);
      const float4 g0 = gp[0], g1 = gp[1];
      qg[ks][0] = g0.x; qg[ks][1] = g0.y; qg[ks][2] = g0.z; qg[ks][3] = g0.w;
      qg[ks][4] = g1.x; qg[ks][5] = g1.y; qg[ks][6] = g1.z; qg[ks][7] = g1.w;
    }
    // Rows past the segment end read a valid table row (their outputs are
    // not stored).
    const int64_t trow = int64_t(it.seg_start) + min(qrow0 + l32, it.seg_len - 1);
#pragma unroll
    for (int ks = 0; ks < RH; ++ks) {
      const float4* cp = reinterpret_cast<const float4*>(qn.cos_sin + trow * qn.half + (2 * ks + hi) * 8);
      const float4* sp = reinterpret_cast<const float4*>(qn.cos_sin + (qn.S + trow) * qn.half + (2 * ks + hi) * 8);
      const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
      qc[ks][0] = c0.x; qc[ks][1] = c0.y; qc[ks][2] = c0.z; qc[ks][3] = c0.w;
      qc[ks][4] = c1.x; qc[ks][5] = c1.y; qc[ks][6] = c1.z; qc[ks][7] = c1.w;
      qs[ks][0] = s0.x; qs[ks][1] = s0.y; qs[ks][2] = s0.z; qs[ks][3] = s0.w;
      qs[ks][4] = s1.x; qs[ks][5] = s1.y; qs[ks][6] = s1.z; qs[ks][7] = s1.w;
    }
  }
  // RMSNorm + rotary of qb in place, operation for operation as the
  // standalone kernel: per-chunk FMA chains for the sum of squares, its
  // shuffle-xor tree (chunk bits 3..1 are ks bits here, bit 0 is the lane
  // half), the same rotation FMAs, one RNE rounding.
  [[maybe_unused]] auto qnorm_apply = [&]() {
    float p[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(float(qb[ks][e]), float(qb[ks][e]), ss);
      p[ks] = ss;
    }
#pragma unroll
    for (int m = KS / 2; m >= 1; m >>= 1) {
      float t[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) t[ks] = p[ks] + p[ks ^ m];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) p[ks] = t[ks];
    }
    const float ssum = p[0] + other_half(p[0], hi);
    const float r = 1.0f / sqrtf(ssum * (1.0f / float(D)) + qn.eps);
    float y[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) y[ks][e] = float(qb[ks][e]) * r * qg[ks][e];
#pragma unroll
    for (int ks = 0; ks < RH; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = y[ks][e], b = y[ks + RH][e];
        y[ks][e] = fmaf(a, qc[ks][e], -b * qs[ks][e]);
        y[ks + RH][e] = fmaf(b, qc[ks][e], a * qs[ks][e]);
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[ks][e] = __bf16(y[ks][e]);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -1e30f;  // reference max of scale*log2(e)*score
  // Kept with it (updated only where m_run moves, not per tile): the bound
  // past which a tile max raises it, and the FP8 PV exponent offset.
  constexpr float kSlack = kPV8 ? kRescaleSlackF8 : kRescaleSlack;
  float m_thr = m_run + kSlack;
  [[maybe_unused]] float m_off = kProbOffsetF8 - m_run;
  float l_run = 0.f;     // this lane's partial row sum (its 16-of-32 keys)
  // FP8 PV: the row sums come from the matrix core instead -- an all-ones
  // A operand against the E4M3 probabilities puts sum_k p[k][q] in every
  // register of lane q (both halves), the same weights PV applies.
  [[maybe_unused]] f32x16 lacc = f32x16{};
  // The all-ones A operand (four E4M3 ones per dword), built once: opaque to
  // the compiler so it stays in registers instead of being rebuilt per tile.
  [[maybe_unused]] i32x8 ones8;
  if constexpr (kPV8) {
    const int one4 = 0x38383838;
    ones8 = i32x8{one4, one4, one4, one4, one4, one4, one4, one4};
    asm volatile("" : "+v"(ones8));
  }
  // kI8: the INT8 score product starts from the bits of the float 1.5 * 2^23,
  // so an integer sum S (|S| < 2^22) reads as the float 1.5 * 2^23 + S: the
  // probabilities then take it straight into their FMA, exp2(c_t * (1.5 *
  // 2^23 + S) - (c_t * 1.5 * 2^23 + m)), with c_t = c * q_scale * k_scale of
  // the tile; an exact integer-to-float conversion at no instruction cost.
  // Kept in registers (opaque to the compiler), like ones8.
  [[maybe_unused]] i32x16 magic;
  if constexpr (kI8) {
    constexpr int m = 0x4B400000;
    magic = i32x16{m, m, m, m, m, m, m, m, m, m, m, m, m, m, m, m};
    if constexpr (!kPV8) asm volatile("" : "+v"(magic));
  }
  // Score multiplier and offset of the tile whose probabilities are formed
  // next: scores are sacc * cmul + cadd (c and 0 but for kI8).  kI8: the k
  // scale of the tile in K ring slot j arrives in kscale[j] with the tile's
  // K load, two tiles before its scores are formed.
  [[maybe_unused]] float cmul = c, cadd = 0.f;
  [[maybe_unused]] float kscale[2] = {0.f, 0.f};
  [[maybe_unused]] auto set_tile_scale = [&](auto slot) {
    if constexpr (kI8) {
      float ks;
      if constexpr (std::is_integral_v<decltype(slot)>) ks = slot ? kscale[1] : kscale[0];
      else ks = kscale[decltype(slot)::value];
      cmul = cq * ks;
      cadd = -cmul * 12582912.0f;
    }
  };

  // LDS-bound loads: slot s = (i * kWaves + wave) * 64 + lane holds physical
  // chunk s % CH of row s / CH; the lane fetches the logical chunk stored there.
  int koff[NDMAK], voff[NDMA];
#pragma unroll
  for (int i = 0; i < NDMAK; ++i) {
    const int s = (i * kWaves + wave) * 64 + lane;
    const int row = s / KCH, pc = s % KCH;
    koff[i] = row * int(sk) * KESZ + ((pc ^ (F8 ? k8_swz<D>(row) : k_swz<D>(row))) * 16);
  }
  if constexpr (kPbf) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int s = (i * kWaves + wave) * 64 + lane;
      const int row = s / CH, pc = s % CH;
      voff[i] = row * int(sv) * 2 + ((pc ^ v_swz<D>(row)) * 16);
    }
  } else {
    // V^T tile: row = dim (64 bytes: 4 chunks), swizzled like 64-byte K rows
#pragma unroll
    for (int i = 0; i < NDMAV8; ++i) {
      const int s = (i * kWaves + wave) * 64 + lane;
      const int row = s / 4, pc = s % 4;
      voff[i] = row * int(sv) + ((pc ^ ((row >> 2) & 3)) * 16);
    }
  }
  // K operand reads: row l32 (+32 kb), logical chunk 2 ks + hi.
  int kaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kaddr[ks] = l32 * ROWB + (((2 * ks + hi) ^ k_swz<D>(l32)) * 16);
  // F8 K operand reads: row l32 (+32 kb), chunks 4 ks8 + hi + {0, 2}.
  [[maybe_unused]] int kaddr8[kF8K ? KS8 : 1][2];
  if constexpr (kF8K)
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) kaddr8[ks][j] = l32 * KROWB + (((4 * ks + hi + 2 * j) ^ k8_swz<D>(l32)) * 16);
  // INT8 K operand reads: row l32 (+32 kb), chunk 2 ks + hi.
  [[maybe_unused]] int kaddr_i8[kI8 ? KS32 : 1];
  if constexpr (kI8)
#pragma unroll
    for (int ks = 0; ks < KS32; ++ks) kaddr_i8[ks] = l32 * KROWB + (((2 * ks + hi) ^ k8_swz<D>(l32)) * 16);
  // V^T operand reads (transposing): 16-lane group g reads keys
  // kk*16 + 4 (g / 2) + {0..3} (and +8) at dims db*32 + 16 (g % 2) + 0..15;
  // lane m of the group addresses row m / 4, columns 4 (m % 4) .. +3.
  int vaddr[DB];
  // FP8 V^T operand reads: row db*32 + l32, chunks hi + {0, 2}.
  [[maybe_unused]] int vaddr8[kPV8 ? DB : 1][2];
  if constexpr (kPV8)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = db * 32 + l32;
        vaddr8[db][j] = row * 64 + (((hi + 2 * j) ^ ((row >> 2) & 3)) * 16);
      }
  {
    const int g = lane >> 4, m = lane & 15;
    const int row = 4 * (g >> 1) + (m >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int lc = db * 4 + 2 * (g & 1) + ((m & 3) >> 1);
      vaddr[db] = row * ROWB + ((lc ^ v_swz<D>(row)) * 16) + 8 * (m & 1);
    }
  }

  const char* kbase = reinterpret_cast<const char*>(k) + (int64_t(it.seg_start) * sk + kv_off) * KESZ;
  const char* vbase = kPV8 ? reinterpret_cast<const char*>(v) + int64_t(kv_off) * sv + it.vt_col0
                              : reinterpret_cast<const char*>(v + int64_t(it.seg_start) * sv + kv_off);
  // Keys the item needs: the whole segment, or (causal) up to its last row.
  const int nkeys = CAUSAL ? min(it.seg_len, it.q_start + kBM) : it.seg_len;
  const int ntiles = (nkeys + kBN - 1) / kBN;
  // This item's key tiles [tb, te): all of them, or one range of a split item
  // (tb even, so every tile keeps the ring slot parity t & 1).
  const int tb = it.kt1 > 0 ? it.kt0 : 0;
  const int te = it.kt1 > 0 ? min(it.kt1, ntiles) : ntiles;
  // First key tile that crosses the causal diagonal of the item's rows.
  [[maybe_unused]] const int tdiag = it.q_start / kBN;

  // ---- building blocks ------------------------------------------------------
  auto load_k = [&](int t, auto slot) {
    const int key0 = t * kBN;
    const auto r = rows_rsrc(kbase + int64_t(key0) * sk * KESZ, it.seg_len - key0, kBN, int(sk) * KESZ);
#pragma unroll
    for (int i = 0; i < NDMAK; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(kslot(slot) + (i * kWaves + wave) * 64 * 8), 16,
                                               koff[i], 0, 0, 0);
    if constexpr (kF8K) {
      // the tile's 64 scale rows, contiguous (head-major scales): lane = key;
      // keys past the segment end read scale code 0 (their codes are 0 too)
      if (wave == 0) {
        const auto rs = rows_rsrc(fs.k + kv_head * fs.k_head + (int64_t(it.seg_start) + key0) * (D / 32),
                                  it.seg_len - key0, kBN, D / 32);
        load_scales(rs, kscl(slot));
      }
    }
    if constexpr (kI8) {
      // the tile's k scale ([kv head][key block], the segment's first block at
      // vt_col0 / 64), one fp32 for every lane; past the segment: 0
      const auto rs = rows_rsrc(fs.k + kv_head * fs.k_head + int64_t(it.vt_col0 / kVtTile) * 4,
                                (it.seg_len + kBN - 1) / kBN, 1 << 20, 4);
      const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, t * 4, 0, 0));
      if constexpr (std::is_integral_v<decltype(slot)>) {
        if (slot) kscale[1] = x;
        else kscale[0] = x;
      } else {
        kscale[decltype(slot)::value] = x;
      }
    }
  };
  auto load_v = [&](int t, auto slot) {
    const int key0 = t * kBN;
    if constexpr (kPbf) {
      const auto r = rows_rsrc(vbase + int64_t(key0) * sv * 2, it.seg_len - key0, kBN, int(sv) * 2);
#pragma unroll
      for (int i = 0; i < NDMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(vslot(slot) + (i * kWaves + wave) * 64 * 8), 16,
                                                 voff[i], 0, 0, 0);
    } else {
      // D rows of sv bytes from the tile's first column; padding columns hold 0
      const auto r = rows_rsrc(vbase + key0, D, D, int(sv));
#pragma unroll
      for (int i = 0; i < NDMAV8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(vslot(slot) + (i * kWaves + wave) * 64 * 8), 16,
                                                 voff[i], 0, 0, 0);
      // the tile's 64 scale words (lane (l32, hi): dims 32 b + l32 of key
      // block hi, byte b), fetched by another wave than the K scales
      if (wave == 1 % kWaves) {
        const uint8_t* vs = fs.v + (int64_t(kv_head) * fs.v_tiles + it.vt_col0 / kVtTile + t) * 64 * (D / 32);
        const auto r = rows_rsrc(vs, 64, 64, D / 32);
        load_scales(r, vscl(slot));
      }
    }
  };
  // S^T = K Q^T for the K tile in `slot` (an IC<> for immediate offsets).
  auto qk = [&](auto slot, f32x16* sacc) {
    if constexpr (F8 == 0) {
      // k-steps outer, the 32-key blocks inner (independent accumulators back
      // to back), each step's K operands read while the previous step's
      // products issue
      constexpr int NB = kBN / 32;
      const LDS char* kp = (const LDS char*)kslot(slot);
      bf16x8 cur[NB], nxt[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        sacc[kb] = f32x16{};
        cur[kb] = *(const LDS bf16x8*)(kp + kaddr[0] + kb * 32 * ROWB);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS)
#pragma unroll
          for (int kb = 0; kb < NB; ++kb) nxt[kb] = *(const LDS bf16x8*)(kp + kaddr[ks + 1] + kb * 32 * ROWB);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[kb], qb[ks], sacc[kb], 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) cur[kb] = nxt[kb];
      }
      return;
    }
    if constexpr (kI8) {
      // as the bf16 product: k-steps outer, 32-key blocks inner, each step's K
      // operands read while the previous step's products issue
      constexpr int NB = kBN / 32;
      const LDS char* kp = (const LDS char*)kslot(slot);
      i32x16 acc[NB];
      i32x4 cur[NB], nxt[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) cur[kb] = *(const LDS i32x4*)(kp + kaddr_i8[0] + kb * 32 * KROWB);
#pragma unroll
      for (int ks = 0; ks < KS32; ++ks) {
        if (ks + 1 < KS32)
#pragma unroll
          for (int kb = 0; kb < NB; ++kb) nxt[kb] = *(const LDS i32x4*)(kp + kaddr_i8[ks + 1] + kb * 32 * KROWB);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
          acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur[kb], qi8[ks], ks == 0 ? magic : acc[kb], 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) cur[kb] = nxt[kb];
      }
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) sacc[kb] = __builtin_bit_cast(f32x16, acc[kb]);
      return;
    }
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      sacc[kb] = f32x16{};
      // key 32 kb + l32's word; byte 2 ks after the shift: dim block 2 ks + hi
      const uint32_t ks_w = scale_word(kscl(slot), 32 * kb + l32) >> (8 * hi);
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const LDS char* kp = (const LDS char*)kslot(slot) + kb * 32 * KROWB;
        const uint4 lo = *(const LDS uint4*)(kp + kaddr8[ks][0]);
        const uint4 up = *(const LDS uint4*)(kp + kaddr8[ks][1]);
        const i32x8 a = {int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(up.x), int(up.y), int(up.z), int(up.w)};
        sacc[kb] = mfma_f8(a, qb8[ks], sacc[kb], 2 * ks, ks_w, 2 * ks, qsc);
      }
    }
  };
  // Keys of tile `tt` past the segment end, or (causal) past the lane's
  // query row, get -inf.  The lane's key offset hi*4 is folded into one
  // bound, so every compare is against a constant.
  auto mask = [&](f32x16* sacc, int tt) {
    if constexpr (kI8) {
      // A zero score multiplier (an all-zero q row or k block, or rows past
      // the segment end) would turn a masked key's -inf into -inf * 0 = NaN:
      // in a masked tile it takes the smallest normal instead (every such
      // score is 0 exactly, or at most 2^22 * 2^-126 from it, a probability of
      // 1 against the reference either way).  A NaN multiplier stays NaN.
      // Only the tiles that hold masked keys pay for this check.
      if (cmul < 1.17549435e-38f) {
        cmul = 1.17549435e-38f;
        cadd = -cmul * 12582912.0f;
      }
    }
    int lim = it.seg_len - tt * kBN - 1;  // last key of the tile inside the segment
    if constexpr (CAUSAL) lim = min(lim, qrow0 + l32 - tt * kBN);
    lim -= hi * 4;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + (r >> 2) * 8 + (r & 3) > lim) sacc[kb][r] = -__builtin_inff();
  };
  // Does key tile `tt` need the mask?
  auto needs_mask = [&](int tt) {
    return (tt + 1) * kBN > it.seg_len || (CAUSAL && tt >= tdiag);
  };
  // Tile max; the reference max m_run only moves when a query's tile max
  // exceeds it by more than kRescaleSlack (log2 units), so probabilities stay
  // below 2^kRescaleSlack and most tiles skip the rescale.  Exact: numerator
  // and denominator share the reference.  Must run after every PV product
  // issued with the old reference.
  auto update_max = [&](const f32x16* sacc) {
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    if constexpr (kI8) mx = fmaf(pair_max(mx), cmul, cadd);
    else mx = pair_max(mx) * c;
    const bool grow = mx > m_thr;
    if (__builtin_expect(__any(grow), 0)) {
      // Rare after the first tiles; the empty asm keeps the compiler from
      // speculating the accumulator rescale onto every tile.
      asm volatile("" ::: "memory");
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 where unchanged
      m_run = m_new;
      m_thr = m_run + kSlack;
      if constexpr (kPV8) m_off = kProbOffsetF8 - m_run;
      l_run *= alpha;
      if constexpr (kPV8) lacc *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
  };
  // p = 2^(c*s - m_run), rounded to bf16 for the PV product, for one tile;
  // returns the lane's sum of the rounded values (v_dot2 against (1, 1)), so
  // the normaliser matches the weights actually applied to V.
  auto probs_part = [&](const f32x16* sacc, bf16x8* pb) {
    const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
    float part = 0.f;
    float mul = c, bias = -m_run;
    if constexpr (kI8) {
      mul = cmul;
      bias = cadd - m_run;
    }
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 v8;
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = __bf16(__builtin_amdgcn_exp2f(fmaf(sacc[kb][hh * 8 + i], mul, bias)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 pr = {v8[2 * i], v8[2 * i + 1]};
          part = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, part, false);
        }
        pb[kb * 2 + hh] = v8;
      }
    return part;
  };
  // With bf16 probabilities the steady state takes no per-tile max: the
  // reference m_run only has to
  // keep every probability bounded, and a lane's sum `part` of its 32
  // probabilities bounds each of them.  When some lane's sum exceeds
  // kSumBound (a probability may be large, or infinite), the tile's true row
  // max raises the reference, the output and row sum are rescaled, and the
  // tile is recomputed; this is exact, as numerator and denominator share the
  // reference.  Otherwise every probability is at most kSumBound.  Must run
  // before the tile's PV product is issued.
  auto probs_checked = [&](const f32x16* sacc, bf16x8* pb, float part) {
    if (__builtin_expect(__any(!(part <= kSumBound)), 0)) {
      asm volatile("" ::: "memory");  // keep the rare path a real branch
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      if constexpr (kI8) mx = fmaf(pair_max(mx), cmul, cadd);
      else mx = pair_max(mx) * c;
      const float m_new = mx > m_run ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 where unchanged
      m_run = m_new;
      m_thr = m_run + kSlack;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      part = probs_part(sacc, pb);
    }
    l_run += part;
  };
  auto probs = [&](const f32x16* sacc, bf16x8* pb) {
    if constexpr (kPV8) {
      // E4M3 weights 2^4 p (p <= 2^4 against the reference, so <= 256), dword
      // g = keys 8g + 4 hi + {0..3}; INT8 scores: s * cmul + cadd
      const float mul = kI8 ? cmul : c;
      const float moff = kI8 ? cadd + m_off : m_off;
      int d[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        float p4[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) p4[w] = __builtin_amdgcn_exp2f(fmaf(sacc[g / 4][4 * (g % 4) + w], mul, moff));
        // bytes 2-3 of the first conversion's destination are overwritten by
        // the second, so any value serves as its prior contents
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], __builtin_bit_cast(int, p4[0]), false);
        d[g] = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], pk, true);
      }
      // Swap dwords 2, 3, 6, 7 of the low half with dwords 0, 1, 4, 5 of the
      // high half: afterwards B dword m of half hi holds keys
      // 32 (m / 4) + 16 hi + 4 (m % 4) + {0..3}, the instruction's numbering.
      int b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = (i / 2) * 4 + i % 2;  // 0, 1, 4, 5
        const auto sw = __builtin_amdgcn_permlane32_swap(d[x], d[x + 2], false, false);
        b[2 * i] = sw[0];
        b[2 * i + 1] = sw[1];
      }
      pb[0] = __builtin_bit_cast(bf16x8, make_int4(b[0], b[1], b[2], b[3]));
      pb[1] = __builtin_bit_cast(bf16x8, make_int4(b[4], b[5], b[6], b[7]));
      return;
    }
    l_run += probs_part(sacc, pb);
  };
  // O^T += V^T P^T for the V tile in `slot`.
  auto pv = [&](auto slot, const bf16x8* pb) {
    if constexpr (kPV8) {
      const int4 b0 = __builtin_bit_cast(int4, pb[0]), b1 = __builtin_bit_cast(int4, pb[1]);
      const i32x8 b = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      const uint32_t vs_w = scale_word(vscl(slot), lane);  // byte db: dim block db, key block hi
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const LDS char* vp = (const LDS char*)vslot(slot);
        const uint4 lo = *(const LDS uint4*)(vp + vaddr8[db][0]);
        const uint4 up = *(const LDS uint4*)(vp + vaddr8[db][1]);
        const i32x8 a = {int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(up.x), int(up.y), int(up.z), int(up.w)};
        oacc[db] = mfma_f8(a, b, oacc[db], db, vs_w, 0, 127u);
      }
      lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, b, lacc, 0, 0, 0, 127, 0, 127);
      return;
    }
    // Products in (16-key step, dim block) order, so consecutive MFMAs use
    // different accumulators; each V^T operand is read two products ahead.
    constexpr int NP = DB * (kBN / 16);
    auto read_vt = [&](int i) {
      const int kk = i / DB, db = i % DB;
      const LDS char* p0 = (const LDS char*)vslot(slot) + vaddr[db] + kk * 16 * ROWB;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS bf16x4*)(p0));
      const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS bf16x4*)(p0 + 8 * ROWB));
      return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 op[3];
    op[0] = read_vt(0);
    op[1] = read_vt(1);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + 2 < NP) op[(i + 2) % 3] = read_vt(i + 2);
      oacc[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % 3], pb[i / DB], oacc[i % DB], 0, 0, 0);
    }
  };
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's LDS-bound loads landed
    __syncthreads();
  };

  // ---- software-pipelined tile loop -----------------------------------------
  // Entering iteration t: `s` holds the scores of tile t with the running max
  // already updated for it, K_{t+1} sits in K slot (t+1) % 2 and V_t in V slot
  // t % 2.  The iteration loads K_{t+2} and V_{t+1} into the slots freed by
  // the previous iteration, turns tile t's scores into probabilities while the
  // MFMA pipe computes tile t+1's scores, then accumulates tile t's PV product
  // while the VALU reduces tile t+1's max.
  f32x16 s[kBN / 32];
  bf16x8 pb[kBN / 16];
  load_k(tb, IC<0>{});
  load_v(tb, IC<0>{});
  if (te > tb + 1) load_k(tb + 1, IC<1>{});
  if constexpr (QNORM) qnorm_apply();
  publish();
  // Every wave computes the first scores, also one whose rows all lie past
  // the segment end: its Q rows read as zeros, so its scores are 0 (or -inf
  // where masked) and the steady loop below, which every wave runs, starts
  // from defined scores and a finite reference.
  qk(IC<0>{}, s);
  set_tile_scale(IC<0>{});
  if (needs_mask(tb)) mask(s, tb);
  update_max(s);
  // Iteration 0 reloads K slot 0: every wave must be done reading K_0 first.
  __syncthreads();

  // Steady state: tiles t and t+1 both exist and t+1 is not the last, so
  // tile t+1 is full and K_{t+2} exists.  Two iterations per trip fix the
  // slot parities as immediates.  No tile computed here needs a mask: a trip
  // at t computes the scores of tiles t+1 and t+2, which stay below
  // ntiles - 1 (bidirectional: only the last tile can be partial) or below
  // ntiles - 2 (causal: the diagonal tiles are the last two).
  auto steady = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    load_k(t + 2, IC<P>{});
    load_v(t + 1, IC<P ^ 1>{});
    // Every wave computes here, also one whose rows all lie past the segment
    // end (rare: last query tile only; its rows are not stored), so the loads
    // and the MFMA/softmax work form one block the scheduler can interleave.
    if constexpr (kPbf) {
      // bf16 probabilities (also behind FP8 or INT8 scores): tile t's
      // probabilities beside tile t+1's scores; the check (rarely taken)
      // still sees tile t's scores in sold
      const f32x16 sold[kBN / 32] = {s[0], s[1]};
      const float part = probs_part(sold, pb);
      qk(IC<P ^ 1>{}, s);
      probs_checked(sold, pb, part);
      pv(IC<P>{}, pb);
    } else {
      probs(s, pb);
      qk(IC<P ^ 1>{}, s);
      pv(IC<P>{}, pb);
      set_tile_scale(IC<P ^ 1>{});  // (kI8) tile t+1's, for its max
      update_max(s);
    }
    publish();
    if constexpr (kPbf) set_tile_scale(IC<P ^ 1>{});  // (kI8) tile t+1's, for the next iteration
  };
  int t = tb;
  constexpr int kTail = CAUSAL ? 4 : 3;
  for (; t + kTail < te; t += 2) {
    steady(t, IC<0>{});
    steady(t + 1, IC<1>{});
  }
  // Remaining iterations (at most kTail), with slot parity in a register.
  for (; t < te; ++t) {
    const int par = t & 1;
    if (t + 2 < te) load_k(t + 2, par);
    if (t + 1 < te) load_v(t + 1, par ^ 1);
    if (active) {
      if constexpr (kPbf) probs_checked(s, pb, probs_part(s, pb));
      else probs(s, pb);
      if (t + 1 < te) {
        qk(par ^ 1, s);
        pv(par, pb);
        set_tile_scale(par ^ 1);
        if (needs_mask(t + 1)) mask(s, t + 1);
        update_max(s);
      } else {
        pv(par, pb);
      }
    }
    publish();
  }

  if (!active) return;
  const int qi = qrow0 + l32;
  const float l_tot = kPV8 ? lacc[0] : l_run + other_half(l_run, hi);
  if (it.part > 0) {
    if (qi >= it.seg_len) return;
    // one key range of a split item: unnormalised rows, their reference max
    // and row sum, for the merge pass
    const int64_t row = int64_t(it.part - 1) * kBM + wave * 32 + l32;
    float* po = sp.o + row * D + hi * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + db * 32 + g * 8) =
            make_float4(oacc[db][g * 4 + 0], oacc[db][g * 4 + 1], oacc[db][g * 4 + 2], oacc[db][g * 4 + 3]);
    if (hi == 0) *reinterpret_cast<float2*>(sp.ml + 2 * row) = make_float2(m_run, l_tot);
    return;
  }
  // The normalised rows go through LDS so that every global store writes
  // whole 16-byte pieces of rows (64 / NCH rows per instruction) instead of
  // 8 bytes in each of 32 rows.  Each wave stages its 32 rows (32 x D bf16)
  // in one ring slot of its own: every wave has passed the last barrier after
  // its last operand read and its K/V loads have landed, so the ring is free.
  // 16-byte chunks are swizzled by row so both phases spread over the banks.
  constexpr int NCH = D / 8;  // 16-byte chunks per output row
  static_assert(32 * D * 2 <= kBN * KROWB && 32 * D * 2 <= (kPV8 ? kBN * D : kBN * D * 2), "staging fits a slot");
  LDS char* stage = (LDS char*)(wave == 0 ? k_slot0 : wave == 1 ? k_slot1 : wave == 2 ? v_slot0 : v_slot1);
  const float inv = 1.0f / l_tot;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk;
      pk.x = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      pk.y = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      const int ch = (db * 4 + g) ^ (l32 & (NCH - 1));
      *(LDS uint2*)(stage + l32 * (D * 2) + ch * 16 + hi * 8) = pk;
    }
  // the wave's LDS writes complete before its reads (one wave, in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int RPI = 64 / NCH;  // rows per store instruction
  const int oc = lane % NCH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / NCH;
    const uint4 v4 = *(const LDS uint4*)(stage + r * (D * 2) + ((oc ^ (r & (NCH - 1))) * 16));
    if (qrow0 + r < it.seg_len)
      *reinterpret_cast<uint4*>(o + int64_t(it.seg_start + qrow0 + r) * so + head_off + oc * 8) = v4;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool CAUSAL, bool QNORM = false, int RH = 0, int F8 = 0>
hipError_t launch(const void* q, const void* k, const void* v, void* o, int64_t sq, int64_t sk,
                  int64_t sv, int64_t so, const WorkItem* items, int64_t n_items, float scale,
                  int kv_group, const QNormArgs& qn, hipStream_t stream, const F8Scales& fs = F8Scales{},
                  const SplitArgs& sp = SplitArgs{}) {
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, QNORM, RH, F8>), dim3(unsigned(n_items)), dim3(64 * kWaves), 0,
                     stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), sq, sk, sv, so, items, c,
                     kv_group, qn, fs, sp);
  return hipGetLastError();
}

// Merge of a split item's partial rows: with m_p, l_p, o_p the reference max,
// row sum and unnormalised row of key range p (all relative to 2^m_p), the
// row over all keys is sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M =
// max_p m_p -- the streaming softmax's own rescale step, applied once per
// range in key order (deterministic).  One workgroup per split item; each
// thread produces 8 dims of a row at a time.
constexpr int kMergeThreads = 256;

template <int D>
__global__ void __launch_bounds__(kMergeThreads)
attn_merge_kernel(const MergeItem* __restrict__ merges, SplitArgs sp, uint16_t* __restrict__ o, int64_t so) {
  const MergeItem g = merges[blockIdx.x];
  const int rows = min(kBM, g.seg_len - g.q_start);
  constexpr int CPR = D / 8;  // 8-dim chunks per row
  for (int u = threadIdx.x; u < rows * CPR; u += kMergeThreads) {
    const int r = u / CPR, ch = u % CPR;
    float M = -INFINITY;
    for (int p = 0; p < g.nparts; ++p) M = fmaxf(M, sp.ml[2 * (int64_t(g.part0 + p) * kBM + r)]);
    float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < g.nparts; ++p) {
      const int64_t row = int64_t(g.part0 + p) * kBM + r;
      const float2 ml = *reinterpret_cast<const float2*>(sp.ml + 2 * row);
      const float w = exp2f(ml.x - M);
      L = fmaf(w, ml.y, L);
      const float4* src = reinterpret_cast<const float4*>(sp.o + row * D + ch * 8);
      const float4 a = src[0], b = src[1];
      acc[0] = fmaf(w, a.x, acc[0]); acc[1] = fmaf(w, a.y, acc[1]);
      acc[2] = fmaf(w, a.z, acc[2]); acc[3] = fmaf(w, a.w, acc[3]);
      acc[4] = fmaf(w, b.x, acc[4]); acc[5] = fmaf(w, b.y, acc[5]);
      acc[6] = fmaf(w, b.z, acc[6]); acc[7] = fmaf(w, b.w, acc[7]);
    }
    const float inv = 1.0f / L;
    uint4 pk;
    pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    pk.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
    pk.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
    *reinterpret_cast<uint4*>(o + int64_t(g.seg_start + g.q_start + r) * so + g.head * D + ch * 8) = pk;
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int32_t D,
                                int64_t sq, int64_t sk, int64_t sv, int64_t so,
                                const WorkItem* items, int64_t n_items, float scale,
                                int32_t kv_group, bool causal, hipStream_t stream, const SplitArgs& sp) {
  if (n_items <= 0) return hipSuccess;
  if (kv_group < 1) return hipErrorInvalidValue;
  const QNormArgs none{};
  const F8Scales nofs{};
  if (D == 128)
    return causal ? launch<128, true>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, none, stream, nofs, sp)
                  : launch<128, false>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, none, stream, nofs, sp);
  if (D == 64)
    return causal ? launch<64, true>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, none, stream, nofs, sp)
                  : launch<64, false>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, none, stream, nofs, sp);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const MergeItem* merges, int64_t n_merges, const SplitArgs& sp, void* o, int32_t D,
                             int64_t so, hipStream_t stream) {
  if (n_merges <= 0) return hipSuccess;
  if (n_merges > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  if (D == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(unsigned(n_merges)), dim3(kMergeThreads), 0, stream, merges, sp,
                       static_cast<uint16_t*>(o), so);
  else if (D == 64)
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(unsigned(n_merges)), dim3(kMergeThreads), 0, stream, merges, sp,
                       static_cast<uint16_t*>(o), so);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_fwd_fp8qk(const void* q8, const void* k8, const void* q8s, const void* k8s, const void* v,
                                 void* o, int32_t D, int64_t sq, int64_t sk, int64_t sqs, int64_t sks, int64_t sv,
                                 int64_t so, const WorkItem* items, int64_t n_items, float scale, int32_t kv_group,
                                 bool causal, hipStream_t stream, const SplitArgs& sp) {
  if (n_items <= 0) return hipSuccess;
  if (kv_group < 1) return hipErrorInvalidValue;
  const QNormArgs none{};
  const F8Scales fs{static_cast<const uint8_t*>(q8s), static_cast<const uint8_t*>(k8s), nullptr, sqs, sks, 0};
#define H3A_F8_CASE(DD)                                                                                     \
  if (D == DD)                                                                                              \
    return causal ? launch<DD, true, false, 0, 1>(q8, k8, v, o, sq, sk, sv, so, items, n_items, scale,        \
                                                  kv_group, none, stream, fs, sp)                          \
                  : launch<DD, false, false, 0, 1>(q8, k8, v, o, sq, sk, sv, so, items, n_items, scale,       \
                                                   kv_group, none, stream, fs, sp);
  H3A_F8_CASE(128) H3A_F8_CASE(64)
#undef H3A_F8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, const void* q8s, const void* k8s,
                               const void* vt8s, void* o, int32_t D, int64_t sq, int64_t sk, int64_t sqs, int64_t sks,
                               int64_t vt_cols, int64_t so, const WorkItem* items, int64_t n_items, float scale,
                               int32_t kv_group, bool causal, hipStream_t stream, const SplitArgs& sp) {
  if (n_items <= 0) return hipSuccess;
  if (kv_group < 1) return hipErrorInvalidValue;
  const QNormArgs none{};
  const F8Scales fs{static_cast<const uint8_t*>(q8s), static_cast<const uint8_t*>(k8s),
                    static_cast<const uint8_t*>(vt8s), sqs, sks, int32_t(vt_cols / kVtTile)};
#define H3A_F8PV_CASE(DD)                                                                                   \
  if (D == DD)                                                                                              \
    return causal ? launch<DD, true, false, 0, 2>(q8, k8, vt8, o, sq, sk, vt_cols, so, items, n_items, scale, \
                                                  kv_group, none, stream, fs, sp)                          \
                  : launch<DD, false, false, 0, 2>(q8, k8, vt8, o, sq, sk, vt_cols, so, items, n_items, scale,\
                                                   kv_group, none, stream, fs, sp);
  H3A_F8PV_CASE(128) H3A_F8PV_CASE(64)
#undef H3A_F8PV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_i8qk(const void* q8, const void* k8, const void* q_scale, const void* k_scale,
                                 const void* v, void* o, int32_t D, int64_t sq, int64_t sk, int64_t sqs, int64_t sks,
                                 int64_t sv, int64_t so, const WorkItem* items, int64_t n_items, float scale,
                                 int32_t kv_group, bool causal, hipStream_t stream, const SplitArgs& sp) {
  if (n_items <= 0) return hipSuccess;
  if (kv_group < 1) return hipErrorInvalidValue;
  const QNormArgs none{};
  const F8Scales fs{static_cast<const uint8_t*>(q_scale), static_cast<const uint8_t*>(k_scale), nullptr, sqs, sks, 0};
#define H3A_I8_CASE(DD)                                                                                     \
  if (D == DD)                                                                                              \
    return causal ? launch<DD, true, false, 0, 3>(q8, k8, v, o, sq, sk, sv, so, items, n_items, scale,        \
                                                  kv_group, none, stream, fs, sp)                          \
                  : launch<DD, false, false, 0, 3>(q8, k8, v, o, sq, sk, sv, so, items, n_items, scale,       \
                                                   kv_group, none, stream, fs, sp);
  H3A_I8_CASE(128) H3A_I8_CASE(64)
#undef H3A_I8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_i8qk_fp8pv(const void* q8, const void* k8, const void* vt8, const void* q_scale,
                                     const void* k_scale, const void* vt8s, void* o, int32_t D, int64_t sq, int64_t sk,
                                     int64_t sqs, int64_t sks, int64_t vt_cols, int64_t so, const WorkItem* items,
                                     int64_t n_items, float scale, int32_t kv_group, bool causal, hipStream_t stream,
                                     const SplitArgs& sp) {
  if (n_items <= 0) return hipSuccess;
  if (kv_group < 1) return hipErrorInvalidValue;
  const QNormArgs none{};
  const F8Scales fs{static_cast<const uint8_t*>(q_scale), static_cast<const uint8_t*>(k_scale),
                    static_cast<const uint8_t*>(vt8s), sqs, sks, int32_t(vt_cols / kVtTile)};
#define H3A_I8PV_CASE(DD)                                                                                   \
  if (D == DD)                                                                                              \
    return causal ? launch<DD, true, false, 0, 4>(q8, k8, vt8, o, sq, sk, vt_cols, so, items, n_items, scale, \
                                                  kv_group, none, stream, fs, sp)                          \
                  : launch<DD, false, false, 0, 4>(q8, k8, vt8, o, sq, sk, vt_cols, so, items, n_items, scale,\
                                                   kv_group, none, stream, fs, sp);
  H3A_I8PV_CASE(128) H3A_I8PV_CASE(64)
#undef H3A_I8PV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_bf16_qnorm(const void* q, const void* k, const void* v, void* o, int32_t D,
                                      int64_t sq, int64_t sk, int64_t sv, int64_t so,
                                      const WorkItem* items, int64_t n_items, float scale, int32_t kv_group,
                                      const float* gamma_q, float eps, const float* cos_sin, int64_t S,
                                      int32_t rot_dim, hipStream_t stream, const SplitArgs& sp) {
  if (n_items <= 0) return hipSuccess;
  if (kv_group < 1 || rot_dim % 32 != 0) return hipErrorInvalidValue;
  const QNormArgs qn{gamma_q, cos_sin, S, rot_dim / 2, eps};
  const F8Scales nofs{};
#define H3A_QNORM_CASE(DD, R)                                                                               \
  if (D == DD && rot_dim == 32 * R)                                                                         \
    return launch<DD, false, true, R>(q, k, v, o, sq, sk, sv, so, items, n_items, scale, kv_group, qn, stream, \
                                      nofs, sp);
  H3A_QNORM_CASE(128, 0) H3A_QNORM_CASE(128, 1) H3A_QNORM_CASE(128, 2) H3A_QNORM_CASE(128, 3)
  H3A_QNORM_CASE(128, 4) H3A_QNORM_CASE(64, 0) H3A_QNORM_CASE(64, 1) H3A_QNORM_CASE(64, 2)
#undef H3A_QNORM_CASE
  return hipErrorInvalidValue;
}

}  // namespace h3a
