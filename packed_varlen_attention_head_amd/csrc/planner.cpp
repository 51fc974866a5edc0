// Segment-aware tile planner for the varlen attention kernels (host only).
//
// The attention of each packed segment is independent of every other segment
// (vllm.cpp PR #26, opening commit: per-document bidirectional attention over
// cu_seqlens), so the work is a flat list of (segment, head, query tile)
// items whose cost grows with the segment length (every query tile streams
// all of its segment's keys).  The plan is a pure function of cu_seqlens and
// is built once per distinct content: the packing is the same for every
// denoising step of a request, the same reason the rotary/mask tables are
// step-invariant caches (h3-spark model card, "What this config does").
//
// Layout of the plan:
//   * items of one (segment, head) are grouped in chunks of consecutive query
//     tiles, so the workgroups that stream the same K/V run side by side;
//   * chunks are assigned to XCDs longest-first (LPT) onto the least-loaded
//     XCD, which balances the per-XCD work;
//   * the per-XCD queues are interleaved so that workgroup b runs on XCD
//     b % n_xcd (the dispatcher hands workgroups to XCDs round-robin), each
//     XCD seeing its own items longest first.  Short queues are padded with
//     empty items.
// Causal items stream only the keys up to their last row, so an item costs
// min(len, (t + 1) block_m) keys and each chunk lists its query tiles last
// to first (costliest first).
#include <algorithm>
#include <cstdint>
#include <vector>

#include "common.h"

namespace h3a {
namespace {

struct Chunk {
  int32_t seg;
  int32_t head;
  int32_t t0, t1;  // query tiles [t0, t1)
  double cost;
};

// Query tiles per chunk: a chunk's workgroups share one K/V stream.
constexpr int32_t kChunkTiles = 16;
// Fixed per-item cost in key-row units (Q load, epilogue, scheduling).
constexpr double kItemOverheadKeys = 128.0;

}  // namespace

std::vector<WorkItem> plan_tiles(const int32_t* cu, int32_t nseg, int32_t heads, int32_t block_m,
                                 int32_t n_xcd, bool causal) {
  // First column of each segment in the padded transposed-V layout (-1 past
  // INT32_MAX: only the FP8-PV path reads it, and its entry point rejects
  // layouts that large).
  std::vector<int32_t> col0(size_t(nseg) + 1, 0);
  int64_t col = 0;
  for (int32_t s = 0; s < nseg; ++s) {
    col += (int64_t(cu[s + 1]) - cu[s] + kVtTile - 1) / kVtTile * kVtTile;
    col0[s + 1] = col > int64_t(INT32_MAX) ? -1 : int32_t(col);
  }
  std::vector<int32_t> order;
  for (int32_t s = 0; s < nseg; ++s)
    if (cu[s + 1] > cu[s]) order.push_back(s);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return (cu[a + 1] - cu[a]) > (cu[b + 1] - cu[b]);
  });

  std::vector<Chunk> chunks;
  for (int32_t s : order) {
    const int32_t len = cu[s + 1] - cu[s];
    const int32_t ntiles = (len + block_m - 1) / block_m;
    auto tile_cost = [&](int32_t t) {
      const int64_t keys = causal ? std::min<int64_t>(len, int64_t(t + 1) * block_m) : len;
      return double(keys) + kItemOverheadKeys;
    };
    for (int32_t h = 0; h < heads; ++h)
      for (int32_t t0 = 0; t0 < ntiles; t0 += kChunkTiles) {
        const int32_t t1 = std::min(ntiles, t0 + kChunkTiles);
        double cost = 0.0;
        for (int32_t t = t0; t < t1; ++t) cost += tile_cost(t);
        chunks.push_back({s, h, t0, t1, cost});
      }
  }

  auto expand = [&](const Chunk& c, std::vector<WorkItem>& out) {
    const int32_t len = cu[c.seg + 1] - cu[c.seg];
    for (int32_t i = c.t0; i < c.t1; ++i) {
      const int32_t t = causal ? c.t0 + c.t1 - 1 - i : i;
      out.push_back({cu[c.seg], len, t * block_m, c.head, col0[c.seg], {0, 0, 0}});
    }
  };

  if (n_xcd <= 1) {
    std::vector<WorkItem> items;
    for (const Chunk& c : chunks) expand(c, items);
    return items;
  }

  std::stable_sort(chunks.begin(), chunks.end(),
                   [](const Chunk& a, const Chunk& b) { return a.cost > b.cost; });
  std::vector<double> load(n_xcd, 0.0);
  std::vector<std::vector<WorkItem>> queue(n_xcd);
  for (const Chunk& c : chunks) {
    int32_t x = 0;
    for (int32_t i = 1; i < n_xcd; ++i)
      if (load[i] < load[x]) x = i;
    load[x] += c.cost;
    expand(c, queue[x]);
  }
  size_t longest = 0;
  for (const auto& qx : queue) longest = std::max(longest, qx.size());
  std::vector<WorkItem> items(longest * size_t(n_xcd), WorkItem{0, 0, 0, 0, 0, {0, 0, 0}});
  for (int32_t x = 0; x < n_xcd; ++x)
    for (size_t p = 0; p < queue[x].size(); ++p) items[p * size_t(n_xcd) + size_t(x)] = queue[x][p];
  return items;
}

}  // namespace h3a
