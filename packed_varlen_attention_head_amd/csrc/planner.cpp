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
//
// Split plans (bidirectional): when a few long items would set the time
// (fewer items than workgroup slots, or whole rounds of long items leaving
// slots idle at the end), an item's keys are cut into ranges of at most Lp
// tiles, each range its own item; a merge pass then combines each item's
// partial rows exactly as the streaming softmax combines tiles (max, rescale,
// sum).  Lp is chosen by list-scheduling the item costs onto the slots,
// charging each partial slot for its round trip through memory and the
// merge launch.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <queue>
#include <vector>

#include "common.h"

namespace h3a {
namespace {

struct Chunk {
  int32_t seg;
  int32_t head;
  int32_t t0, t1;    // query tiles [t0, t1)
  int32_t kt0, kt1;  // key tiles [kt0, kt1); kt1 == 0: all
  int32_t part;      // first partial slot + 1 of the chunk's first query tile (0: not split)
  int32_t nparts;    // key ranges per query tile (its part index is part + q * nparts + range)
  double cost;
};

// Query tiles per chunk: a chunk's workgroups share one K/V stream.
constexpr int32_t kChunkTiles = 16;
// Fixed per-item cost in key-row units (Q load, epilogue, scheduling).
constexpr double kItemOverheadKeys = 128.0;
// Split plans, in the same key-row units of per-slot time: the merge pass
// runs after the attention on the whole GPU, so each partial slot adds the
// time the GPU takes to read its 64 KB back (measured: 1,524 slots in 27 us,
// while one slot streams 64 keys in about 1.8 us), plus the merge launch.
constexpr double kMergeKeysPerPart = 0.65;
constexpr double kMergeLaunchKeys = 192.0;
// A split must promise this much: the estimate ignores that a fuller GPU
// draws more power and runs at a lower clock (measured on a 3-head share of
// the S = 20,423 packing: 24% estimated, 9% realised by the attention).
constexpr double kSplitMinGain = 0.10;
// Shortest key range of a split item in automatic plans (tiles).
constexpr int32_t kMinPartTiles = 8;
// Most partial slots a split plan may use: 16,384 slots of 128 rows x 128
// fp32 dims (+ max and sum) are 1.1 GB of workspace.  Splits only pay where
// items are few, far below this.
constexpr int64_t kMaxSplitParts = 16384;

int32_t key_tiles(int32_t len) { return (len + kVtTile - 1) / kVtTile; }

// Even part length (tiles) for `parts` near-equal ranges of nk tiles.
int32_t part_len(int32_t nk, int32_t parts) {
  int32_t L = (nk + parts - 1) / parts;
  return L + (L & 1);
}

// Makespan of list-scheduling costs (longest first) onto `slots` machines.
double list_makespan(std::vector<double> costs, int32_t slots) {
  std::sort(costs.begin(), costs.end(), std::greater<double>());
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int32_t i = 0; i < slots; ++i) free_at.push(0.0);
  double end = 0.0;
  for (double c : costs) {
    const double t = free_at.top() + c;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  return end;
}

// Chunks -> items, balanced over n_xcd XCDs (see the file comment).
std::vector<WorkItem> lay_out(std::vector<Chunk> chunks, const int32_t* cu, const std::vector<int32_t>& col0,
                              int32_t block_m, int32_t n_xcd, bool causal) {
  auto expand = [&](const Chunk& c, std::vector<WorkItem>& out) {
    const int32_t len = cu[c.seg + 1] - cu[c.seg];
    for (int32_t i = c.t0; i < c.t1; ++i) {
      const int32_t t = causal ? c.t0 + c.t1 - 1 - i : i;
      const int32_t part = c.part > 0 ? c.part + (t - c.t0) * c.nparts : 0;
      out.push_back({cu[c.seg], len, t * block_m, c.head, col0[c.seg], c.kt0, c.kt1, part});
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
  std::vector<WorkItem> items(longest * size_t(n_xcd), WorkItem{0, 0, 0, 0, 0, 0, 0, 0});
  for (int32_t x = 0; x < n_xcd; ++x)
    for (size_t p = 0; p < queue[x].size(); ++p) items[p * size_t(n_xcd) + size_t(x)] = queue[x][p];
  return items;
}

// First column of each segment in the padded transposed-V layout (-1 past
// INT32_MAX: only the FP8-PV path reads it, and its entry point rejects
// layouts that large), and the non-empty segments longest first.
void segments_of(const int32_t* cu, int32_t nseg, std::vector<int32_t>* col0, std::vector<int32_t>* order) {
  col0->assign(size_t(nseg) + 1, 0);
  int64_t col = 0;
  for (int32_t s = 0; s < nseg; ++s) {
    col += (int64_t(cu[s + 1]) - cu[s] + kVtTile - 1) / kVtTile * kVtTile;
    (*col0)[s + 1] = col > int64_t(INT32_MAX) ? -1 : int32_t(col);
  }
  order->clear();
  for (int32_t s = 0; s < nseg; ++s)
    if (cu[s + 1] > cu[s]) order->push_back(s);
  std::stable_sort(order->begin(), order->end(), [&](int32_t a, int32_t b) {
    return (cu[a + 1] - cu[a]) > (cu[b + 1] - cu[b]);
  });
}

}  // namespace

std::vector<WorkItem> plan_tiles(const int32_t* cu, int32_t nseg, int32_t heads, int32_t block_m,
                                 int32_t n_xcd, bool causal) {
  std::vector<int32_t> col0, order;
  segments_of(cu, nseg, &col0, &order);
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
        chunks.push_back({s, h, t0, t1, 0, 0, 0, 0, cost});
      }
  }
  return lay_out(std::move(chunks), cu, col0, block_m, n_xcd, causal);
}

std::vector<WorkItem> plan_tiles_split(const int32_t* cu, int32_t nseg, int32_t heads, int32_t block_m,
                                       int32_t n_xcd, int32_t slots, bool causal, int32_t policy,
                                       std::vector<MergeItem>* merges, int64_t* n_parts) {
  merges->clear();
  *n_parts = 0;
  if (causal || policy == kSplitNever) return plan_tiles(cu, nseg, heads, block_m, n_xcd, causal);
  std::vector<int32_t> col0, order;
  segments_of(cu, nseg, &col0, &order);
  if (order.empty()) return plan_tiles(cu, nseg, heads, block_m, n_xcd, causal);

  // Parts per item of segment s for a maximum part length Lp (tiles).
  auto parts_for = [&](int32_t s, int32_t Lp) {
    const int32_t nk = key_tiles(cu[s + 1] - cu[s]);
    if (policy == kSplitAlways) {
      if (nk < 4) return 1;
      const int32_t L = part_len(nk, 3);
      return (nk + L - 1) / L;
    }
    if (Lp <= 0 || nk <= Lp) return 1;
    const int32_t L = part_len(nk, (nk + Lp - 1) / Lp);
    return (nk + L - 1) / L;
  };

  int32_t Lp = 0;  // 0: no split
  if (policy == kSplitAuto) {
    // With many rounds of items per slot the ragged last round is a small
    // share of the time: not worth estimating.
    int64_t n_items = 0;
    for (int32_t s : order) n_items += int64_t(heads) * ((cu[s + 1] - cu[s] + block_m - 1) / block_m);
    if (n_items > 64 * int64_t(slots)) return plan_tiles(cu, nseg, heads, block_m, n_xcd, causal);
    const int32_t nk_max = key_tiles(cu[order[0] + 1] - cu[order[0]]);
    auto estimate = [&](int32_t L) {
      std::vector<double> costs;
      int64_t parts = 0;
      for (int32_t s : order) {
        const int32_t len = cu[s + 1] - cu[s];
        const int32_t nq = (len + block_m - 1) / block_m, nk = key_tiles(len);
        const int32_t k = parts_for(s, L);
        const int32_t pl = part_len(nk, k);
        for (int32_t r = 0; r < k; ++r) {
          const int32_t keys = std::min(len, (r + 1) * pl * kVtTile) - r * pl * kVtTile;
          const double c = double(keys) + kItemOverheadKeys;
          for (int64_t i = 0; i < int64_t(nq) * heads; ++i) costs.push_back(c);
          if (k > 1) parts += int64_t(nq) * heads;
        }
      }
      if (parts > kMaxSplitParts) return 1e300;
      return list_makespan(std::move(costs), slots) +
             (parts > 0 ? kMergeLaunchKeys + kMergeKeysPerPart * double(parts) : 0.0);
    };
    double best = estimate(0);
    for (int32_t j = 2; j <= 16; ++j) {
      const int32_t L = part_len(nk_max, j);
      if (L < kMinPartTiles) break;
      const double e = estimate(L);
      if (e < best * (1.0 - kSplitMinGain)) {
        best = e;
        Lp = L;
      }
    }
    if (Lp == 0) return plan_tiles(cu, nseg, heads, block_m, n_xcd, causal);
  }

  // Partial slots this choice needs: none at all when over the limit.
  int64_t need = 0;
  for (int32_t s : order) {
    const int32_t k = parts_for(s, Lp);
    if (k > 1) need += int64_t(k) * heads * ((cu[s + 1] - cu[s] + block_m - 1) / block_m);
  }
  if (need > kMaxSplitParts) return plan_tiles(cu, nseg, heads, block_m, n_xcd, causal);

  std::vector<Chunk> chunks;
  int32_t next_part = 0;
  for (int32_t s : order) {
    const int32_t len = cu[s + 1] - cu[s];
    const int32_t nq = (len + block_m - 1) / block_m, nk = key_tiles(len);
    const int32_t k = parts_for(s, Lp);
    const int32_t pl = part_len(nk, k);
    for (int32_t h = 0; h < heads; ++h)
      for (int32_t t0 = 0; t0 < nq; t0 += kChunkTiles) {
        const int32_t t1 = std::min(nq, t0 + kChunkTiles);
        const int32_t base = k > 1 ? next_part : -1;
        if (k > 1) {
          for (int32_t t = t0; t < t1; ++t)
            merges->push_back({cu[s], len, t * block_m, h, next_part + (t - t0) * k, k, {0, 0}});
          next_part += (t1 - t0) * k;
        }
        for (int32_t r = 0; r < k; ++r) {
          const int32_t kt0 = r * pl, kt1 = std::min(nk, (r + 1) * pl);
          const double cost = double(t1 - t0) * (double(std::min(len, kt1 * kVtTile) - kt0 * kVtTile) +
                                                 kItemOverheadKeys);
          // part index of query tile t0, range r: base + r (+ (t - t0) * k per tile)
          chunks.push_back({s, h, t0, t1, k > 1 ? kt0 : 0, k > 1 ? kt1 : 0, k > 1 ? base + r + 1 : 0, k, cost});
        }
      }
  }
  *n_parts = next_part;
  return lay_out(std::move(chunks), cu, col0, block_m, n_xcd, causal);
}

}  // namespace h3a
