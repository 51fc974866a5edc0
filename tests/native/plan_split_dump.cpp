// Prints the split plan of a packing as text, for the planner tests:
//   plan_split_dump POLICY SLOTS N_XCD HEADS BLOCK_M LEN...
// Output: "items N", then one line per item (seg_start seg_len q_start head
// vt_col0 kt0 kt1 part), "merges M", one line per merge (seg_start seg_len
// q_start head part0 nparts), then "parts P".
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "common.h"

int main(int argc, char** argv) {
  if (argc < 7) {
    std::fprintf(stderr, "usage: %s POLICY SLOTS N_XCD HEADS BLOCK_M LEN...\n", argv[0]);
    return 2;
  }
  const int policy = std::atoi(argv[1]), slots = std::atoi(argv[2]), n_xcd = std::atoi(argv[3]);
  const int heads = std::atoi(argv[4]), block_m = std::atoi(argv[5]);
  std::vector<int32_t> cu{0};
  for (int i = 6; i < argc; ++i) cu.push_back(cu.back() + std::atoi(argv[i]));
  std::vector<h3a::MergeItem> merges;
  int64_t parts = 0;
  const auto items = h3a::plan_tiles_split(cu.data(), int32_t(cu.size() - 1), heads, block_m, n_xcd, slots, false,
                                           policy, &merges, &parts);
  std::printf("items %zu\n", items.size());
  for (const auto& w : items)
    std::printf("%d %d %d %d %d %d %d %d\n", w.seg_start, w.seg_len, w.q_start, w.head, w.vt_col0, w.kt0, w.kt1,
                w.part);
  std::printf("merges %zu\n", merges.size());
  for (const auto& m : merges)
    std::printf("%d %d %d %d %d %d\n", m.seg_start, m.seg_len, m.q_start, m.head, m.part0, m.nparts);
  std::printf("parts %lld\n", (long long)parts);
  return 0;
}
