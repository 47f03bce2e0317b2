// Host work-list planner: LPT greedy and round-robin over identical bins.
//
// LPT follows the db-SP post on balancing sparse-attention heads ("longest
// processing time first": the longest remaining job goes to the currently
// least-loaded machine; identical-machines scheduling with the makespan
// objective).  On one GPU the machines are the persistent kernel's workgroups
// and a job is one (batch, head, Q-block) item whose load is its number of live
// tiles (the mask row sum of the post's scenario 2).  Tie rules, which the post
// leaves open: items with equal load in ascending id order; among equally
// loaded bins the lowest index (the rule the post's [8,7,6,5,4] example needs
// to print 8+5+4 | 7+6).
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <queue>
#include <utility>
#include <vector>

#include "internal.h"

namespace sa {

void assign(const int64_t* loads, int n, int m, int order, int32_t* items_out, int32_t* bin_ptr_out,
            int64_t* bin_load_out) {
  std::vector<std::vector<int32_t>> bins(m);
  std::vector<int64_t> bin_load(m, 0);
  if (order == SA_ORDER_NAIVE) {
    for (int i = 0; i < n; ++i) {
      bins[i % m].push_back(i);
      bin_load[i % m] += loads[i];
    }
  } else {
    std::vector<int32_t> ids(n);
    std::iota(ids.begin(), ids.end(), 0);
    std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return loads[a] > loads[b]; });
    // min-heap of (load, bin): the top is the least-loaded bin, lowest index on ties
    using Entry = std::pair<int64_t, int32_t>;
    std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap;
    for (int b = 0; b < m; ++b) heap.push({0, b});
    for (int32_t id : ids) {
      Entry e = heap.top();
      heap.pop();
      bins[e.second].push_back(id);
      e.first += loads[id];
      bin_load[e.second] = e.first;
      heap.push(e);
    }
  }
  int32_t pos = 0;
  for (int b = 0; b < m; ++b) {
    bin_ptr_out[b] = pos;
    for (int32_t id : bins[b]) items_out[pos++] = id;
    if (bin_load_out) bin_load_out[b] = bin_load[b];
  }
  bin_ptr_out[m] = pos;
}

}  // namespace sa
