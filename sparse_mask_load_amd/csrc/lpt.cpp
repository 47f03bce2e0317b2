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
#include <functional>
#include <cstdint>
#include <numeric>
#include <queue>
#include <utility>
#include <vector>

#include "internal.h"

namespace sa {

// Work lists of one plan are rebuilt for every mask, so this runs in the
// timed path: a counting sort replaces the comparison sort (loads are small
// non-negative integers; equal loads keep ascending id order), a ring of
// per-load bin bitsets replaces the bin heap, and the per-bin lists come from
// a stable counting sort of the items by bin.
void assign(const int64_t* loads, int n, int m, int order, int32_t* items_out, int32_t* bin_ptr_out,
            int64_t* bin_load_out) {
  std::vector<int32_t> bin_of(n);
  std::vector<int64_t> bin_load(m, 0);
  if (order == SA_ORDER_NAIVE) {
    for (int i = 0; i < n; ++i) {
      bin_of[i] = i % m;
      bin_load[i % m] += loads[i];
    }
  } else {
    int64_t lmax = 0;
    for (int i = 0; i < n; ++i) lmax = std::max(lmax, loads[i]);
    std::vector<int32_t> ids(n);
    if (lmax <= 4 * (int64_t)n + 65536) {
      // counting sort, load descending, id ascending within a load
      std::vector<int32_t> start(lmax + 2, 0);
      for (int i = 0; i < n; ++i) ++start[lmax - loads[i] + 1];
      for (int64_t v = 1; v <= lmax + 1; ++v) start[v] += start[v - 1];
      for (int i = 0; i < n; ++i) ids[start[lmax - loads[i]]++] = i;
    } else {
      std::iota(ids.begin(), ids.end(), 0);
      std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return loads[a] > loads[b]; });
    }
    // Least-loaded bin, lowest index first: bins are grouped by load in a ring of lmax + 1
    // buckets (each a bitset of bins).  Every bin load lies in [lo, lo + lmax], lo being the
    // current minimum, because a bin only receives an item while it is least loaded; lo
    // never decreases, so the search for the lowest non-empty bucket only moves forward.
    if (lmax <= (1 << 16)) {
      const int words = (m + 63) / 64;
      const int64_t nb = lmax + 1;
      std::vector<uint64_t> bucket((size_t)nb * words, 0);
      for (int b = 0; b < m; ++b) bucket[b / 64] |= 1ull << (b % 64);
      int64_t lo = 0;
      for (int32_t id : ids) {
        uint64_t* w = &bucket[(size_t)(lo % nb) * words];
        int k = 0;
        for (;;) {
          while (k < words && w[k] == 0) ++k;
          if (k < words) break;
          ++lo;
          w = &bucket[(size_t)(lo % nb) * words];
          k = 0;
        }
        const int b = k * 64 + __builtin_ctzll(w[k]);
        w[k] &= w[k] - 1;
        bin_of[id] = b;
        bin_load[b] += loads[id];
        bucket[(size_t)(bin_load[b] % nb) * words + b / 64] |= 1ull << (b % 64);
      }
    } else {
      // very large loads (host callers): a binary heap of packed (load << 32 | bin) keys
      std::vector<std::pair<int64_t, int32_t>> heap(m);
      for (int b = 0; b < m; ++b) heap[b] = {0, b};
      for (int32_t id : ids) {
        std::pop_heap(heap.begin(), heap.end(), std::greater<std::pair<int64_t, int32_t>>());
        auto& e = heap.back();
        bin_of[id] = e.second;
        e.first += loads[id];
        bin_load[e.second] = e.first;
        std::push_heap(heap.begin(), heap.end(), std::greater<std::pair<int64_t, int32_t>>());
      }
    }
    // per-bin order is assignment order, which is the order of ids
    std::vector<int32_t> pos(m + 1, 0);
    for (int i = 0; i < n; ++i) ++pos[bin_of[i] + 1];
    for (int b = 0; b < m; ++b) pos[b + 1] += pos[b];
    for (int b = 0; b <= m; ++b) bin_ptr_out[b] = pos[b];
    for (int32_t id : ids) items_out[pos[bin_of[id]]++] = id;
    if (bin_load_out)
      for (int b = 0; b < m; ++b) bin_load_out[b] = bin_load[b];
    return;
  }
  std::vector<int32_t> pos(m + 1, 0);
  for (int i = 0; i < n; ++i) ++pos[bin_of[i] + 1];
  for (int b = 0; b < m; ++b) pos[b + 1] += pos[b];
  for (int b = 0; b <= m; ++b) bin_ptr_out[b] = pos[b];
  for (int i = 0; i < n; ++i) items_out[pos[bin_of[i]]++] = i;
  if (bin_load_out)
    for (int b = 0; b < m; ++b) bin_load_out[b] = bin_load[b];
}

// Two-level LPT for XCD affinity (the db-SP "stay-home" bonus re-read for one
// chip): a head's items should share one XCD's L2, and the persistent
// workgroups b with b mod groups == g run on XCD g.  Level 1 assigns heads
// (load = sum of their items) to the groups by LPT; level 2 assigns, per group,
// the items of its heads (in the order the heads were given to the group,
// then by Q-block) to the group's bins by LPT; the k-th bin of group g is bin
// k * groups + g.  With groups <= 1, or m not a multiple of groups, plain LPT.
void assign_grouped(const int64_t* loads, int n_heads, int per_head, int m, int groups, int32_t* items_out,
                    int32_t* bin_ptr_out, int64_t* bin_load_out) {
  const int n = n_heads * per_head;
  if (groups <= 1 || m % groups != 0) {
    assign(loads, n, m, SA_ORDER_LPT, items_out, bin_ptr_out, bin_load_out);
    return;
  }
  std::vector<int64_t> head_load(n_heads, 0);
  for (int h = 0; h < n_heads; ++h)
    for (int q = 0; q < per_head; ++q) head_load[h] += loads[(size_t)h * per_head + q];
  std::vector<int32_t> heads(std::max(n_heads, 1)), head_ptr(groups + 1);
  assign(head_load.data(), n_heads, groups, SA_ORDER_LPT, heads.data(), head_ptr.data(), nullptr);
  const int per = m / groups;
  std::vector<int32_t> bin_of(n), rank_in_bin(n), bin_count(m, 0);
  std::vector<int64_t> bin_load(m, 0);
  std::vector<int32_t> order(n);  // items in global assignment order within their bins
  for (int g = 0; g < groups; ++g) {
    std::vector<int32_t> ids;
    for (int p = head_ptr[g]; p < head_ptr[g + 1]; ++p)
      for (int q = 0; q < per_head; ++q) ids.push_back(heads[p] * per_head + q);
    const int ng = (int)ids.size();
    std::vector<int64_t> local(ng);
    for (int i = 0; i < ng; ++i) local[i] = loads[ids[i]];
    std::vector<int32_t> litems(std::max(ng, 1)), lptr(per + 1);
    std::vector<int64_t> lload(per);
    assign(local.data(), ng, per, SA_ORDER_LPT, litems.data(), lptr.data(), lload.data());
    for (int k = 0; k < per; ++k) {
      const int b = k * groups + g;
      bin_load[b] = lload[k];
      for (int p = lptr[k]; p < lptr[k + 1]; ++p) {
        const int32_t id = ids[litems[p]];
        bin_of[id] = b;
        rank_in_bin[id] = bin_count[b]++;
      }
    }
  }
  std::vector<int32_t> pos(m + 1, 0);
  for (int b = 0; b < m; ++b) pos[b + 1] = pos[b] + bin_count[b];
  for (int b = 0; b <= m; ++b) bin_ptr_out[b] = pos[b];
  for (int i = 0; i < n; ++i) items_out[pos[bin_of[i]] + rank_in_bin[i]] = i;
  if (bin_load_out)
    for (int b = 0; b < m; ++b) bin_load_out[b] = bin_load[b];
}

}  // namespace sa
