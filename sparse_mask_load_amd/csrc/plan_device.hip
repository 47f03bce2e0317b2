// Work lists on the GPU: round-based LPT over the mask's row counts, with no
// host round trip, so that a plan for a runtime mask (the db-SP post's
// scenario 1: masks known only when the step runs) costs the host nothing and
// its lists are ready as soon as the popcount is.
//
// Rule (a parallel form of the post's LPT paragraph): items in LPT order (load
// descending, id ascending) are handed out m at a time; in each round the
// bins are ordered by their load at the round's start (ascending, lower index
// first) and the round's j-th item goes to the j-th bin.  Every bin gets one
// item per round except in a last, partial round, so a bin's list is its items
// in round order.  On the block workloads here this reaches the makespan of
// the sequential LPT greedy.
//
// One workgroup of 1024 threads per list (list 0: the full chunk range over
// the row counts; list 1 + c: chunk c over its per-chunk counts):
//  1. keys (4095 - load) << 20 | id, padded to a power of two, bitonic-sorted
//     in LDS (ascending key = LPT order; ids are unique, so the order is total);
//  2. per round, the m bin keys (load << 16 | bin, one per thread) are
//     bitonic-sorted in registers (lane shuffles below 64, LDS exchange above)
//     and thread j records the bin of the round's j-th item;
//  3. bin counts, an exclusive scan for bin_ptr, and the scatter of each item
//     to bin_ptr[bin] + round.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kIdBits = 20;  // item ids below 2^20; loads below 4096

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const int lo = __shfl_xor((int)(uint32_t)v, mask);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), mask);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__global__ __launch_bounds__(kThreads) void plan_rounds_kernel(const int32_t* __restrict__ row,
                                                               const int32_t* __restrict__ crow, int BH, int nQ,
                                                               int C, int m, int32_t* __restrict__ items,
                                                               int32_t* __restrict__ bin_ptr,
                                                               int64_t* __restrict__ bin_load,
                                                               int64_t* __restrict__ stats, int list0,
                                                               int32_t* __restrict__ order,
                                                               int32_t* __restrict__ dyn_ctr) {
  __shared__ uint32_t key[kDevicePlanMaxItems];   // sort keys; after the sort, items in LPT order
  __shared__ uint16_t bin_at[kDevicePlanMaxItems];  // bin of the item at each LPT position
  __shared__ uint64_t xch[kThreads];               // bitonic exchange across waves / scan buffer
  __shared__ unsigned long long red_sum;
  __shared__ unsigned int red_max, red_span;

  const int list = list0 + blockIdx.x;  // which list; its outputs go to slot blockIdx.x
  const int slot = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = BH * nQ;
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  int mp = 1;
  while (mp < m) mp <<= 1;

  if (tid == 0) {
    red_sum = 0;
    red_max = 0;
    red_span = 0;
  }
  __syncthreads();
  // 1. keys and load statistics
  unsigned long long my_sum = 0;
  unsigned int my_max = 0;
  for (int p = tid; p < n2; p += kThreads) {
    uint32_t k = 0xFFFFFFFFu;
    if (p < n) {
      const int load = list == 0 ? row[p] : crow[((int64_t)(p / nQ) * C + (list - 1)) * nQ + p % nQ];
      k = ((uint32_t)(4095 - load) << kIdBits) | (uint32_t)p;
      my_sum += (unsigned long long)load;
      my_max = max(my_max, (unsigned int)load);
    }
    key[p] = k;
  }
  atomicAdd(&red_sum, my_sum);
  atomicMax(&red_max, my_max);
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int p = tid; p < n2 / 2; p += kThreads) {
        const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));  // bit j of i is clear; its partner is i + j
        const uint32_t a = key[i], b = key[i + j];
        if ((a > b) == ((i & k) == 0)) {
          key[i] = b;
          key[i + j] = a;
        }
      }
      __syncthreads();
    }

  // the queue of the run-time order: the items in LPT order, and its counters at zero
  if (order)
    for (int p = tid; p < n; p += kThreads) order[(int64_t)slot * n + p] = (int32_t)(key[p] & ((1u << kIdBits) - 1));
  if (dyn_ctr && tid < kQueueCtrs) dyn_ctr[kQueueCtrs * slot + tid] = 0;

  // 2. rounds; thread t holds one bin key (load << 16 | bin), sentinels beyond m
  uint64_t bkey = tid < m ? (uint64_t)tid : ~0ull;
  const int rounds = (n + m - 1) / m;
  for (int r = 0; r < rounds; ++r) {
    if (r > 0) {  // before round 0 every load is 0 and the keys are already in order
      for (int k = 2; k <= mp; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
          uint64_t other;
          if (j >= 64) {
            xch[tid] = bkey;
            __syncthreads();
            other = xch[tid ^ j];
            __syncthreads();
          } else {
            other = shfl_xor_u64(bkey, j);
          }
          const bool keep_min = ((tid & j) == 0) == ((tid & k) == 0);
          bkey = keep_min ? min(bkey, other) : max(bkey, other);
        }
    }
    const int p = r * m + tid;
    if (tid < m && p < n) {
      const uint32_t k = key[p];
      const int load = 4095 - (int)(k >> kIdBits);
      bin_at[p] = (uint16_t)(bkey & 0xFFFF);
      bkey += (uint64_t)load << 16;
    }
  }

  // 3. bin loads and counts: full rounds give every bin one item; the last round's takers one more
  const int full = n / m;
  const int rem = n - full * m;
  int32_t* const ptr_out = bin_ptr + (int64_t)slot * (m + 1);
  uint32_t* const cnt = (uint32_t*)xch;  // reused: no exchange is pending
  __syncthreads();
  if (tid < m) {
    const int b = (int)(bkey & 0xFFFF);
    const int64_t load = (int64_t)(bkey >> 16);
    bin_load[(int64_t)slot * m + b] = load;
    atomicMax(&red_span, (unsigned int)load);
  }
  for (int b = tid; b < kThreads; b += kThreads) cnt[b] = b < m ? (uint32_t)full : 0u;
  __syncthreads();
  if (tid < rem) cnt[bin_at[full * m + tid]] += 1;  // distinct bins: no two threads collide
  __syncthreads();
  // inclusive Hillis-Steele scan over the 1024 counts, in place with a register copy
  uint32_t v = cnt[tid];
  for (int d = 1; d < kThreads; d <<= 1) {
    const uint32_t add = tid >= d ? cnt[tid - d] : 0u;
    __syncthreads();
    v += add;
    cnt[tid] = v;
    __syncthreads();
  }
  if (tid < m) ptr_out[tid + 1] = (int32_t)v;
  if (tid == 0) ptr_out[0] = 0;
  int32_t* const items_out = items + (int64_t)slot * n;
  for (int p = tid; p < n; p += kThreads) {
    const int b = bin_at[p];
    const uint32_t start = b == 0 ? 0u : cnt[b - 1];
    items_out[start + p / m] = (int32_t)(key[p] & ((1u << kIdBits) - 1));
  }
  if (tid == 0) {
    const int64_t total = (int64_t)red_sum, pmax = (int64_t)red_max;
    int64_t* s = stats + (int64_t)slot * 4;
    s[0] = total;
    s[1] = pmax;
    s[2] = (int64_t)red_span;
    const int64_t even = (total + m - 1) / m;
    s[3] = pmax > even ? pmax : even;
  }
}

}  // namespace

hipError_t launch_plan_rounds(const int32_t* row, const int32_t* crow, int BH, int nQ, int C, int m, int32_t* items,
                              int32_t* bin_ptr, int64_t* bin_load, int64_t* stats, hipStream_t stream, int list0,
                              int n_lists, int32_t* order, int32_t* dyn_ctr) {
  if (n_lists < 0) n_lists = C + 1 - list0;
  if (BH * nQ > kDevicePlanMaxItems || m > kDevicePlanMaxBins || m < 1 || list0 < 0 || n_lists < 1 ||
      list0 + n_lists > C + 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_rounds_kernel, dim3(n_lists), dim3(kThreads), 0, stream, row, crow, BH, nQ, C, m, items,
                     bin_ptr, bin_load, stats, list0, order, dyn_ctr);
  return hipGetLastError();
}

}  // namespace sa
