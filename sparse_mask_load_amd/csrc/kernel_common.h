// Device helpers shared by the block-sparse attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace sa {

// Builds the ordered list of live KV tiles of one work item (one Q-block row of
// the block mask) for chunks [c0, c1), using one wavefront.  Chunk c of the
// contiguous layout covers KV blocks [c*nK/C, (c+1)*nK/C); a descriptor carries
// the block index and a full group code.  Chunk c of the striped layout
// (striped attention: token j belongs to chunk j mod C) is cut into compacted
// tiles of `block` tokens; compacted tile t of chunk c spans original blocks
// C*t .. C*t+C-1, each contributing block/C consecutive compacted keys, so its
// liveness is the C-bit code of those mask entries.  Order: chunk, then tile.
// Returns the number of descriptors (valid in every lane); only writes `list`
// when `write` is set, so every wave can count while one wave fills the list.
__device__ inline int build_tile_list(const uint8_t* __restrict__ mrow, int nK, int n_chunks,
                                      int layout, int c0, int c1, int* list, bool write = true) {
  const int lane = threadIdx.x & 63;
  const int per_chunk = nK / n_chunks;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int count = 0;
  for (int c = c0; c < c1; ++c) {
    if (layout == SA_LAYOUT_CONTIGUOUS) {
      const int j0 = c * per_chunk, j1 = j0 + per_chunk;
      for (int base = j0; base < j1; base += 64) {
        const int j = base + lane;
        const bool live = j < j1 && mrow[j] != 0;
        const uint64_t bits = __ballot(live);
        if (write && live)
          list[count + __popcll(bits & below)] = j | (0xF << kDescCodeShift) | (c << kDescChunkShift);
        count += __popcll(bits);
      }
    } else {
      for (int base = 0; base < per_chunk; base += 64) {
        const int t = base + lane;
        int code = 0;
        if (t < per_chunk)
          for (int g = 0; g < n_chunks; ++g) code |= (mrow[n_chunks * t + g] != 0 ? 1 : 0) << g;
        const bool live = code != 0;
        const uint64_t bits = __ballot(live);
        if (write && live)
          list[count + __popcll(bits & below)] = t | (code << kDescCodeShift) | (c << kDescChunkShift);
        count += __popcll(bits);
      }
    }
  }
  return count;
}

// Tile list of a Q-block pair: the union of the live KV tiles of mask rows qa
// (mrow_a) and qa + 1 (the next row, when has_b), for chunks [c0, c1), in chunk
// then tile order, tiles as in build_tile_list (contiguous KV blocks, or the
// compacted tiles of the striped layout).  A pair descriptor holds the tile
// index in bits 0..11, the group code of row qa in bits 12..15 and that of row
// qa + 1 in bits 16..19 (contiguous: all four bits set when the row has the
// tile), and the chunk in the usual chunk field.
constexpr int kPairTileMask = 0xFFF;
constexpr int kPairCodeShift = 12;
__device__ inline int build_pair_tile_list(const uint8_t* __restrict__ mrow_a, bool has_b, int nK, int n_chunks,
                                           int layout, int c0, int c1, int* list, bool write = true) {
  const int lane = threadIdx.x & 63;
  const int per_chunk = nK / n_chunks;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint8_t* __restrict__ mrow_b = mrow_a + nK;
  int count = 0;
  for (int c = c0; c < c1; ++c) {
    for (int base = 0; base < per_chunk; base += 64) {
      const int t = base + lane;
      int ca = 0, cb = 0;
      if (t < per_chunk) {
        if (layout == SA_LAYOUT_CONTIGUOUS) {
          const int j = c * per_chunk + t;
          ca = mrow_a[j] != 0 ? 15 : 0;
          cb = has_b && mrow_b[j] != 0 ? 15 : 0;
        } else {
          for (int g = 0; g < n_chunks; ++g) {
            ca |= (mrow_a[n_chunks * t + g] != 0 ? 1 : 0) << g;
            cb |= (has_b && mrow_b[n_chunks * t + g] != 0 ? 1 : 0) << g;
          }
        }
      }
      const bool live = (ca | cb) != 0;
      const uint64_t bits = __ballot(live);
      const int tile = layout == SA_LAYOUT_CONTIGUOUS ? c * per_chunk + t : t;
      if (write && live)
        list[count + __popcll(bits & below)] =
            tile | (ca << kPairCodeShift) | (cb << (kPairCodeShift + 4)) | (c << kDescChunkShift);
      count += __popcll(bits);
    }
  }
  return count;
}

// Workgroup index remapped so that each XCD works through one contiguous range
// of [0, n) in order.  Workgroups b = 0, 1, ... of a launch are dealt to the
// n_xcd XCDs round-robin (b mod n_xcd); XCD x then runs logical indices
// start(x) + b / n_xcd, where start(x) counts the workgroups of the XCDs before
// it (the first n mod n_xcd XCDs get one more).  A bijection on [0, n).  Work
// indexed head-major thereby keeps each head on one XCD, in one L2.
__device__ __forceinline__ int xcd_contiguous(int b, int n, int n_xcd) {
  if (n_xcd <= 1) return b;
  const int x = b % n_xcd, s = b / n_xcd;
  const int per = n / n_xcd, rem = n % n_xcd;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + s;
}

__device__ inline int64_t realtime_now() { return (int64_t)__builtin_amdgcn_s_memrealtime(); }

// (XCC_ID << 32) | HW_ID of the executing wave: identifies the compute unit.
__device__ inline int64_t hw_location() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
  return ((int64_t)xcc << 32) | (int64_t)hw;
}

}  // namespace sa
