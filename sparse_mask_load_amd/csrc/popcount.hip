// Block-mask popcounts: the per-Q-block and per-KV-block work of the db-SP
// post (scenario 2: a Q-block's work is its mask row sum, a KV-block's its
// column sum), plus each row's count per KV chunk (one ring step's shard).
//
// One workgroup per (batch, head) mask of nQ x nK bytes (16 KiB for a
// 128 x 128 mask).  Row and chunk counts: a thread per row reads the row in
// 16-byte vectors and counts its non-zero bytes with a bit trick (4 bytes per
// 32-bit word; a byte is non-zero iff its low 7 bits are or its top bit is).
// Column counts: a thread per column walks the rows with coalesced byte loads.
// Counts are integers accumulated exactly.  The grand total is the sum of the
// row counts, taken on the host.  With Q-block pairs (prow non-null) a thread
// per pair p also counts the union of rows 2p and 2p+1 (the OR of their bytes),
// in total and per chunk: the tiles the pair's work item visits.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sa {
namespace {

__device__ __forceinline__ int nonzero_bytes(uint32_t v) {
  const uint32_t low7 = (v & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;  // top bit of a byte: its low 7 bits are non-zero
  return __builtin_popcount((low7 | v) & 0x80808080u);
}

__global__ __launch_bounds__(256) void popcount_kernel(const uint8_t* __restrict__ mask, int nQ, int nK,
                                                       int n_chunks, int layout, int32_t* __restrict__ row,
                                                       int32_t* __restrict__ col, int32_t* __restrict__ crow,
                                                       int32_t* __restrict__ prow, int32_t* __restrict__ pcrow) {
  const int bh = blockIdx.x;
  const uint8_t* m = mask + (int64_t)bh * nQ * nK;
  const int per_chunk = nK / n_chunks;
  const bool vec = per_chunk % 16 == 0 && nK % 16 == 0;  // rows and chunks split into whole 16-byte vectors
  for (int i = threadIdx.x; i < nQ; i += blockDim.x) {
    const uint8_t* mr = m + (int64_t)i * nK;
    int tot = 0;
    for (int c = 0; c < n_chunks; ++c) {
      int cnt = 0;
      if (vec) {
        for (int j = c * per_chunk; j < (c + 1) * per_chunk; j += 16) {
          const uint4 v = *(const uint4*)(mr + j);
          cnt += nonzero_bytes(v.x) + nonzero_bytes(v.y) + nonzero_bytes(v.z) + nonzero_bytes(v.w);
        }
      } else {
        for (int j = c * per_chunk; j < (c + 1) * per_chunk; ++j) cnt += mr[j] != 0;
      }
      tot += cnt;
      if (layout == SA_LAYOUT_CONTIGUOUS) crow[((int64_t)bh * n_chunks + c) * nQ + i] = cnt;
    }
    row[(int64_t)bh * nQ + i] = tot;
    // striped: every chunk holds a 1/n_chunks slice of each live block, so each chunk's load is the row's
    if (layout == SA_LAYOUT_STRIPED)
      for (int c = 0; c < n_chunks; ++c) crow[((int64_t)bh * n_chunks + c) * nQ + i] = tot;
  }
  if (prow) {
    const int nP = (nQ + 1) / 2;
    for (int p = threadIdx.x; p < nP; p += blockDim.x) {
      const uint8_t* ma = m + (int64_t)(2 * p) * nK;
      const bool has_b = 2 * p + 1 < nQ;
      const uint8_t* mb = has_b ? ma + nK : ma;  // a lone last row is its own union
      int tot = 0;
      for (int c = 0; c < n_chunks; ++c) {
        int cnt = 0;
        if (vec) {
          for (int j = c * per_chunk; j < (c + 1) * per_chunk; j += 16) {
            const uint4 va = *(const uint4*)(ma + j), vb = *(const uint4*)(mb + j);
            cnt += nonzero_bytes(va.x | vb.x) + nonzero_bytes(va.y | vb.y) + nonzero_bytes(va.z | vb.z) +
                   nonzero_bytes(va.w | vb.w);
          }
        } else {
          for (int j = c * per_chunk; j < (c + 1) * per_chunk; ++j) cnt += (ma[j] | mb[j]) != 0;
        }
        tot += cnt;
        if (layout == SA_LAYOUT_CONTIGUOUS) pcrow[((int64_t)bh * n_chunks + c) * nP + p] = cnt;
      }
      prow[(int64_t)bh * nP + p] = tot;
      // striped: every chunk holds a slice of each live block, so each chunk's load is the pair's
      if (layout == SA_LAYOUT_STRIPED)
        for (int c = 0; c < n_chunks; ++c) pcrow[((int64_t)bh * n_chunks + c) * nP + p] = tot;
    }
  }
  for (int j = threadIdx.x; j < nK; j += blockDim.x) {
    int cnt = 0;
    int i = 0;
    for (; i + 4 <= nQ; i += 4)
      cnt += (m[(int64_t)i * nK + j] != 0) + (m[(int64_t)(i + 1) * nK + j] != 0) +
             (m[(int64_t)(i + 2) * nK + j] != 0) + (m[(int64_t)(i + 3) * nK + j] != 0);
    for (; i < nQ; ++i) cnt += m[(int64_t)i * nK + j] != 0;
    col[(int64_t)bh * nK + j] = cnt;
  }
}

}  // namespace

hipError_t launch_popcount(const uint8_t* mask, int BH, int nQ, int nK, int n_chunks, int layout, int32_t* row,
                           int32_t* col, int32_t* crow, hipStream_t stream, int32_t* prow, int32_t* pcrow) {
  if (BH == 0) return hipSuccess;
  hipLaunchKernelGGL(popcount_kernel, dim3(BH), dim3(256), 0, stream, mask, nQ, nK, n_chunks, layout, row, col,
                     crow, prow, pcrow);
  return hipGetLastError();
}

}  // namespace sa
