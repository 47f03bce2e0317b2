// Block-mask popcounts: the per-Q-block and per-KV-block work of the db-SP
// post (scenario 2: a Q-block's work is its mask row sum, a KV-block's its
// column sum), plus each row's count per KV chunk (one ring step's shard).
//
// rows:  one wavefront per mask row; 64 mask bytes per ballot, so a row of nK
//        entries costs nK/64 coalesced 64-byte reads.
// cols:  one thread per column, walking the rows (each step reads 64
//        consecutive bytes across the wavefront).
// Counts are integers accumulated exactly; the total uses a 64-bit atomic add,
// whose result does not depend on the order of the additions.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sa {
namespace {

__global__ __launch_bounds__(256) void popcount_rows_kernel(const uint8_t* __restrict__ mask, int n_rows,
                                                            int nQ, int nK, int n_chunks, int layout,
                                                            int32_t* __restrict__ row,
                                                            int32_t* __restrict__ crow,
                                                            unsigned long long* __restrict__ total) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const uint8_t* m = mask + (int64_t)r * nK;
  const int bh = r / nQ, i = r % nQ;
  const int per_chunk = nK / n_chunks;
  int tot = 0;
  for (int c = 0; c < n_chunks; ++c) {
    int cnt = 0;
    const int j1 = (c + 1) * per_chunk;
    for (int base = c * per_chunk; base < j1; base += 64) {
      const int j = base + lane;
      cnt += __popcll(__ballot(j < j1 && m[j] != 0));
    }
    tot += cnt;
    if (layout == SA_LAYOUT_CONTIGUOUS && lane == 0) crow[((int64_t)bh * n_chunks + c) * nQ + i] = cnt;
  }
  if (lane == 0) {
    row[r] = tot;
    if (layout == SA_LAYOUT_STRIPED)
      for (int c = 0; c < n_chunks; ++c) crow[((int64_t)bh * n_chunks + c) * nQ + i] = tot;
    atomicAdd(total, (unsigned long long)tot);
  }
}

__global__ __launch_bounds__(256) void popcount_cols_kernel(const uint8_t* __restrict__ mask, int BH,
                                                            int nQ, int nK, int32_t* __restrict__ col) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)BH * nK) return;
  const int bh = (int)(g / nK), j = (int)(g % nK);
  const uint8_t* m = mask + (int64_t)bh * nQ * nK + j;
  int cnt = 0;
  for (int i = 0; i < nQ; ++i) cnt += m[(int64_t)i * nK] != 0;
  col[g] = cnt;
}

}  // namespace

hipError_t launch_popcount(const uint8_t* mask, int BH, int nQ, int nK, int n_chunks, int layout,
                           int32_t* row, int32_t* col, int32_t* crow, unsigned long long* total,
                           hipStream_t stream) {
  const int n_rows = BH * nQ;
  hipError_t e = hipMemsetAsync(total, 0, sizeof(unsigned long long), stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(popcount_rows_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, stream, mask, n_rows, nQ,
                     nK, n_chunks, layout, row, crow, total);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_cols = (int64_t)BH * nK;
  hipLaunchKernelGGL(popcount_cols_kernel, dim3((unsigned)((n_cols + 255) / 256)), dim3(256), 0, stream,
                     mask, BH, nQ, nK, col);
  return hipGetLastError();
}

}  // namespace sa
