// Persistent block-sparse attention in fp32 (vector ALU, no reduced-precision
// modes), for block 64 and head dim 64 or 128.
//
// Same algorithm and work list as the bf16 matrix-core kernel: each workgroup
// walks its bin's (batch, head, Q-block) items; per live KV tile it computes
// S = scale * Q K^T, updates the running max m and sum l, rescales O by
// alpha = exp(m_old - m_new) and adds exp(S - m) V (ring-attention step and
// online-softmax update, 6D-parallel notes section 2.1).  The tile math runs on
// plain fp32 FMAs through LDS: 4 threads per query row, 16 keys each.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace sa {
namespace {

constexpr int BLK = 64;
constexpr int NT = 256;
constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
__global__ __launch_bounds__(NT) void attn_f32_kernel(FwdArgs a) {
  constexpr int DQ = D / 4;  // head dims per thread in P V
  __shared__ float sQ[BLK][D + 1];
  __shared__ float sK[BLK][D + 1];
  __shared__ float sV[BLK][D];
  __shared__ float sP[BLK][BLK + 1];
  __shared__ int sList[kMaxTilesPerRow];
  __shared__ int sCount;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = tid >> 2, quarter = tid & 3;
  const bool full = a.o != nullptr;
  const bool striped = a.layout == SA_LAYOUT_STRIPED;
  const float* __restrict__ gQ = (const float*)a.q;
  const float* __restrict__ gK = (const float*)a.k;
  const float* __restrict__ gV = (const float*)a.v;
  const int bin = blockIdx.x;
  const int p_begin = a.bin_ptr[bin], p_end = a.bin_ptr[bin + 1];

  for (int pos = p_begin; pos < p_end; ++pos) {
    const int64_t t_start = realtime_now();
    const int item = a.items[pos];
    const int qb = item % a.nQ;
    const int bh = item / a.nQ;
    const int b = bh / a.H, h = bh % a.H;
    const int64_t bh_base = (int64_t)b * a.sb + (int64_t)h * a.sh;
    const int qrow = qb * BLK + row;

    __syncthreads();
    for (int e = tid; e < BLK * D; e += NT) {
      const int r = e / D, d = e % D;
      sQ[r][d] = gQ[bh_base + (int64_t)min(qb * BLK + r, a.S - 1) * a.ss + d];
    }
    if (wave == 0) {
      const int n = build_tile_list(a.mask + (int64_t)item * a.nK, a.nK, a.n_chunks, a.layout, a.c0,
                                    a.c1, sList);
      if (lane == 0) sCount = n;
    }
    __syncthreads();
    const int n_tiles = sCount;

    float o[DQ];
    for (int d = 0; d < DQ; ++d) o[d] = 0.f;
    float m_run = kNegInf, l_run = 0.f;  // identical in the 4 threads of a row
    int cur_chunk = a.c0;

    auto flush_partial = [&](int chunk) {
      if (qrow < a.S) {
        const int64_t prow = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + qrow;
        for (int d = 0; d < DQ; ++d) a.o_part[prow * D + quarter * DQ + d] = o[d];
        if (quarter == 0) {
          a.m_part[prow] = m_run;
          a.l_part[prow] = l_run;
        }
      }
      for (int d = 0; d < DQ; ++d) o[d] = 0.f;
      m_run = kNegInf;
      l_run = 0.f;
    };

    for (int t = 0; t < n_tiles; ++t) {
      const int desc = sList[t];
      const int tchunk = (desc >> kDescChunkShift) & 63;
      if (!full)
        while (cur_chunk < tchunk) flush_partial(cur_chunk++);
      const int tidx = desc & 0xFFFFF;
      const int code = (desc >> kDescCodeShift) & 15;
      __syncthreads();
      for (int e = tid; e < BLK * D; e += NT) {
        const int r = e / D, d = e % D;
        int64_t p;
        if (!striped)
          p = min(tidx * BLK + r, a.S - 1);
        else
          p = tchunk + (int64_t)a.n_chunks * ((int64_t)tidx * BLK + r);
        sK[r][d] = gK[bh_base + p * a.ss + d];
        sV[r][d] = gV[bh_base + p * a.ss + d];
      }
      __syncthreads();

      float s[16];
      float mx = kNegInf;
      for (int jj = 0; jj < 16; ++jj) {
        const int j = quarter * 16 + jj;
        bool live;
        int kpos;  // token position of key j
        if (!striped) {
          kpos = tidx * BLK + j;
          live = kpos < a.S;
        } else {
          kpos = tchunk + a.n_chunks * (tidx * BLK + j);
          live = (code >> (j / (BLK / a.n_chunks))) & 1;
        }
        if (a.token_causal && kpos > qrow) live = false;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(sQ[row][d], sK[j][d], acc);
        s[jj] = live ? acc * a.scale : kNegInf;
        mx = fmaxf(mx, s[jj]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      const float m_new = fmaxf(m_run, mx);
      // a row with no finite score yet (token-causal) keeps p = 0 and alpha = 0
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = expf(m_run - m_use);
      float lsum = 0.f;
      for (int jj = 0; jj < 16; ++jj) {
        const float p = expf(s[jj] - m_use);
        lsum += p;
        sP[row][quarter * 16 + jj] = p;
      }
      lsum += __shfl_xor(lsum, 1);
      lsum += __shfl_xor(lsum, 2);
      l_run = alpha * l_run + lsum;
      m_run = m_new;
      __syncthreads();
      for (int d = 0; d < DQ; ++d) o[d] *= alpha;
      for (int j = 0; j < BLK; ++j) {
        const float p = sP[row][j];
        for (int d = 0; d < DQ; ++d) o[d] = fmaf(p, sV[j][quarter * DQ + d], o[d]);
      }
    }

    if (!full) {
      while (cur_chunk < a.c1) flush_partial(cur_chunk++);
    } else if (qrow < a.S) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      float* op = (float*)a.o + bh_base + (int64_t)qrow * a.ss + quarter * DQ;
      for (int d = 0; d < DQ; ++d) op[d] = o[d] * inv;
    }
    if (a.trace && tid == 0) {
      int64_t* tr = a.trace + (int64_t)pos * 4;
      tr[0] = t_start;
      tr[1] = realtime_now();
      tr[2] = hw_location();
      tr[3] = ((int64_t)bin << 32) | (int64_t)(uint32_t)item;
    }
  }
}

}  // namespace

hipError_t launch_attn_f32(const FwdArgs& a, int D, int block, hipStream_t stream) {
  if (block != BLK) return hipErrorInvalidValue;
  if (D == 64)
    hipLaunchKernelGGL((attn_f32_kernel<64>), dim3(a.num_bins), dim3(NT), 0, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128>), dim3(a.num_bins), dim3(NT), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
