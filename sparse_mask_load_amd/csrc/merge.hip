// Online-softmax merge of per-chunk partials (6D-parallel notes, section 2.1).
// Each part holds (O_p, m_p, l_p): its unnormalised output and row sum taken
// relative to its own row maximum m_p.  A row keeps one running triple; taking
// in the next part raises the running maximum to the larger of the two and
// scales both sides' O and l by the exponential of their distance below it
// before adding them.  After the last part the row is O / l, and
// lse = m + log l.  A part with m_p = -inf contributes nothing, so it is
// skipped and its O_p is never read; a row whose every part is empty yields
// O = 0, lse = -inf.
//
// HBM-bound: D/4 threads per row, each folding one 16-byte fp32 vector per part.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
constexpr float kNegInf = -__builtin_huge_valf();

template <int D, typename OutT>
__global__ __launch_bounds__(256) void chunk_merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= a.rows) return;
  const int dq = (threadIdx.x % TPR) * 4;
  float m_acc = kNegInf, l_acc = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  // Parts are read in groups of G: the statistics of the group first, then
  // the O vectors of its non-empty parts, all in flight together; the fold
  // itself runs in part order.
  constexpr int G = 4;
  for (int p0 = 0; p0 < a.n_parts; p0 += G) {
    float mp[G], lp[G];
    f32x4 op[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      mp[i] = p0 + i < a.n_parts ? a.m[p0 + i][row] : kNegInf;
      lp[i] = p0 + i < a.n_parts ? a.l[p0 + i][row] : 0.f;
    }
    // the statistics are complete here; passing them through an empty asm
    // keeps the compiler from waiting on loads in flight at each test below
#pragma unroll
    for (int i = 0; i < G; ++i) asm volatile("" : "+v"(mp[i]));
#pragma unroll
    for (int i = 0; i < G; ++i) {
      op[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      // each O vector is read once: a streaming (nontemporal) load
      if (mp[i] != kNegInf) op[i] = __builtin_nontemporal_load((const f32x4*)(a.o[p0 + i] + row * D + dq));
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (mp[i] == kNegInf) continue;
      const float m_new = fmaxf(m_acc, mp[i]);
      const float alpha = expf(m_acc - m_new);
      const float beta = expf(mp[i] - m_new);
      o = alpha * o + beta * op[i];
      l_acc = alpha * l_acc + beta * lp[i];
      m_acc = m_new;
    }
  }
  const float inv = l_acc > 0.f ? 1.f / l_acc : 0.f;
  OutT* out = (OutT*)a.out + row * D + dq;
  if constexpr (sizeof(OutT) == 2) {
    const bf16x4 v = {(__bf16)(o[0] * inv), (__bf16)(o[1] * inv), (__bf16)(o[2] * inv), (__bf16)(o[3] * inv)};
    *(bf16x4*)out = v;
  } else {
    *(f32x4*)out = o * inv;
  }
  if (a.lse && dq == 0) a.lse[row] = l_acc > 0.f ? m_acc + logf(l_acc) : kNegInf;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int D, int out_dtype, hipStream_t stream) {
  const int rpb = 256 / (D / 4);
  const unsigned grid = (unsigned)((a.rows + rpb - 1) / rpb);
  if (D == 128 && out_dtype == SA_BF16)
    hipLaunchKernelGGL((chunk_merge_kernel<128, __bf16>), dim3(grid), dim3(256), 0, stream, a);
  else if (D == 128 && out_dtype == SA_F32)
    hipLaunchKernelGGL((chunk_merge_kernel<128, float>), dim3(grid), dim3(256), 0, stream, a);
  else if (D == 64 && out_dtype == SA_BF16)
    hipLaunchKernelGGL((chunk_merge_kernel<64, __bf16>), dim3(grid), dim3(256), 0, stream, a);
  else if (D == 64 && out_dtype == SA_F32)
    hipLaunchKernelGGL((chunk_merge_kernel<64, float>), dim3(grid), dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
