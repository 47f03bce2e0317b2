// Attention over a per-query list of selected keys (DSA, 6D-parallel notes
// section 7.1: gather K and V at the top-k indices, then softmax and the
// weighted sum of V over those keys only).  Scale 1/sqrt(d) unless the problem
// gives one.
//
// One wavefront per query.  A key row of D bf16 values is read by D/8 lanes
// (16 bytes each), so a wave reads 64/(D/8) gathered rows per instruction.
// Pass 1 forms the scores (in-group reduction over the D/8 lanes) into LDS;
// pass 2 takes the max, the exp2 weights and the weighted V sum; the partial
// sums of the row groups are combined at the end.  Bound by the gather: every
// selected key costs one K row and one V row, and a row's address is known
// only once its index is loaded, so each pass issues kUnroll independent row
// loads per lane group before it uses any of them (a few: occupancy, which the
// LDS score buffer sized to top_k keeps high, matters more than depth per wave).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sa {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kWaves = 4;
constexpr int kMaxTopK = 2048;
constexpr int kUnroll = 4;  // gathered rows in flight per lane group

template <int D>
__global__ __launch_bounds__(64 * kWaves) void gather_attn_kernel(GatherArgs a) {
  constexpr int LPR = D / 8;     // lanes per key row
  constexpr int KPI = 64 / LPR;  // key rows per wave instruction
  extern __shared__ float sScore[];  // [kWaves][top_k]: sized by the launch, so short lists keep occupancy
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gq = (int64_t)blockIdx.x * kWaves + wave;
  if (gq >= (int64_t)a.B * a.H * a.S) return;
  const int bh = (int)(gq / a.S), i = (int)(gq % a.S);
  const int b = bh / a.H, h = bh % a.H;
  const int64_t base = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int grp = lane / LPR, sub = lane % LPR;
  const bf16* gK = (const bf16*)a.k + base + 8 * sub;
  const bf16* gV = (const bf16*)a.v + base + 8 * sub;
  const int32_t* sel = a.idx + gq * a.top_k;
  const int cnt = a.count[gq];
  float* sc = sScore + wave * a.top_k;

  float q[8];
  {
    const bf16x8 qv = *(const bf16x8*)((const bf16*)a.q + base + (int64_t)i * a.ss + 8 * sub);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (float)qv[e];
  }
  float mx = kNegInf;
  for (int t0 = 0; t0 < cnt; t0 += KPI * kUnroll) {
    // indices first (a missing one reads key 0 and is discarded), then all rows, then the math
    int kidx[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * KPI + grp;
      kidx[u] = t < cnt ? sel[t] : 0;
    }
    bf16x8 kv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) kv[u] = *(const bf16x8*)(gK + (int64_t)kidx[u] * a.ss);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * KPI + grp;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(q[e], (float)kv[u][e], dot);
#pragma unroll
      for (int w = LPR / 2; w >= 1; w >>= 1) dot += __shfl_xor(dot, w);
      const float s2 = dot * a.scale_log2;
      if (t < cnt) {
        if (sub == 0) sc[t] = s2;
        mx = fmaxf(mx, s2);
      }
    }
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) mx = fmaxf(mx, __shfl_xor(mx, w));
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  for (int t0 = 0; t0 < cnt; t0 += KPI * kUnroll) {
    int vidx[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * KPI + grp;
      vidx[u] = t < cnt ? sel[t] : 0;
    }
    bf16x8 vv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) vv[u] = *(const bf16x8*)(gV + (int64_t)vidx[u] * a.ss);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * KPI + grp;
      const float sv = sc[t < cnt ? t : 0];  // no read past the query's scores
      const float p = t < cnt ? __builtin_amdgcn_exp2f(sv - mx) : 0.f;
      if (sub == 0) lsum += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, (float)vv[u][e], acc[e]);
    }
  }
#pragma unroll
  for (int w = LPR; w < 64; w <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], w);
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) lsum += __shfl_xor(lsum, w);
  if (grp == 0) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    bf16x8 ov;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = (bf16)(acc[e] * inv);
    *(bf16x8*)((bf16*)a.o + base + (int64_t)i * a.ss + 8 * sub) = ov;
  }
}

}  // namespace

hipError_t launch_gather_attn(const GatherArgs& a, hipStream_t stream) {
  if (a.top_k > kMaxTopK) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)a.B * a.H * a.S;
  const unsigned grid = (unsigned)((rows + kWaves - 1) / kWaves);
  const size_t lds = (size_t)kWaves * a.top_k * sizeof(float);
  if (a.D == 128)
    hipLaunchKernelGGL((gather_attn_kernel<128>), dim3(grid), dim3(64 * kWaves), lds, stream, a);
  else if (a.D == 64)
    hipLaunchKernelGGL((gather_attn_kernel<64>), dim3(grid), dim3(64 * kWaves), lds, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
