// Attention over a per-query list of selected keys (DSA, 6D-parallel notes
// section 7.1: gather K and V at the top-k indices, then softmax and the
// weighted sum of V over those keys only).  Scale 1/sqrt(d) unless the problem
// gives one.
//
// One wavefront per query.  A key row of D bf16 values is read by D/8 lanes
// (16 bytes each), so a wave holds 64/(D/8) lane groups, each taking its own
// keys.  One pass: a group gathers the K and V rows of kUnroll keys together,
// forms their scores (in-group reduction over the D/8 lanes) and folds them into
// its online-softmax state (running max, row sum and weighted V sum, rescaled
// when the max grows); the groups' states are merged at the end by the same
// rule.  Scores and weighted V sums are bf16 dot products with fp32 sums (the
// weights rounded to bf16, the value the row sum also adds), so the bf16 rows
// need no conversion.  Bound by the gather: every selected key costs one K row
// and one V row, and a row's address is known only once its index is loaded, so
// the indices of the next kUnroll keys are loaded while the current rows are in
// flight.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sa {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kWaves = 4;
constexpr int kMaxTopK = 2048;
constexpr int kUnroll = 4;  // keys per lane group and step (their K and V rows in flight together)

// x from another lane of the same 16-lane row (a DPP move; CTRL is the DPP control code)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum of x over each aligned group of N lanes (N = 8 or 16), in every lane of the group:
// swaps within quads (lanes ^1, ^2), then the mirrored lane of the 8-lane half row (the
// other quad), then, for 16, the mirrored lane of the row (the other half).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (N == 16) x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// OFF32: a head's rows span less than 2^31 bytes and fewer than 2^23 rows of stride below
// 2^22 elements, so a gathered row's byte offset from the head's base is one 24-bit multiply
// and an add, and the load takes the head's base as its uniform (scalar) address.
template <int D, bool OFF32>
__global__ __launch_bounds__(64 * kWaves) void gather_attn_kernel(GatherArgs a) {
  constexpr int LPR = D / 8;     // lanes per key row
  constexpr int KPI = 64 / LPR;  // lane groups (keys per wave instruction)
  constexpr int STEP = KPI * kUnroll;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gq = (int64_t)blockIdx.x * kWaves + wave;
  if (gq >= (int64_t)a.B * a.H * a.S) return;
  const int bh = (int)(gq / a.S), i = (int)(gq % a.S);
  const int b = bh / a.H, h = bh % a.H;
  const int64_t base = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int grp = lane / LPR, sub = lane % LPR;
  const bf16* gK = (const bf16*)a.k + base + 8 * sub;
  const bf16* gV = (const bf16*)a.v + base + 8 * sub;
  const char* const kbase = (const char*)((const bf16*)a.k + base);  // uniform
  const char* const vbase = (const char*)((const bf16*)a.v + base);
  const int row_bytes = (int)a.ss * 2;
  const int32_t* sel = a.idx + gq * a.top_k;
  const int cnt = a.count[gq];

  const bf16x8 qv = *(const bf16x8*)((const bf16*)a.q + base + (int64_t)i * a.ss + 8 * sub);
  // key u of a step for this group: position t0 + u * KPI + grp of the list (a position
  // past the count reads key 0 and is discarded)
  int kid[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int t = u * KPI + grp;
    const int ld = sel[min(t, a.top_k - 1)];  // always a valid slot of the list
    kid[u] = t < cnt ? ld : 0;
  }
  float m = kNegInf, l = 0.f;  // the group's running max (log2 units) and row sum
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 < cnt; t0 += STEP) {
    bf16x8 kv[kUnroll], vv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if constexpr (OFF32) {
        const uint32_t off = (uint32_t)__mul24(kid[u], row_bytes) + 16u * sub;
        kv[u] = *(const bf16x8*)(kbase + off);
        vv[u] = *(const bf16x8*)(vbase + off);
      } else {
        kv[u] = *(const bf16x8*)(gK + (int64_t)kid[u] * a.ss);
        vv[u] = *(const bf16x8*)(gV + (int64_t)kid[u] * a.ss);
      }
    }
    // the next step's indices, in flight with the rows
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + STEP + u * KPI + grp;
      const int ld = sel[min(t, a.top_k - 1)];
      kid[u] = t < cnt ? ld : 0;
    }
    float s[kUnroll];
    float mx = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // bf16 pair products summed in fp32 (exact products, as the fma form)
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        dot = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{qv[e], qv[e + 1]}, bf16x2{kv[u][e], kv[u][e + 1]}, dot, false);
      dot = group_sum<LPR>(dot);
      s[u] = t0 + u * KPI + grp < cnt ? dot * a.scale_log2 : kNegInf;
      mx = fmaxf(mx, s[u]);
    }
    if (mx == kNegInf) continue;  // (the group has no key in this step, nor before)
    const float alpha = __builtin_amdgcn_exp2f(m - mx);  // exp2(-inf) = 0 for an empty state
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // the weight in bf16 (0 for a discarded key); the row sum adds the same rounded value,
      // and each V element takes it with one bf16 dot product against (p, 0) or (0, p)
      const bf16 pb = (bf16)__builtin_amdgcn_exp2f(s[u] - mx);
      l += (float)pb;
      const bf16x2 p_lo = {pb, (bf16)0.f}, p_hi = {(bf16)0.f, pb};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 v2 = {vv[u][e], vv[u][e + 1]};
        acc[e] = __builtin_amdgcn_fdot2_f32_bf16(v2, p_lo, acc[e], false);
        acc[e + 1] = __builtin_amdgcn_fdot2_f32_bf16(v2, p_hi, acc[e + 1], false);
      }
    }
    m = mx;
  }
  // merge the groups' states (lanes LPR apart hold the same head-dim slice)
#pragma unroll
  for (int w = LPR; w < 64; w <<= 1) {
    const float mo = __shfl_xor(m, w), lo = __shfl_xor(l, w);
    const float mm = fmaxf(m, mo);
    const float ref = mm == kNegInf ? 0.f : mm;
    const float a0 = __builtin_amdgcn_exp2f(m - ref), a1 = __builtin_amdgcn_exp2f(mo - ref);
    l = l * a0 + lo * a1;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a0 + __shfl_xor(acc[e], w) * a1;
    m = mm;
  }
  if (grp == 0) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
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
  const int64_t extent = ((int64_t)(a.S - 1) * a.ss + a.D) * 2;
  const bool off32 = extent < ((int64_t)1 << 31) && a.S < (1 << 23) && a.ss < (1 << 21);
  if (a.D == 128 && off32)
    hipLaunchKernelGGL((gather_attn_kernel<128, true>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else if (a.D == 128)
    hipLaunchKernelGGL((gather_attn_kernel<128, false>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else if (a.D == 64 && off32)
    hipLaunchKernelGGL((gather_attn_kernel<64, true>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else if (a.D == 64)
    hipLaunchKernelGGL((gather_attn_kernel<64, false>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
