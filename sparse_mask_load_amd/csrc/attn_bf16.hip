// Persistent block-sparse flash attention for gfx950, bf16 in / fp32 accumulate.
//
// One workgroup per bin of the LPT plan walks its work items; an item is one
// (batch, head, Q-block) row of the block mask (db-SP post, scenario 2).  For
// each live KV tile of the item, chunk by chunk, the workgroup computes a
// flash-attention tile: S = scale * Q K^T on the matrix cores, a running row
// max m and row sum l, P = exp(S - m), O = alpha*O + P V — the per-step
// flash_attention plus online-softmax update of the ring-attention pseudocode
// in the 6D-parallel notes, section 2.1.  Full mode folds every chunk of the
// range into one state and writes O / l; partial mode writes each chunk's
// (O unnormalised, m, l) and resets the state (the ring step's output).
//
// gfx950 mapping (one wave = 32 query rows, BLOCK/32 waves per workgroup):
//  * The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows are
//    the A operand read from LDS, Q^T the B operand kept in registers for the
//    whole item.  In the accumulator layout a lane then owns one query column
//    and 16 keys per 32-key block, so the row max and row sum are in-lane
//    reductions plus one v_permlane32_swap between the two half-waves.
//  * K rows are loaded permuted within each 32-key block (row bits 2 and 3
//    swapped) so that accumulator register r of half h holds key
//    16*(r/8) + 8*h + r%8: each lane's 8 consecutive P values are then a
//    ready-made B operand of O^T = V^T P^T, and the V^T A operand comes from
//    two ds_read_b64_tr_b16 transposed reads of the row-major V tile.  O^T's
//    accumulator again gives a lane one query column, so the alpha rescale is
//    in-lane too.
//  * K and V tiles are double-buffered in LDS and filled by
//    global_load_lds_dwordx4 (no VGPR staging); tile t+1 streams in while
//    tile t is computed.  16-byte chunks are XOR-swizzled per row so the
//    operand reads above are free of bank conflicts.
//  * exp is exp2 on scores pre-multiplied by scale*log2(e); the exported m is
//    converted back to natural-log units.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace sa {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;

// Row-dependent XOR applied to the 16-byte chunk index of a tile row in LDS.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 128)
    return 2 * (row & 3) + ((row >> 3) & 1) + 8 * ((row >> 2) & 1);
  else
    return 2 * (row & 3) + ((row >> 3) & 1);
}

// Value held by lane l ^ 32.
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// Issue the global->LDS loads of one K and one V tile (this wave's share).
template <int D, int BLK>
__device__ __forceinline__ void load_tile(const bf16* __restrict__ gK, const bf16* __restrict__ gV,
                                          int64_t bh_base, int64_t ss, int S, int layout, int n_chunks,
                                          int desc, bf16* sK, bf16* sV) {
  constexpr int NW = BLK / 32;
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int IPW = BLK * CPR / (64 * NW);      // load instructions per wave per tensor
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int idx = desc & 0xFFFFF;
  const int c = (desc >> kDescChunkShift) & 63;
#pragma unroll
  for (int n = 0; n < IPW; ++n) {
    const int slot0 = (wave * IPW + n) * 64;
    const int slot = slot0 + lane;
    const int r = slot / CPR;
    const int p = slot % CPR;
    const int lc = p ^ chunk_swizzle<D>(r);
    int64_t pos;
    if (layout == SA_LAYOUT_CONTIGUOUS) {
      pos = min(idx * BLK + r, S - 1);
    } else {
      pos = c + (int64_t)n_chunks * ((int64_t)idx * BLK + r);
    }
    const int64_t g = bh_base + pos * ss + lc * 8;
    __builtin_amdgcn_global_load_lds(gK + g, LDS_PTR(void, sK + slot0 * 8), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gV + g, LDS_PTR(void, sV + slot0 * 8), 16, 0, 0);
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void attn_bf16_kernel(FwdArgs a) {
  constexpr int NKB = BLK / 32;  // 32-key blocks per tile
  constexpr int ND = D / 32;     // 32-wide head-dim blocks
  constexpr int NKS = D / 16;    // k-steps of S^T
  constexpr int TILE = BLK * D;
  constexpr int MAXT = BLK >= 128 ? kMaxTilesPerRow : kMaxTilesPerRow / 2;

  __shared__ __attribute__((aligned(1024))) bf16 sK[2][TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][TILE];
  __shared__ int sList[MAXT];
  __shared__ int sCount;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const bool full = a.o != nullptr;
  const bool striped = a.layout == SA_LAYOUT_STRIPED;
  const int kb_div = striped ? NKB / a.n_chunks : NKB;  // key blocks per liveness group
  const bf16* __restrict__ gQ = (const bf16*)a.q;
  const bf16* __restrict__ gK = (const bf16*)a.k;
  const bf16* __restrict__ gV = (const bf16*)a.v;

  // Per-lane LDS operand offsets (independent of tile, key block and step).
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);  // bits 2,3 swapped
  const int k_off = krow * D;
  const int k_swz = chunk_swizzle<D>(krow);
  int v_off[2], v_swz[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int vrow = 8 * h2 + 4 * rr + ((lane & 15) >> 2);
    v_off[rr] = vrow * D + 4 * (lane & 1);
    v_swz[rr] = chunk_swizzle<D>(vrow);
  }
  const int v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);

  const int bin = blockIdx.x;
  const int p_begin = a.bin_ptr[bin], p_end = a.bin_ptr[bin + 1];
  const float sl2 = a.scale_log2;

  for (int pos = p_begin; pos < p_end; ++pos) {
    const int64_t t_start = realtime_now();
    const int item = a.items[pos];
    const int qb = item % a.nQ;
    const int bh = item / a.nQ;
    const int b = bh / a.H, h = bh % a.H;
    const int64_t bh_base = (int64_t)b * a.sb + (int64_t)h * a.sh;

    // Q^T operand of this wave's 32 rows: lane holds row q0 + l32, dims 16*ks + 8*h2 .. +7.
    const int qrow = qb * BLK + wave * 32 + l32;
    const int qrow_c = min(qrow, a.S - 1);
    bf16x8 qf[NKS];
    {
      const bf16* qp = gQ + bh_base + (int64_t)qrow_c * a.ss + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    }

    __syncthreads();  // every wave is done with the previous item's list and tiles
    if (wave == 0) {
      const int n = build_tile_list(a.mask + (int64_t)item * a.nK, a.nK, a.n_chunks, a.layout, a.c0,
                                    a.c1, sList);
      if (lane == 0) sCount = n;
    }
    __syncthreads();
    const int n_tiles = sCount;

    f32x16 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;
    int cur_chunk = a.c0;

    auto flush_partial = [&](int chunk) {
      const float l_tot = l_run + other_half(l_run);
      if (qrow < a.S) {
        const int64_t prow = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + qrow;
        float* op = a.o_part + prow * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v4 = {acc[d][4 * g], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]};
            *(f32x4*)(op + d * 32 + 8 * g + 4 * h2) = v4;
          }
        if (h2 == 0) {
          a.m_part[prow] = m_run * kLn2;
          a.l_part[prow] = l_tot;
        }
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
      m_run = kNegInf;
      l_run = 0.f;
    };

    if (n_tiles > 0)
      load_tile<D, BLK>(gK, gV, bh_base, a.ss, a.S, a.layout, a.n_chunks, sList[0], sK[0], sV[0]);

    for (int t = 0; t < n_tiles; ++t) {
      const int desc = __builtin_amdgcn_readfirstlane(sList[t]);
      const int tchunk = (desc >> kDescChunkShift) & 63;
      if (!full)
        while (cur_chunk < tchunk) flush_partial(cur_chunk++);

      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // tile t is in LDS; tile t-1's buffer is free
      if (t + 1 < n_tiles)
        load_tile<D, BLK>(gK, gV, bh_base, a.ss, a.S, a.layout, a.n_chunks,
                          __builtin_amdgcn_readfirstlane(sList[t + 1]), sK[(t + 1) & 1], sV[(t + 1) & 1]);

      const bf16* Kt = sK[t & 1];
      const bf16* Vt = sV[t & 1];
      const int code = (desc >> kDescCodeShift) & 15;
      const int tidx = desc & 0xFFFFF;
      const bool ragged = !striped && (tidx + 1) * BLK > a.S;
      const int key0 = tidx * BLK;

      // S^T = K Q^T for the live 32-key blocks.
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        if (!((code >> (kb / kb_div)) & 1)) continue;
        const bf16* kp = Kt + kb * 32 * D + k_off;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 kv = *(const bf16x8*)(kp + (((2 * ks + h2) ^ k_swz) << 3));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qf[ks], s[kb], 0, 0, 0);
        }
      }

      // Online softmax (row = this lane's query column).
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (!((code >> (kb / kb_div)) & 1)) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r];
          if (ragged) {
            const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * h2 + (r & 7);
            if (key >= a.S) x = kNegInf;
            s[kb][r] = x;
          }
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, other_half(mx));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[d] *= alpha;

      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (!((code >> (kb / kb_div)) & 1)) continue;
        bf16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -m_new));
          lsum += p;
          pb[r >> 3][r & 7] = (bf16)p;
        }
        // O^T += V^T P^T over this block's two 16-key steps.
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16* vp = Vt + (kb * 32 + 16 * st) * D;
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const int ch = 4 * d + v_chunk;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                LDS_PTR(bf16x4, vp + v_off[0] + ((ch ^ v_swz[0]) << 3)));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                LDS_PTR(bf16x4, vp + v_off[1] + ((ch ^ v_swz[1]) << 3)));
            const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[st], acc[d], 0, 0, 0);
          }
        }
      }
      l_run += lsum;
    }

    if (!full) {
      while (cur_chunk < a.c1) flush_partial(cur_chunk++);
    } else {
      const float l_tot = l_run + other_half(l_run);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (qrow < a.S) {
        bf16* op = (bf16*)a.o + bh_base + (int64_t)qrow * a.ss;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const bf16x4 v4 = {(bf16)(acc[d][4 * g] * inv), (bf16)(acc[d][4 * g + 1] * inv),
                               (bf16)(acc[d][4 * g + 2] * inv), (bf16)(acc[d][4 * g + 3] * inv)};
            *(bf16x4*)(op + d * 32 + 8 * g + 4 * h2) = v4;
          }
      }
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

hipError_t launch_attn_bf16(const FwdArgs& a, int D, int block, hipStream_t stream) {
  if (D == 128 && block == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<128, 128>), dim3(a.num_bins), dim3(256), 0, stream, a);
  else if (D == 64 && block == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<64, 128>), dim3(a.num_bins), dim3(256), 0, stream, a);
  else if (D == 128 && block == 64)
    hipLaunchKernelGGL((attn_bf16_kernel<128, 64>), dim3(a.num_bins), dim3(128), 0, stream, a);
  else if (D == 64 && block == 64)
    hipLaunchKernelGGL((attn_bf16_kernel<64, 64>), dim3(a.num_bins), dim3(128), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
