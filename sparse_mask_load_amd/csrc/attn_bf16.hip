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
//  * One K and one V tile live in LDS (72 KiB with the tile list), so two
//    workgroups share a compute unit and every SIMD holds two waves: one
//    wave's softmax (VALU) runs while the other's MFMAs execute.  Tiles are
//    filled by global_load_lds_dwordx4 (no VGPR staging) on a two-barrier
//    schedule: K of tile t+1 streams in during the softmax and P V of tile t,
//    V of tile t+1 during S of tile t+1.  16-byte chunks are XOR-swizzled per
//    row so the operand reads above are free of bank conflicts.
//  * exp is exp2 on scores pre-multiplied by scale*log2(e).  The reference max
//    used in the exponent only moves when a row's max grows by more than 2^8
//    (the result O/l does not depend on the reference), so O is rarely
//    rescaled; the true row max is tracked and the exported partial is
//    converted to it, in natural-log units.  The row sum adds the bf16-rounded
//    P values that also feed P V (v_dot2c_f32_bf16).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace sa {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: P values stay below 2^8

template <int D, int BLK>
struct Shape {
  static constexpr int NW = BLK / 32;    // waves per workgroup
  static constexpr int NKB = BLK / 32;   // 32-key blocks per tile
  static constexpr int ND = D / 32;      // 32-wide head-dim blocks
  static constexpr int NKS = D / 16;     // k-steps of S^T
  static constexpr int TILE = BLK * D;
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int IPW = BLK * CPR / (64 * NW);  // load instructions per wave per tile
  static constexpr int WG_PER_CU = BLK >= 128 ? 2 : 4;
};

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

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Where the rows of one K/V tile live in global memory: row r of the tile is
// element base + r * row_stride; rows at or beyond `rows` repeat the last
// valid row (the partial last block of a ragged sequence).
struct TileSrc {
  int64_t base;
  int row_stride;
  int rows;
};

__device__ __forceinline__ TileSrc tile_source(int desc, int64_t bh_base, int64_t ss, int S, int layout,
                                               int n_chunks, int BLK) {
  const int idx = desc & 0xFFFFF;
  const int c = (desc >> kDescChunkShift) & 63;
  TileSrc t;
  if (layout == SA_LAYOUT_CONTIGUOUS) {
    t.base = bh_base + (int64_t)idx * BLK * ss;
    t.row_stride = (int)ss;
    t.rows = min(BLK, S - idx * BLK);
  } else {  // compacted position p of chunk c is token c + n_chunks * p
    t.base = bh_base + ((int64_t)c + (int64_t)n_chunks * idx * BLK) * ss;
    t.row_stride = (int)(ss * n_chunks);
    t.rows = BLK;
  }
  return t;
}

// Per-lane part of the tile loads.  Load instruction n of a wave writes the
// 64 consecutive 16-byte LDS slots (wave*IPW + n)*64 + lane; slot s holds row
// s / CPR, physical chunk s % CPR, i.e. logical chunk (s % CPR) ^ swizzle(row).
// For the shapes here the swizzle of row lane_row + n*RPI is the lane's base
// swizzle XOR a constant of n, so one XOR per instruction finds the chunk.
template <int D, int BLK>
struct TileLoader {
  int lane_row;    // tile row of this lane's slot in instruction 0
  int lane_chunk;  // logical chunk of that slot, before the per-instruction constant
  __device__ __forceinline__ void init(int wave, int lane) {
    using SH = Shape<D, BLK>;
    constexpr int RPI = 64 / SH::CPR;
    lane_row = wave * SH::IPW * RPI + lane / SH::CPR;
    lane_chunk = (lane % SH::CPR) ^ chunk_swizzle<D>(lane_row);
  }
  static __device__ __forceinline__ constexpr int chunk_xor(int n) {
    // swizzle(row + n*RPI) ^ swizzle(row) for rows with bits 0-1 from the lane and IPW % 4 == 0
    return D == 128 ? (((n >> 1) & 1) | (8 * (n & 1))) : (n & 1);
  }
  template <bool MAY_CLAMP>
  __device__ __forceinline__ void issue(const bf16* __restrict__ g, const TileSrc& src, bf16* lds, int wave) const {
    using SH = Shape<D, BLK>;
    constexpr int RPI = 64 / SH::CPR;
    static_assert(SH::IPW % 4 == 0 || D == 64, "row bits 2-3 of a load instruction must come from n");
    const bf16* gt = g + src.base;
    const bool clamp = MAY_CLAMP && src.rows < BLK;
#pragma unroll
    for (int n = 0; n < SH::IPW; ++n) {
      int r = lane_row + n * RPI;
      if (clamp) r = min(r, src.rows - 1);
      const uint32_t off = (uint32_t)(r * src.row_stride + ((lane_chunk ^ chunk_xor(n)) << 3));
      __builtin_amdgcn_global_load_lds(gt + off, LDS_PTR(void, lds + (wave * SH::IPW + n) * 64 * 8), 16, 0, 0);
    }
  }
};

// Online-softmax state of one wave (32 query rows; a lane owns row l % 32).
template <int ND>
struct RowState {
  f32x16 acc[ND];  // O^T (unnormalised, relative to m_ref)
  float m_ref;     // reference max used in the exponent (log2 units)
  float m_true;    // true running max (log2 units)
  float l;         // this lane's share of the row sum (relative to m_ref)
};

template <int ND>
__device__ __forceinline__ void reset(RowState<ND>& st) {
#pragma unroll
  for (int d = 0; d < ND; ++d) st.acc[d] = f32x16{};
  st.m_ref = kNegInf;
  st.m_true = kNegInf;
  st.l = 0.f;
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// One live tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
// GENERAL = false: every 32-key block is live and no key lies beyond S (the
// common case, straight-line code).  GENERAL = true: live_kb has bit kb set
// when key block kb holds live keys (striped layout) and `ragged` masks keys
// at or beyond S (the last, partial block).
// LDS operand reads are issued two MFMAs ahead of their use.
template <int D, int BLK, bool GENERAL>
__device__ __forceinline__ void tile_step(const bf16* __restrict__ Kt, const bf16* __restrict__ Vt,
                                          const bf16x8 (&qf)[D / 16], RowState<D / 32>& st, int live_kb,
                                          bool ragged, int key0, float sl2, int k_off, int k_swz,
                                          const int (&v_off)[2], const int (&v_swz)[2], int v_chunk, int h2,
                                          bool last, const FwdArgs& a, const TileLoader<D, BLK>& loader,
                                          const TileSrc& next, int wave, bf16* kbuf, bf16* vbuf) {
  using SH = Shape<D, BLK>;
  auto kb_live = [&](int kb) { return !GENERAL || ((live_kb >> kb) & 1); };

  f32x16 s[SH::NKB];
#pragma unroll
  for (int kb = 0; kb < SH::NKB; ++kb) {
    if (!kb_live(kb)) continue;
    const bf16* kp = Kt + kb * 32 * D + k_off;
    bf16x8 kf[SH::NKS];
#pragma unroll
    for (int ks = 0; ks < SH::NKS; ++ks) kf[ks] = *(const bf16x8*)(kp + (((2 * ks + h2) ^ k_swz) << 3));
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < SH::NKS; ++ks) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s[kb], 0, 0, 0);
    SCHED_GROUP(kSchedDsRead, 2);
#pragma unroll
    for (int ks = 0; ks < SH::NKS - 2; ++ks) {
      SCHED_GROUP(kSchedMfma, 1);
      SCHED_GROUP(kSchedDsRead, 1);
    }
    SCHED_GROUP(kSchedMfma, 2);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Barrier A: every wave is done reading K of this tile and V of this tile has landed.
  wait_vm();
  __syncthreads();
  if (!last) loader.template issue<GENERAL>((const bf16*)a.k, next, kbuf, wave);

  if (GENERAL && ragged) {
#pragma unroll
    for (int kb = 0; kb < SH::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + kb * 32 + 16 * (r >> 3) + 8 * h2 + (r & 7) >= a.S) s[kb][r] = kNegInf;
  }
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < SH::NKB; ++kb) {
    if (!kb_live(kb)) continue;
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
  }
  mx = fmaxf(mx, other_half(mx)) * sl2;
  st.m_true = fmaxf(st.m_true, mx);
  if (__builtin_amdgcn_ballot_w64(mx > st.m_ref + kRescaleSlack)) {
    const float m_new = (mx > st.m_ref + kRescaleSlack) ? st.m_true : st.m_ref;
    const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);
    st.m_ref = m_new;
    st.l *= alpha;
#pragma unroll
    for (int d = 0; d < SH::ND; ++d) st.acc[d] *= alpha;
  }
  const float m_ref = st.m_ref;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  float lsum0 = 0.f, lsum1 = 0.f;

#pragma unroll
  for (int kb = 0; kb < SH::NKB; ++kb) {
    if (!kb_live(kb)) continue;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -m_ref));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lsum0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0][2 * e], pb[0][2 * e + 1]}, ones, lsum0, false);
      lsum1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[1][2 * e], pb[1][2 * e + 1]}, ones, lsum1, false);
    }
    bf16x8 va[2][SH::ND];
#pragma unroll
    for (int stp = 0; stp < 2; ++stp) {
      const bf16* vp = Vt + (kb * 32 + 16 * stp) * D;
#pragma unroll
      for (int d = 0; d < SH::ND; ++d) {
        const int ch = 4 * d + v_chunk;
        const bf16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vp + v_off[0] + ((ch ^ v_swz[0]) << 3)));
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vp + v_off[1] + ((ch ^ v_swz[1]) << 3)));
        va[stp][d] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
#pragma unroll
    for (int stp = 0; stp < 2; ++stp)
#pragma unroll
      for (int d = 0; d < SH::ND; ++d)
        st.acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[stp][d], pb[stp], st.acc[d], 0, 0, 0);
    // two transposed reads per MFMA operand, issued one operand ahead
    SCHED_GROUP(kSchedDsRead, 4);
#pragma unroll
    for (int i = 0; i < 2 * SH::ND - 2; ++i) {
      SCHED_GROUP(kSchedMfma, 1);
      SCHED_GROUP(kSchedDsRead, 2);
    }
    SCHED_GROUP(kSchedMfma, 2);
  }
  st.l += lsum0 + lsum1;

  // Barrier B: every wave is done reading V of this tile and K of the next tile has landed.
  wait_vm();
  __syncthreads();
  if (!last) loader.template issue<GENERAL>((const bf16*)a.v, next, vbuf, wave);
}

// GENERAL: the problem has striped chunks or a partial last block, so a tile
// may have dead 32-key groups or keys beyond S; otherwise every tile is full.
template <int D, int BLK, bool GENERAL>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(FwdArgs a) {
  using SH = Shape<D, BLK>;
  __shared__ __attribute__((aligned(1024))) bf16 sK[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV[SH::TILE];
  __shared__ int sList[kMaxTilesPerRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const bool full = a.o != nullptr;
  const bool striped = a.layout == SA_LAYOUT_STRIPED;
  const int kb_div = striped ? SH::NKB / a.n_chunks : SH::NKB;
  TileLoader<D, BLK> loader;
  loader.init(wave, lane);  // key blocks per liveness group
  const bf16* __restrict__ gQ = (const bf16*)a.q;

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
    bf16x8 qf[SH::NKS];
    {
      const bf16* qp = gQ + bh_base + (int64_t)qrow_c * a.ss + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < SH::NKS; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    }

    __syncthreads();  // every wave is done with the previous item's list and tiles
    // every wave counts the live tiles; wave 0 also writes the list
    const int n_tiles = build_tile_list(a.mask + (int64_t)item * a.nK, a.nK, a.n_chunks, a.layout, a.c0, a.c1,
                                        sList, wave == 0);
    __syncthreads();
    const int* list = sList;

    RowState<SH::ND> st;
    reset(st);
    int cur_chunk = a.c0;

    auto flush_partial = [&](int chunk) {
      const bool any = st.m_true != kNegInf;
      const float corr = any ? __builtin_amdgcn_exp2f(st.m_ref - st.m_true) : 0.f;
      const float l_tot = (st.l + other_half(st.l)) * corr;
      if (qrow < a.S) {
        const int64_t prow = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + qrow;
        float* op = a.o_part + prow * D;
#pragma unroll
        for (int d = 0; d < SH::ND; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v4 = {st.acc[d][4 * g] * corr, st.acc[d][4 * g + 1] * corr, st.acc[d][4 * g + 2] * corr,
                              st.acc[d][4 * g + 3] * corr};
            *(f32x4*)(op + d * 32 + 8 * g + 4 * h2) = v4;
          }
        if (h2 == 0) {
          a.m_part[prow] = any ? st.m_true * kLn2 : kNegInf;
          a.l_part[prow] = l_tot;
        }
      }
      reset(st);
    };

    if (n_tiles > 0) {
      const TileSrc src0 = tile_source(__builtin_amdgcn_readfirstlane(list[0]), bh_base, a.ss, a.S, a.layout,
                                       a.n_chunks, BLK);
      loader.template issue<GENERAL>((const bf16*)a.k, src0, sK, wave);
      loader.template issue<GENERAL>((const bf16*)a.v, src0, sV, wave);
      wait_vm();
      __syncthreads();
    }

    for (int t = 0; t < n_tiles; ++t) {
      const int desc = __builtin_amdgcn_readfirstlane(list[t]);
      const bool last = t + 1 == n_tiles;
      const int next_desc = last ? 0 : __builtin_amdgcn_readfirstlane(list[t + 1]);
      const int tchunk = (desc >> kDescChunkShift) & 63;
      if (!full)
        while (cur_chunk < tchunk) flush_partial(cur_chunk++);
      const int code = (desc >> kDescCodeShift) & 15;
      const int tidx = desc & 0xFFFFF;
      const int key0 = tidx * BLK;
      int live_kb = (1 << SH::NKB) - 1;
      if (striped) {
        live_kb = 0;
#pragma unroll
        for (int kb = 0; kb < SH::NKB; ++kb) live_kb |= ((code >> (kb / kb_div)) & 1) << kb;
      }
      const bool ragged = !striped && key0 + BLK > a.S;
      const TileSrc next = tile_source(next_desc, bh_base, a.ss, a.S, a.layout, a.n_chunks, BLK);
      tile_step<D, BLK, GENERAL>(sK, sV, qf, st, live_kb, ragged, key0, sl2, k_off, k_swz, v_off, v_swz, v_chunk,
                                 h2, last, a, loader, next, wave, sK, sV);
    }

    if (!full) {
      while (cur_chunk < a.c1) flush_partial(cur_chunk++);
    } else {
      const float l_tot = st.l + other_half(st.l);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (qrow < a.S) {
        bf16* op = (bf16*)a.o + bh_base + (int64_t)qrow * a.ss;
#pragma unroll
        for (int d = 0; d < SH::ND; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const bf16x4 v4 = {(bf16)(st.acc[d][4 * g] * inv), (bf16)(st.acc[d][4 * g + 1] * inv),
                               (bf16)(st.acc[d][4 * g + 2] * inv), (bf16)(st.acc[d][4 * g + 3] * inv)};
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

int attn_bf16_wg_per_cu(int block) { return block >= 128 ? 2 : 4; }

template <int D, int BLK>
hipError_t launch_variant(const FwdArgs& a, hipStream_t stream) {
  const bool general = a.layout == SA_LAYOUT_STRIPED || a.S % BLK != 0;
  if (general)
    hipLaunchKernelGGL((attn_bf16_kernel<D, BLK, true>), dim3(a.num_bins), dim3(BLK * 2), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, BLK, false>), dim3(a.num_bins), dim3(BLK * 2), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const FwdArgs& a, int D, int block, hipStream_t stream) {
  if (D == 128 && block == 128) return launch_variant<128, 128>(a, stream);
  if (D == 64 && block == 128) return launch_variant<64, 128>(a, stream);
  if (D == 128 && block == 64) return launch_variant<128, 64>(a, stream);
  if (D == 64 && block == 64) return launch_variant<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
