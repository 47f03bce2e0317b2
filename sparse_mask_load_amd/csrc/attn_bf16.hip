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
// gfx950 mapping (a wave owns 32 query rows and one half of the keys of every
// tile; two waves per SIMD, so the matrix cores run one wave's MFMAs while the
// other wave does its softmax arithmetic):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows are the A operand read
//    from LDS, Q^T the B operand kept in registers for the whole item.  In the
//    accumulator layout a lane owns one query column and 16 keys per 32-key
//    block, so the row max and row sum are in-lane reductions plus one
//    v_permlane32_swap between the two half-waves.
//  * K rows are loaded permuted within each 32-key block (row bits 2 and 3
//    swapped) so that accumulator register r of half h holds key
//    16*(r/8) + 8*h + r%8: each lane's 8 consecutive P values are then a
//    ready-made B operand of O^T = V^T P^T, and the V^T A operand comes from
//    two ds_read_b64_tr_b16 transposed reads of the row-major V tile.  O^T's
//    accumulator again gives a lane one query column, so the alpha rescale is
//    in-lane too.
//  * The two key halves of a row keep separate online-softmax states (each is
//    a flash-attention pass over a disjoint key subset) and are merged through
//    LDS with the same rule that merges chunks, when a chunk is flushed and at
//    the end of the item.
//  * Two kernels share this mapping.  The pipelined kernel (128-key tiles, S a
//    multiple of the block; contiguous or striped chunks, with or without
//    token-level causality) runs each wave as a stream of 32-key blocks: one
//    section per block issues the S MFMAs of the block two ahead and the P V
//    MFMAs of the current block, each MFMA slot also holding the LDS operand
//    reads four MFMAs ahead and one stage of the next block's softmax, with
//    scheduling fences between the slots.  The general kernel (64-key tiles,
//    ragged S) takes the row max per tile and reads operands just before use.
//  * K and V tiles are double-buffered in LDS (128 KiB for 128-key tiles, four
//    separate arrays so that the compiler can tell operand reads from loads in
//    flight) and filled by buffer_load_dwordx4 ... lds (no VGPR staging), with
//    one workgroup barrier per tile.  16-byte chunks are XOR-swizzled per row
//    so that the operand reads are free of bank conflicts.
//  * exp is exp2 on scores pre-multiplied by scale*log2(e).  The reference max
//    used in the exponent only moves when a row's max grows by more than a
//    factor 2^8 (the result O/l does not depend on the reference), so O is
//    rarely rescaled (the pipelined kernel checks per 32-key block and brings
//    the accumulators to a block's reference just before that block's P V);
//    the true row max is tracked and the exported partial is converted to it,
//    in natural-log units.  The row sum adds the bf16-rounded
//    P values that also feed P V (v_dot2c_f32_bf16).
#include <hip/hip_runtime.h>

#include <type_traits>

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
  static constexpr int NRG = BLK / 32;   // 32-row groups of a Q block
  static constexpr int NW = 2 * NRG;     // waves per workgroup: row group x key half
  static constexpr int NKB = BLK / 32;   // 32-key blocks per tile
  static constexpr int NKBW = NKB / 2;   // key blocks of one wave (its half of the tile)
  static constexpr int ND = D / 32;      // 32-wide head-dim blocks
  static constexpr int NKS = D / 16;     // k-steps of S^T
  static constexpr int TILE = BLK * D;
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int IPW = BLK * CPR / (64 * NW);  // load instructions per wave per tile
  static constexpr int WG_PER_CU = 8 / NW;           // two waves per SIMD
  static constexpr int RB = ND / 2;                  // head-dim blocks per merge round
};

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time loop).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Row-dependent XOR applied to the 16-byte chunk index of a tile row in LDS.
// The LDS serves 256 bytes (64 banks) per clock: 16 lanes of a ds_read_b128 or
// 32 lanes of a ds_read_b64_tr_b16.  The K-operand read touches 16 different
// rows (bits 0-3 of the row index all vary) at one logical chunk, so the XOR
// must be a bijection on row % 16; the V^T read touches 4 consecutive rows
// (4*i .. 4*i+3) at 4 consecutive chunks, so those rows need different chunk
// bits 2-3 (D = 128; for D = 64 two rows share a 256-byte bank line, so rows of
// equal parity need different chunk bit 2).
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 128)
    return 4 * (row & 3) + ((row >> 2) & 3);
  else
    return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Value held by lane l ^ 32.
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// The value of x, opaque to the compiler: computations derived from it stay
// where they are written instead of being hoisted (and kept live) elsewhere.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without the memory fence of __syncthreads, whose release part waits for
// every load and store the wave has in flight: for a barrier that only orders LDS reads that
// are complete (consumed by the instructions that needed them) before tile loads that
// overwrite them.  The compiler moves no memory access across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Run-time work queue (the list-scheduling form of LPT).  The queue holds the items in LPT
// order; its positions are dealt to the 8 XCDs in turn (position i belongs to XCD i mod 8, as
// workgroup b runs on XCD b mod 8), one counter per XCD.  One thread of a workgroup takes its
// XCD's next position with a device-scope atomic add, so the items that share a head's K/V
// in one LPT round stay on one XCD's L2; once its XCD's positions are all taken it takes
// another XCD's next one.  Every position below n is returned exactly once (each comes from
// one counter value), n means the queue is empty.  The last workgroup to finish returns the
// counters (ctr[0..7] next positions, ctr[8] finished workgroups) to zero for the next launch.
__device__ __forceinline__ int queue_take(int32_t* ctr, int n) {
  const int home = blockIdx.x & 7;
  const int c = __hip_atomic_fetch_add(ctr + home, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (c * 8 + home < n) return c * 8 + home;
  for (int k = 1; k < 8; ++k) {
    const int x = (home + k) & 7;
    // (a counter only grows: one read as exhausted stays exhausted)
    if (__hip_atomic_load(ctr + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * 8 + x >= n) continue;
    const int cx = __hip_atomic_fetch_add(ctr + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (cx * 8 + x < n) return cx * 8 + x;
  }
  return n;
}
__device__ __forceinline__ void queue_finish(int32_t* ctr) {
  if (__hip_atomic_fetch_add(ctr + 8, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
#pragma unroll
    for (int x = 0; x < 9; ++x) __hip_atomic_store(ctr + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

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
// swizzle XOR a constant of n, so the byte offset of every slot in the tile
// depends only on the row stride and is computed once per item.  The loads
// are buffer loads through a per-tile resource whose base is the tile's first
// row, so no vector address arithmetic is left per tile.
template <int D, int BLK>
struct TileLoader {
  static constexpr int IPW = Shape<D, BLK>::IPW;
  static constexpr int RPI = 64 / Shape<D, BLK>::CPR;  // rows per load instruction
  int lane_row;    // tile row of this lane's slot in instruction 0
  int lane_chunk;  // logical chunk of that slot, before the per-instruction constant
  uint32_t voff[IPW];
  __device__ __forceinline__ void init(int wave, int lane) {
    lane_row = wave * IPW * RPI + lane / Shape<D, BLK>::CPR;
    lane_chunk = (lane % Shape<D, BLK>::CPR) ^ chunk_swizzle<D>(lane_row);
  }
  static __device__ __forceinline__ constexpr int chunk_xor(int n) {
    // swizzle(lane_row + n*RPI) ^ swizzle(lane_row): row bits below log2(RPI) come from the lane,
    // the bits above from wave*IPW + n, whose low bits are those of n (IPW is a multiple of 4
    // for D = 128 and of 2 for D = 64, the bits the swizzle reads)
    return D == 128 ? (n & 3) : 2 * (n & 1);
  }
  __device__ __forceinline__ uint32_t slot_offset(int row, int n, int row_stride) const {
    return (uint32_t)(row * row_stride + ((lane_chunk ^ chunk_xor(n)) << 3)) * 2u;
  }
  // Per-item byte offsets of this lane's slots (rows are row_stride elements apart).
  __device__ __forceinline__ void set_stride(int row_stride) {
    static_assert(IPW % (D == 128 ? 4 : 2) == 0, "row bits of a load instruction above the lane bits must come from n");
#pragma unroll
    for (int n = 0; n < IPW; ++n) voff[n] = slot_offset(lane_row + n * RPI, n, row_stride);
  }
  // Issues load instructions n0 .. n1-1 of this wave (all of them by default).
  // Rows at or beyond src.rows (partial last block) repeat the last valid row.
  template <bool MAY_CLAMP, int N0 = 0, int N1 = IPW>
  __device__ __forceinline__ void issue(const bf16* __restrict__ g, const TileSrc& src, bf16* lds, int wave) const {
    const uint32_t bytes = (uint32_t)((src.rows - 1) * src.row_stride + D) * 2u;  // extent of the valid rows
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(g + src.base), 0, bytes, 0x00020000);
    const bool clamp = MAY_CLAMP && src.rows < BLK;
#pragma unroll
    for (int n = N0; n < N1; ++n) {
      const uint32_t off = clamp ? slot_offset(min(lane_row + n * RPI, src.rows - 1), n, src.row_stride) : voff[n];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, lds + (wave * IPW + n) * 64 * 8), 16, off, 0, 0, 0);
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

// Per-lane LDS operand geometry (independent of tile, key block and step);
// key block j of a wave is block kb0 + j of the tile.  PINNED: the element
// offsets of every read are formed once and pinned, so that each read is one
// register plus an immediate (the buffer's address and the key-block offset)
// with no address arithmetic left per tile (measured faster in the full-tile
// variant); otherwise the row base and the swizzle are combined per read
// (measured faster where scores are masked per element).
template <int D, bool PINNED>
struct OperandLanes;

template <int D>
struct OperandLanes<D, true> {
  int k_ofs[D / 16];     // K rows at k-step ks
  int v_ofs[D / 32][2];  // the two V^T row quads of head-dim block d
  __device__ __forceinline__ void init(int lane, int kb0) {
    const int h2 = lane >> 5;
    const int l32 = lane & 31;
    const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);  // bits 2,3 swapped
    const int k_swz = chunk_swizzle<D>(krow);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      k_ofs[ks] = (kb0 * 32 + krow) * D + (((2 * ks + h2) ^ k_swz) << 3);
      asm volatile("" : "+v"(k_ofs[ks]));
    }
    const int v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int vrow = 8 * h2 + 4 * rr + ((lane & 15) >> 2);
      const int v_swz = chunk_swizzle<D>(vrow);
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        v_ofs[d][rr] = (kb0 * 32 + vrow) * D + 4 * (lane & 1) + (((4 * d + v_chunk) ^ v_swz) << 3);
        asm volatile("" : "+v"(v_ofs[d][rr]));
      }
    }
  }
  // K rows of 32-key block kb at k-step ks (A operand of S^T).
  __device__ __forceinline__ bf16x8 k_frag(const bf16* Kt, int kb, int ks) const {
    return *(const bf16x8*)(Kt + kb * 32 * D + k_ofs[ks]);
  }
  // V^T rows of head-dim block d for the 16-key step `half` of key block kb (A operand of O^T).
  __device__ __forceinline__ bf16x8 v_frag(const bf16* Vt, int kb, int half, int d) const {
    const bf16* vp = Vt + (kb * 32 + 16 * half) * D;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vp + v_ofs[d][0]));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vp + v_ofs[d][1]));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

template <int D>
struct OperandLanes<D, false> {
  int k_off, k_swz, h2;
  int v_off[2], v_swz[2], v_chunk;
  __device__ __forceinline__ void init(int lane, int kb0) {
    h2 = lane >> 5;
    const int l32 = lane & 31;
    const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);  // bits 2,3 swapped
    k_off = (kb0 * 32 + krow) * D;
    k_swz = chunk_swizzle<D>(krow);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int vrow = 8 * h2 + 4 * rr + ((lane & 15) >> 2);
      v_off[rr] = (kb0 * 32 + vrow) * D + 4 * (lane & 1);
      v_swz[rr] = chunk_swizzle<D>(vrow);
    }
    v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  }
  __device__ __forceinline__ bf16x8 k_frag(const bf16* Kt, int kb, int ks) const {
    return *(const bf16x8*)(Kt + kb * 32 * D + k_off + (((2 * ks + h2) ^ k_swz) << 3));
  }
  __device__ __forceinline__ bf16x8 v_frag(const bf16* Vt, int kb, int half, int d) const {
    const bf16* vp = Vt + (kb * 32 + 16 * half) * D;
    const int ch = 4 * d + v_chunk;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vp + v_off[0] + ((ch ^ v_swz[0]) << 3)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, vp + v_off[1] + ((ch ^ v_swz[1]) << 3)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// S^T = K Q^T of the wave's key blocks of one tile, k-step major: one MFMA per
// live 32-key block per step, the K fragments of the next step read while the
// current MFMAs run.
template <int D, int BLK, bool GENERAL, class OL>
__device__ __forceinline__ void tile_scores(const bf16* __restrict__ Kt, const bf16x8 (&qf)[D / 16],
                                            const OL& ol, int live_w, f32x16 (&s)[BLK / 64]) {
  using SH = Shape<D, BLK>;
  constexpr int NB = SH::NKBW, NKS = SH::NKS;
  auto live = [&](int j) { return !GENERAL || ((live_w >> j) & 1); };
  bf16x8 kf[2][NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (live(j)) kf[0][j] = ol.k_frag(Kt, j, 0);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks + 1 < NKS) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (live(j)) kf[(ks + 1) & 1][j] = ol.k_frag(Kt, j, ks + 1);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (live(j))
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks & 1][j], qf[ks], ks == 0 ? f32x16{} : s[j], 0, 0, 0);
  }
}

// Row max of the wave's tile scores and the lazy move of the exponent's
// reference max.  When `masked`, score (j, r) is first dropped if its key
// offset j*32 + 16*(r>>3) + (r&7) within the lane's keys exceeds off_max (keys
// beyond S on a ragged tile, keys after the query on a diagonal tile).
// Returns the reference to use: 0 for a row that has no finite score yet, so
// that its dropped scores give probabilities 0 rather than exp(-inf + inf).
template <int D, int BLK, bool GENERAL, bool MASKED>
__device__ __forceinline__ float tile_max(f32x16 (&s)[BLK / 64], RowState<D / 32>& st, int live_w, bool masked,
                                          int off_max, float sl2) {
  using SH = Shape<D, BLK>;
  auto live = [&](int j) { return !GENERAL || ((live_w >> j) & 1); };
  if (MASKED && masked) {
#pragma unroll
    for (int j = 0; j < SH::NKBW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (j * 32 + 16 * (r >> 3) + (r & 7) > off_max) s[j][r] = kNegInf;
  }
  float mx;
  if constexpr (!MASKED) {
    // two running maxima, each taking two scores per step (one v_max3 each)
    float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
    for (int j = 0; j < SH::NKBW; ++j) {
      if (!live(j)) continue;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        mx0 = fmaxf(fmaxf(mx0, s[j][r]), s[j][r + 1]);
        mx1 = fmaxf(fmaxf(mx1, s[j][r + 2]), s[j][r + 3]);
      }
    }
    mx = fmaxf(mx0, mx1);
  } else {
    // pairwise form: measured faster in the variants that mask scores per element
    mx = kNegInf;
#pragma unroll
    for (int j = 0; j < SH::NKBW; ++j) {
      if (!live(j)) continue;
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[j][r], s[j][r + 1]));
    }
  }
  mx = fmaxf(mx, other_half(mx)) * sl2;
  st.m_true = fmaxf(st.m_true, mx);
  if (__builtin_amdgcn_ballot_w64(mx > st.m_ref + kRescaleSlack)) {
    // while every lane's reference is -inf the state is still all zeros (nothing
    // has been accumulated), so the first move of the reference needs no rescale
    const bool fresh = !__builtin_amdgcn_ballot_w64(st.m_ref != kNegInf);
    const float m_new = (mx > st.m_ref + kRescaleSlack) ? st.m_true : st.m_ref;
    // a lane with no finite score yet (possible only under token-level causality) keeps
    // its zero state: alpha = 1 instead of exp2(-inf - -inf)
    const float alpha = (MASKED && m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(st.m_ref - m_new);
    st.m_ref = m_new;
    if (!fresh) {
      st.l *= alpha;
#pragma unroll
      for (int d = 0; d < SH::ND; ++d) st.acc[d] *= alpha;
    }
  }
  return (MASKED && st.m_ref == kNegInf) ? 0.f : st.m_ref;
}

// P of one key block as two bf16x8 B operands (keys 16*half + 8*h2 + 0..7),
// accumulating the row sum of the rounded values.
__device__ __forceinline__ void tile_probs(const f32x16& s, float sl2, float m_ref, bf16x8 (&pb)[2], float& lsum0,
                                           float& lsum1) {
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[r], sl2, -m_ref));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lsum0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0][2 * e], pb[0][2 * e + 1]}, ones, lsum0, false);
    lsum1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[1][2 * e], pb[1][2 * e + 1]}, ones, lsum1, false);
  }
}

// Folds the key-half-1 state of every row group into the key-half-0 wave of the
// same rows (the merge rule of two partials over disjoint keys).  Called by all
// waves of the workgroup at the same point (it has barriers); kscr and mscr are
// LDS buffers that no wave reads or loads into meanwhile.  On return the
// half-0 wave holds, in the true-max basis, acc (unnormalised O^T), m (true row
// max, log2 units, -inf for a row without keys) and l_row (full row sum).  Each
// half's move from its lazy reference to its true max (corr) is folded into
// the merge factors, so the accumulators are scaled once.
template <int D, int BLK>
__device__ __forceinline__ void merge_halves(RowState<D / 32>& st, float& m, float& l_row, float* kscr, float* mscr,
                                             int rg, int kh, int lane) {
  using SH = Shape<D, BLK>;
  constexpr int ND = SH::ND, RB = SH::RB;
  const bool any = st.m_true != kNegInf;
  const float corr = any ? __builtin_amdgcn_exp2f(st.m_ref - st.m_true) : 0.f;
  m = st.m_true;
  l_row = (st.l + other_half(st.l)) * corr;
  const int l32 = lane & 31;
  float fa = 1.f, fb = 0.f;
#pragma unroll
  for (int round = 0; round < ND / RB; ++round) {
    // kscr layout: [row group][block i of the round][group g of 4 registers][lane] f32x4
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v4 = {st.acc[round * RB + i][4 * g], st.acc[round * RB + i][4 * g + 1],
                            st.acc[round * RB + i][4 * g + 2], st.acc[round * RB + i][4 * g + 3]};
          *(f32x4*)(kscr + (((rg * RB + i) * 4 + g) * 64 + lane) * 4) = v4;
        }
      // mscr layout: [row group][m of 32 rows | l of 32 rows | corr of 32 rows]
      if (round == 0) {
        mscr[rg * 96 + lane] = lane < 32 ? m : l_row;
        if (lane < 32) mscr[rg * 96 + 64 + lane] = corr;
      }
    }
    __syncthreads();
    if (kh == 0) {
      if (round == 0) {
        const float mo = mscr[rg * 96 + l32], lo = mscr[rg * 96 + 32 + l32], co = mscr[rg * 96 + 64 + l32];
        const float mn = fmaxf(m, mo);
        fa = mn == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        fb = mn == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        l_row = l_row * fa + lo * fb;
        m = mn;
        fa *= corr;  // this half's accumulators are still relative to its lazy reference
        fb *= co;    // and so are the other half's
      }
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v4 = *(const f32x4*)(kscr + (((rg * RB + i) * 4 + g) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st.acc[round * RB + i][4 * g + e] = st.acc[round * RB + i][4 * g + e] * fa + v4[e] * fb;
        }
    }
    __syncthreads();
  }
}

// GENERAL: the problem has striped chunks or a partial last block, so a tile
// may have dead 32-key groups or keys beyond S; otherwise every tile is full.
// Token-level causality (keys after some of a tile's queries) is handled by the
// GENERAL variant, or by TCAUSAL on top of the full-tile one.
template <int D, int BLK, bool GENERAL, bool TCAUSAL>
__global__ __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(FwdArgs a) {
  using SH = Shape<D, BLK>;
  constexpr bool MASKED = GENERAL || TCAUSAL;  // scores may be dropped per element
  static_assert(SH::NW * 64 == BLK * 4, "launch bounds");
  constexpr int NKB = SH::NKB, NB = SH::NKBW, ND = SH::ND, NKS = SH::NKS, NRG = SH::NRG;
  static_assert(SH::TILE * 2 >= NRG * SH::RB * 4096, "merge round must fit in a K buffer");
  static_assert(SH::TILE * 2 >= NRG * 96 * 4, "merge statistics must fit in a V buffer");
  // Four separate LDS arrays (not one indexed array): the compiler can then
  // prove that operand reads of one buffer do not alias the tile loads in
  // flight into another, and need not wait for those loads to land.
  __shared__ __attribute__((aligned(1024))) bf16 sK0[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[SH::TILE];
  __shared__ int sList[kMaxTilesPerRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % NRG, kh = wave / NRG;  // row group, key half
  const int kb0 = kh * NB;                     // first key block of this wave
  const int h2 = lane >> 5, l32 = lane & 31;
  const bool full = a.o != nullptr;
  const bool striped = a.layout == SA_LAYOUT_STRIPED;
  const int kb_div = striped ? NKB / a.n_chunks : NKB;  // key blocks per liveness group
  TileLoader<D, BLK> loader;
  loader.init(wave, lane);
  loader.set_stride(striped ? (int)(a.ss * a.n_chunks) : (int)a.ss);
  OperandLanes<D, !MASKED> ol;
  ol.init(lane, kb0);
  const bf16* __restrict__ gQ = (const bf16*)a.q;
  const bf16* __restrict__ gK = (const bf16*)a.k;
  const bf16* __restrict__ gV = (const bf16*)a.v;
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
    const int qrow = qb * BLK + rg * 32 + l32;
    const int qrow_c = min(qrow, a.S - 1);
    bf16x8 qf[NKS];
    {
      const bf16* qp = gQ + bh_base + (int64_t)qrow_c * a.ss + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    }

    __syncthreads();  // every wave is done with the previous item's list, tiles and merge buffers
    // every wave counts the live tiles; wave 0 also writes the list
    const int n_tiles = build_tile_list(a.mask + (int64_t)item * a.nK, a.nK, a.n_chunks, a.layout, a.c0, a.c1,
                                        sList, wave == 0);
    __syncthreads();

    RowState<ND> st;
    reset(st);
    int cur_chunk = a.c0;
    bool acc_live = false;  // the accumulation in progress has taken a tile (uniform)

    // Merges the two key halves and writes chunk `chunk`'s partial (O in the
    // true-max basis, m in natural-log units, l), then resets the state.
    // The merged O rows are staged through the two free tile buffers (rows
    // [0, BLK/2) in kscr, the rest in mscr, 16-byte chunks XOR-swizzled by
    // row) and then stored by all waves as whole rows, so that each store
    // instruction writes contiguous rows instead of 32-byte pieces of 32 rows.
    auto flush_partial = [&](int chunk, float* kscr, float* mscr) {
      constexpr int CH = D / 4;                // 16-byte chunks per fp32 row
      constexpr int HALF = BLK / 2;            // rows per staging buffer
      constexpr int RPS = 64 / CH;             // rows per store instruction
      constexpr int NST = BLK / SH::NW / RPS;  // store instructions per wave
      static_assert(HALF * D * 4 <= SH::TILE * 2, "staging half must fit in a tile buffer");
      static_assert(NST * RPS * SH::NW == BLK, "store rows must cover the block");
      // lane-derived addresses are formed here, not kept live across the tile loop
      const int ln = opaque(lane), l32 = ln & 31, h2 = ln >> 5;
      float m, l_row;
      merge_halves<D, BLK>(st, m, l_row, kscr, mscr, rg, kh, ln);
      const int64_t prow0 = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + (int64_t)qb * BLK;
      if (kh == 0) {
        const int r = rg * 32 + l32;  // a wave's 32 rows lie in one staging buffer
        float* const rowp = (rg * 32 < HALF ? kscr : mscr) + (r % HALF) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = 8 * d + 2 * g + h2;
            const f32x4 v4 = {st.acc[d][4 * g], st.acc[d][4 * g + 1], st.acc[d][4 * g + 2], st.acc[d][4 * g + 3]};
            *(f32x4*)(rowp + 4 * (c ^ (r & (CH - 1)))) = v4;
          }
        if (h2 == 0 && qrow < a.S) {
          a.m_part[prow0 + r] = m == kNegInf ? kNegInf : m * kLn2;
          a.l_part[prow0 + r] = l_row;
        }
      }
      __syncthreads();
      {
        // rows [wave*NST*RPS, (wave+1)*NST*RPS) of one staging buffer
        const float* const buf = (wave * NST * RPS < HALF ? kscr : mscr);
        const int c = ln % CH;
#pragma unroll 1
        for (int i = 0; i < NST; ++i) {
          const int r = (wave * NST + i) * RPS + ln / CH;
          const f32x4 v4 = *(const f32x4*)(buf + (r % HALF) * D + 4 * (c ^ (r & (CH - 1))));
          if (qb * BLK + r < a.S) *(f32x4*)(a.o_part + (prow0 + r) * D + 4 * c) = v4;
        }
      }
      __syncthreads();  // the staging buffers are free again (tile loads go there next)
      reset(st);
    };
    // An empty accumulation's partial, (0, -inf, 0), is written by every wave for its own
    // rows, with no merge of the key halves and no staging (nor their barriers).
    auto flush_empty = [&](int chunk) {
      constexpr int RPW = BLK / SH::NW;  // rows per wave
      const int ln = opaque(lane);
      const int64_t prow0 = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + (int64_t)qb * BLK;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      static_assert(RPW * (D / 4) % 64 == 0, "the wave's rows split evenly over its lanes");
#pragma unroll
      for (int k = 0; k < RPW * (D / 4) / 64; ++k) {
        const int idx = ln + 64 * k;
        const int r = wave * RPW + idx / (D / 4), c = idx % (D / 4);
        if (qb * BLK + r < a.S) *(f32x4*)(a.o_part + (prow0 + r) * D + 4 * c) = z;
      }
      if (ln < RPW && qb * BLK + wave * RPW + ln < a.S) {
        a.m_part[prow0 + wave * RPW + ln] = kNegInf;
        a.l_part[prow0 + wave * RPW + ln] = 0.f;
      }
    };
    auto flush_chunk = [&](int chunk, float* kscr, float* mscr) {
      if (acc_live)
        flush_partial(chunk, kscr, mscr);
      else
        flush_empty(chunk);
      acc_live = false;
    };
    // live bits of this wave's key blocks of a tile
    auto live_of = [&](int desc) {
      int live = (1 << NB) - 1;
      if (striped) {
        const int code = (desc >> kDescCodeShift) & 15;
        live = 0;
#pragma unroll
        for (int j = 0; j < NB; ++j) live |= ((code >> ((kb0 + j) / kb_div)) & 1) << j;
      }
      return live;
    };
    auto src_of = [&](int desc) { return tile_source(desc, bh_base, a.ss, a.S, a.layout, a.n_chunks, BLK); };

    // Prologue: K and V of tile 0, K of tile 1; S of tile 0.
    f32x16 s[NB];
    if (n_tiles > 0) {
      const int d0 = __builtin_amdgcn_readfirstlane(sList[0]);
      loader.template issue<GENERAL>(gK, src_of(d0), sK0, wave);
      loader.template issue<GENERAL>(gV, src_of(d0), sV0, wave);
      if (n_tiles > 1)
        loader.template issue<GENERAL>(gK, src_of(__builtin_amdgcn_readfirstlane(sList[1])), sK1, wave);
      wait_vm();
      __syncthreads();
      tile_scores<D, BLK, GENERAL>(sK0, qf, ol, live_of(d0), s);
    }

    // One tile per call; the parity P = t & 1 selects the buffers at compile
    // time (tile t reads K of tile t+1 and V of tile t, and loads K of tile t+2
    // and V of tile t+1).
    auto tile = [&](int t, auto parity) {
      constexpr int P = decltype(parity)::value;
      bf16* const kfree = P ? sK1 : sK0;  // K of tile t: consumed, refilled below
      bf16* const vfree = P ? sV0 : sV1;  // V of tile t-1: consumed, refilled below
      const bf16* const Kt1 = P ? sK0 : sK1;  // K of tile t+1
      const bf16* const Vt = P ? sV1 : sV0;   // V of tile t
      const int desc = __builtin_amdgcn_readfirstlane(sList[t]);
      const bool has_next = t + 1 < n_tiles;
      // the fast variant always computes "next" scores (discarded after the last tile) so that
      // the S MFMAs and the exponentials share one basic block
      const int desc1 = has_next ? __builtin_amdgcn_readfirstlane(sList[t + 1]) : desc;
      const int live_w = live_of(desc);
      // Token positions of the wave's keys: kpos0 + kstep * offset (a striped
      // chunk's compacted position p is token chunk + n_chunks * p).
      const int key0 = (desc & 0xFFFFF) * BLK + kb0 * 32;
      const int kstep = striped ? a.n_chunks : 1;
      const int kpos0 = striped ? ((desc >> kDescChunkShift) & 63) + a.n_chunks * key0 : key0;
      const bool ragged = !striped && key0 - kb0 * 32 + BLK > a.S;
      // diagonal: the wave's last key lies after its first query
      const bool diag = MASKED && a.token_causal && kpos0 + kstep * (NB * 32 - 1) > qb * BLK + rg * 32;
      int off_max = 0;
      if (MASKED && (ragged || diag)) {
        const int rel = (diag ? min(qrow, a.S - 1) : a.S - 1) - kpos0 - kstep * 8 * h2;
        off_max = rel < 0 ? -1 : rel / kstep;
      }

      // K of tile t+1 and V of tile t have landed; K of tile t and V of tile t-1 are free.
      wait_vm();
      __syncthreads();
      if (!full) {
        const int tchunk = (desc >> kDescChunkShift) & 63;
        while (cur_chunk < tchunk) flush_chunk(cur_chunk++, (float*)kfree, (float*)vfree);
        acc_live = true;  // this tile belongs to the accumulation of chunk tchunk
      }
      // K of tile t+2 and V of tile t+1 are loaded in slices, one per key block,
      // so that no wave stalls on a full memory-request queue.  Near the end of
      // the list the slices reload the last tile into a buffer that is free
      // (this keeps the loop body branch-free; the loads are drained below).
      const TileSrc srcK = src_of(__builtin_amdgcn_readfirstlane(sList[min(t + 2, n_tiles - 1)]));
      const TileSrc srcV = src_of(desc1);

      // Rolling pipeline over the wave's 32-key blocks j of tile t: the
      // exponentials of block j of tile t (VALU), the S MFMAs of block j of
      // tile t+1 and the P V MFMAs of block j of tile t all issue in one basic
      // block; block j of the scores is overwritten by tile t+1 once its
      // probabilities are formed.
      const float m_ref = tile_max<D, BLK, GENERAL, MASKED>(s, st, live_w, ragged || diag, off_max, sl2);
      const int live_next = live_of(desc1);
      float lsum0 = 0.f, lsum1 = 0.f;
      constexpr int LPB = SH::IPW / NB;  // load instructions per tensor per key block
      static_assert(SH::IPW % NB == 0, "loads must split evenly over the key blocks");
      static_for<NB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        loader.template issue<GENERAL, j * LPB, (j + 1) * LPB>(gK, srcK, kfree, wave);
        loader.template issue<GENERAL, j * LPB, (j + 1) * LPB>(gV, srcV, vfree, wave);
        bf16x8 pb[2];
        const bool live_now = !GENERAL || ((live_w >> j) & 1);
        if (live_now) tile_probs(s[j], sl2, m_ref, pb, lsum0, lsum1);
        if (!GENERAL || (has_next && ((live_next >> j) & 1))) {
          bf16x8 kf[NKS];
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) kf[ks] = ol.k_frag(Kt1, j, ks);
          s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
          for (int ks = 1; ks < NKS; ++ks)
            s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s[j], 0, 0, 0);
        }
        if (!live_now) return;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 va[ND];
#pragma unroll
          for (int d = 0; d < ND; ++d) va[d] = ol.v_frag(Vt, j, half, d);
#pragma unroll
          for (int d = 0; d < ND; ++d)
            st.acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[d], pb[half], st.acc[d], 0, 0, 0);
        }
      });
      st.l += lsum0 + lsum1;
    };
    for (int t = 0; t < n_tiles; t += 2) {
      tile(t, std::integral_constant<int, 0>{});
      if (t + 1 < n_tiles) tile(t + 1, std::integral_constant<int, 1>{});
    }

    wait_vm();  // no tile load may still be in flight when the merge buffers are used
    __syncthreads();
    if (!full) {
      while (cur_chunk < a.c1) flush_chunk(cur_chunk++, (float*)sK0, (float*)sV0);
    } else {
      const int ln = opaque(lane), h2 = ln >> 5;
      float m, l_row;
      merge_halves<D, BLK>(st, m, l_row, (float*)sK0, (float*)sV0, rg, kh, ln);
      const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
      if (kh == 0 && qrow < a.S) {
        bf16* op = (bf16*)a.o + bh_base + (int64_t)qrow * a.ss;
#pragma unroll
        for (int d = 0; d < ND; ++d)
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

// Probabilities of one 32-key block that wait for their P V product, with the
// reference they were taken against.
struct PBlock {
  bf16x8 p[2];  // B operands of O^T += V^T P^T: keys 16*half + 8*h2 + 0..7
  float ref;    // reference subtracted in the exponent (log2 units)
  float lsum;   // this lane's share of the block's row sum of the rounded P
};

// Token-level causality on one wave's 32-key block: drops score r (key
// offset 16*(r/8) + 8*h2 + r%8 within the block, in steps of kstep token
// positions from the block's first key kpos) when its key lies after the
// lane's query qpos.
__device__ __forceinline__ void drop_future(f32x16& s, int qpos, int kpos, int kstep, int h2) {
  const int rel = qpos - kpos - kstep * 8 * h2;
  const int off_max = rel < 0 ? -1 : rel / kstep;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (16 * (r >> 3) + (r & 7) > off_max) s[r] = kNegInf;
}

// Full-tile kernel for 128-key blocks (S a multiple of the block, no
// token-level causality), software-pipelined per 32-key block.  The
// wave's work is a stream of blocks b (two per tile): the S MFMAs of block
// b+2 and the P V MFMAs of block b issue while the vector units take block
// b+1's row max and exponentials, so neither waits for the other.  The
// reference max therefore moves per block, one block ahead of the P V product
// that consumes it; before block b's P V the accumulators are brought to
// block b's reference (a rescale only when some row's reference moved, which
// the lazy rule makes rare).  MFMA operands are read from LDS a few MFMAs
// ahead of their use, one MFMA slot at a time.  STRIPED: chunks of the
// striped layout, where a tile's 32-key groups come from different KV blocks
// and a dead group's block takes no part (its row max is -inf and its
// probabilities are 0; its MFMAs still run).  TCAUSAL: token-level causality;
// a block whose last key lies after the wave's first query drops the scores
// of keys after each lane's query before its row max (a uniform branch, taken
// on diagonal tiles only), and rows that have no key yet keep an empty state.
template <int D, bool STRIPED, bool TCAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_pipe_kernel(FwdArgs a) {
  constexpr int BLK = 128;
  using SH = Shape<D, BLK>;
  constexpr int NB = SH::NKBW, ND = SH::ND, NKS = SH::NKS, NRG = SH::NRG;
  static_assert(NB == 2, "two 32-key blocks per wave and tile");
  static_assert(SH::NW * 64 == 512, "launch bounds");
  static_assert(SH::TILE * 2 >= NRG * SH::RB * 4096, "merge round must fit in a K buffer");
  static_assert(SH::TILE * 2 >= NRG * 96 * 4, "merge statistics must fit in a V buffer");
  constexpr int NOPS = NKS + 2 * ND;  // MFMAs of one section: S of one block and P V of one block
  static_assert(NKS == 2 * ND, "a section alternates S and P V MFMAs one for one");
  constexpr int AHEAD = 4;            // operands read this many MFMAs ahead
  constexpr int LPS = SH::IPW;        // tile-load instructions per section (K and V slices)
  __shared__ __attribute__((aligned(1024))) bf16 sK0[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[SH::TILE];
  __shared__ int sList[kMaxTilesPerRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % NRG, kh = wave / NRG;
  const int kb0 = kh * NB;
  const bool full = a.o != nullptr;
  constexpr int LAYOUT = STRIPED ? SA_LAYOUT_STRIPED : SA_LAYOUT_CONTIGUOUS;
  const int kb_div = SH::NKB / a.n_chunks;  // striped: 32-key blocks per liveness group
  TileLoader<D, BLK> loader;
  loader.init(wave, lane);
  loader.set_stride(STRIPED ? (int)(a.ss * a.n_chunks) : (int)a.ss);
  OperandLanes<D, true> ol;
  ol.init(lane, kb0);
  const bf16* __restrict__ gQ = (const bf16*)a.q;
  const bf16* __restrict__ gK = (const bf16*)a.k;
  const bf16* __restrict__ gV = (const bf16*)a.v;
  const int bin = blockIdx.x;
  const float sl2 = a.scale_log2;   // > 0
  const float inv_sl2 = 1.f / sl2;
  // the workgroup's items: its bin's list, or positions taken from the run-time queue
  const bool dyn = a.dyn_items != nullptr;
  __shared__ int sQueuePos;
  int pos = 0, p_end = 0, next_pos = 0;
  if (dyn) {
    p_end = a.bin_ptr[a.num_bins];
    if (tid == 0) sQueuePos = queue_take(a.dyn_ctr, p_end);
    __syncthreads();
    pos = __builtin_amdgcn_readfirstlane(sQueuePos);
  } else {
    pos = a.bin_ptr[bin];
    p_end = a.bin_ptr[bin + 1];
  }

  while (pos < p_end) {
    const int64_t t_start = realtime_now();
    const int item = dyn ? a.dyn_items[pos] : a.items[pos];
    const int qb = item % a.nQ;
    const int bh = item / a.nQ;
    const int b = bh / a.H, h = bh % a.H;
    const int64_t bh_base = (int64_t)b * a.sb + (int64_t)h * a.sh;
    const int qrow = qb * BLK + rg * 32 + (lane & 31);

    bf16x8 qf[NKS];
    {
      const bf16* qp = gQ + bh_base + (int64_t)qrow * a.ss + 8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    }

    __syncthreads();  // every wave is done with the previous item's list, tiles and merge buffers
    const int n_tiles = build_tile_list(a.mask + (int64_t)item * a.nK, a.nK, a.n_chunks, LAYOUT, a.c0, a.c1, sList,
                                        wave == 0);
    __syncthreads();

    RowState<ND> st;  // acc and l relative to st.m_ref (the reference of the last consumed block)
    reset(st);
    int cur_chunk = a.c0;
    bool acc_live = false;  // the accumulation in progress has taken a tile (uniform)
    // Row maxima are kept per lane, over the lane's own keys and in raw score units (the
    // scale is positive): lmax for the accumulation in progress, lmax_next for one that starts
    // with the next tile (partial mode).  The wave's row max (both half-waves) is formed when
    // a reference may move and when the key halves are merged (st.m_true).
    float lmax = kNegInf, lmax_next = kNegInf;
    auto true_max = [&]() { st.m_true = fmaxf(lmax, other_half(lmax)) * sl2; };

    // Same flush as the general kernel: merge the key halves, write chunk
    // `chunk`'s partial through the staging buffers, reset the state.
    auto flush_partial = [&](int chunk, float* kscr, float* mscr) {
      constexpr int CH = D / 4;
      constexpr int HALF = BLK / 2;
      constexpr int RPS = 64 / CH;
      constexpr int NST = BLK / SH::NW / RPS;
      static_assert(HALF * D * 4 <= SH::TILE * 2, "staging half must fit in a tile buffer");
      static_assert(NST * RPS * SH::NW == BLK, "store rows must cover the block");
      // lane-derived addresses are formed here, not kept live across the tile loop
      const int ln = opaque(lane), l32 = ln & 31, h2 = ln >> 5;
      float m, l_row;
      true_max();
      merge_halves<D, BLK>(st, m, l_row, kscr, mscr, rg, kh, ln);
      const int64_t prow0 = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + (int64_t)qb * BLK;
      if (kh == 0) {
        const int r = rg * 32 + l32;
        float* const rowp = (rg * 32 < HALF ? kscr : mscr) + (r % HALF) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = 8 * d + 2 * g + h2;
            const f32x4 v4 = {st.acc[d][4 * g], st.acc[d][4 * g + 1], st.acc[d][4 * g + 2], st.acc[d][4 * g + 3]};
            *(f32x4*)(rowp + 4 * (c ^ (r & (CH - 1)))) = v4;
          }
        if (h2 == 0) {
          a.m_part[prow0 + r] = m == kNegInf ? kNegInf : m * kLn2;
          a.l_part[prow0 + r] = l_row;
        }
      }
      __syncthreads();
      {
        const float* const buf = (wave * NST * RPS < HALF ? kscr : mscr);
        const int c = ln % CH;
#pragma unroll 1
        for (int i = 0; i < NST; ++i) {
          const int r = (wave * NST + i) * RPS + ln / CH;
          const f32x4 v4 = *(const f32x4*)(buf + (r % HALF) * D + 4 * (c ^ (r & (CH - 1))));
          *(f32x4*)(a.o_part + (prow0 + r) * D + 4 * c) = v4;
        }
      }
      __syncthreads();
      reset(st);
      lmax = kNegInf;
    };
    // An empty accumulation's partial, (0, -inf, 0), is written by every wave for its own
    // rows, with no merge of the key halves and no staging (nor their barriers).
    auto flush_empty = [&](int chunk) {
      constexpr int RPW = BLK / SH::NW;  // rows per wave
      const int ln = opaque(lane);
      const int64_t prow0 = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + (int64_t)qb * BLK;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      static_assert(RPW * (D / 4) % 64 == 0, "the wave's rows split evenly over its lanes");
#pragma unroll
      for (int k = 0; k < RPW * (D / 4) / 64; ++k) {
        const int idx = ln + 64 * k;
        const int r = wave * RPW + idx / (D / 4), c = idx % (D / 4);
        *(f32x4*)(a.o_part + (prow0 + r) * D + 4 * c) = z;
      }
      if (ln < RPW) {
        a.m_part[prow0 + wave * RPW + ln] = kNegInf;
        a.l_part[prow0 + wave * RPW + ln] = 0.f;
      }
      lmax = kNegInf;
    };
    auto flush_chunk = [&](int chunk, float* kscr, float* mscr) {
      if (acc_live)
        flush_partial(chunk, kscr, mscr);
      else
        flush_empty(chunk);
      acc_live = false;
    };
    auto src_of = [&](int desc) { return tile_source(desc, bh_base, a.ss, a.S, LAYOUT, a.n_chunks, BLK); };
    auto chunk_of = [&](int desc) { return (desc >> kDescChunkShift) & 63; };
    // key block j of this wave in the tile of `desc` has no live key (striped layout only)
    auto dead_of = [&](int desc, int j) {
      return STRIPED && !((desc >> (kDescCodeShift + (kb0 + j) / kb_div)) & 1);
    };
    // token position of the first key of this wave's block j of the tile of `desc`, and the
    // step between the wave's keys (striped chunk c's compacted position p is token c + C p)
    const int kstep = STRIPED ? a.n_chunks : 1;
    auto kpos_of = [&](int desc, int j) {
      const int key = (desc & 0xFFFFF) * BLK + (kb0 + j) * 32;
      return STRIPED ? ((desc >> kDescChunkShift) & 63) + a.n_chunks * key : key;
    };
    // block j of the tile of `desc` has a key after the wave's first query
    auto diag_of = [&](int desc, int j) {
      return TCAUSAL && kpos_of(desc, j) + kstep * 31 > qb * BLK + rg * 32;
    };

    f32x16 sc[NB];       // scores of the two blocks of the next tile to be exponentiated
    PBlock pb[NB];       // probabilities waiting for their P V product
    uint64_t moved[NB];  // rows whose reference moved with that block
    float ref_cur = kNegInf;  // reference of the latest block exponentiated (log2 units)
    float thr = kNegInf;      // raw score above which that reference moves: (ref_cur + slack) / scale
    // A row's reference moves when its running max (both half-waves) exceeds thr: the lanes
    // compare their own maxima, and only a ballot with a lane above thr forms the row maxima.
    // A block's PBlock::ref is written only then (it is read only for a block whose ballot
    // of moved rows is not empty).
    auto move_ref = [&](float mx, float& ref, float& th, float& pref) {
      uint64_t mv = 0;
      if (__builtin_amdgcn_ballot_w64(mx > th)) {
        const float rm = fmaxf(mx, other_half(mx));
        const bool up = rm > th;
        ref = up ? rm * sl2 : ref;
        th = up ? (ref + kRescaleSlack) * inv_sl2 : th;
        pref = ref;
        mv = __builtin_amdgcn_ballot_w64(up);
      }
      return mv;
    };
    if (n_tiles > 0) {
      const int d0 = __builtin_amdgcn_readfirstlane(sList[0]);
      loader.template issue<false>(gK, src_of(d0), sK0, wave);
      loader.template issue<false>(gV, src_of(d0), sV0, wave);
      if (n_tiles > 1) loader.template issue<false>(gK, src_of(__builtin_amdgcn_readfirstlane(sList[1])), sK1, wave);
      wait_vm();
      __syncthreads();
      tile_scores<D, BLK, false>(sK0, qf, ol, 0, sc);
      // block 0 starts an accumulation: its running max goes to lmax_next, which
      // the first tile takes over (after flushing any empty leading chunks)
      if (diag_of(d0, 0)) drop_future(sc[0], qrow, kpos_of(d0, 0), kstep, lane >> 5);
      const bool dead = dead_of(d0, 0);
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
      lmax_next = dead ? kNegInf : mx;
      moved[0] = move_ref(lmax_next, ref_cur, thr, pb[0].ref);
      float l0 = 0.f, l1 = 0.f;
      tile_probs(sc[0], sl2, dead ? __builtin_huge_valf() : (ref_cur == kNegInf ? 0.f : ref_cur), pb[0].p, l0, l1);
      pb[0].lsum = l0 + l1;
    }

    // Brings the accumulators and row sum to the reference of block pb, then
    // adds the block's row sum (its P V follows).
    auto consume = [&](const PBlock& p, uint64_t mv) {
      if (mv) {
        // (rows that are still empty on both sides keep factor 1)
        const float alpha = (TCAUSAL && st.m_ref == p.ref) ? 1.f : __builtin_amdgcn_exp2f(st.m_ref - p.ref);
        st.l *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d) st.acc[d] *= alpha;
        st.m_ref = p.ref;  // (changes only with a moved reference)
      }
      st.l += p.lsum;
    };

    auto tile = [&](int t, auto parity) {
      constexpr int P = decltype(parity)::value;
      bf16* const kfree = P ? sK1 : sK0;
      bf16* const vfree = P ? sV0 : sV1;
      const bf16* const Kt1 = P ? sK0 : sK1;
      const bf16* const Vt = P ? sV1 : sV0;
      const int desc = __builtin_amdgcn_readfirstlane(sList[t]);
      const bool has_next = t + 1 < n_tiles;
      const int desc1 = has_next ? __builtin_amdgcn_readfirstlane(sList[t + 1]) : desc;
      // the next tile starts a new accumulation (a chunk of its own in partial mode)
      const bool next_new = !full && has_next && chunk_of(desc1) != chunk_of(desc);
      const bool dead_sec[NB] = {dead_of(desc, 1), dead_of(desc1, 0)};  // blocks exponentiated in sections 0, 1
      const bool diag_sec[NB] = {diag_of(desc, 1), diag_of(desc1, 0)};
      const int kpos_sec[NB] = {kpos_of(desc, 1), kpos_of(desc1, 0)};

      wait_vm();
      __syncthreads();
      // (thread 0) the position of the workgroup's next item, taken from the run-time queue
      // here, right after a wait for every load in flight: the next such wait is a tile away
      if (dyn && t == 0 && tid == 0) next_pos = queue_take(a.dyn_ctr, p_end);
      bool fresh = t == 0;  // block 0 of this tile opens an accumulation
      if (!full && cur_chunk < chunk_of(desc)) {
        while (cur_chunk < chunk_of(desc)) flush_chunk(cur_chunk++, (float*)kfree, (float*)vfree);
        fresh = true;
      }
      if (fresh) lmax = lmax_next;
      acc_live = true;  // this tile belongs to the accumulation in progress
      const TileSrc srcK = src_of(__builtin_amdgcn_readfirstlane(sList[min(t + 2, n_tiles - 1)]));
      const TileSrc srcV = src_of(desc1);

      // The tile's MFMA stream: section j = S of block j of tile t+1 (NKS MFMAs, K
      // fragments), then P V of block j of tile t (2*ND MFMAs, V^T fragments).
      bf16x8 fr[2 * NOPS];
      auto rd = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int j = i / NOPS, k = i % NOPS;
        if constexpr (k < NKS)
          fr[i] = ol.k_frag(Kt1, j, k);
        else
          fr[i] = ol.v_frag(Vt, j, (k - NKS) / ND, (k - NKS) % ND);
      };
      auto mm = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int j = i / NOPS, k = i % NOPS;
        if constexpr (k < NKS) {
          sc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], qf[k], k == 0 ? f32x16{} : sc[j], 0, 0, 0);
        } else {
          constexpr int half = (k - NKS) / ND, d = (k - NKS) % ND;
          st.acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], pb[j].p[half], st.acc[d], 0, 0, 0);
        }
      };
      // slot q of a section runs op ord(q): all S MFMAs, then all P V MFMAs (alternating
      // them, as the pair kernel does, measured 1% slower here)
      auto ord = [](int q) constexpr { return q; };
      static_for<AHEAD>([&](auto ic) { rd(std::integral_constant<int, ord(decltype(ic)::value)>{}); });

      static_for<NB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        consume(pb[j], moved[j]);
        // vector work of this section, in stages: block 1 of tile t (section 0), or
        // block 0 of tile t+1 (section 1, on the scores of section 0's S MFMAs)
        constexpr int SRC = j == 0 ? 1 : 0;
        const f32x16& s = sc[SRC];
        PBlock& out = pb[SRC];
        float mx_a, mx_b, mx, seed, ref_exp, l0, l1;
        uint64_t mv;
        constexpr bool NEXT = j == 1;  // block 0 of the next tile
        const bool dead = STRIPED && dead_sec[j];  // uniform
        auto stage = [&](auto sc_) {
          constexpr int g = decltype(sc_)::value;
          if constexpr (g == 0) {
            if constexpr (TCAUSAL)
              if (diag_sec[j]) drop_future(sc[SRC], qrow, kpos_sec[j], kstep, lane >> 5);
            // the running max this block folds into (a new accumulation starts empty)
            seed = (NEXT && next_new) ? kNegInf : lmax;
            mx_a = fmaxf(fmaxf(seed, s[0]), s[1]);
            mx_a = fmaxf(fmaxf(mx_a, s[2]), s[3]);
            mx_a = fmaxf(fmaxf(mx_a, s[4]), s[5]);
          } else if constexpr (g == 1) {
            mx_b = fmaxf(fmaxf(s[6], s[7]), s[8]);
            mx_b = fmaxf(fmaxf(mx_b, s[9]), s[10]);
            mx_b = fmaxf(fmaxf(mx_b, s[11]), s[12]);
            mx_b = fmaxf(fmaxf(mx_b, s[13]), s[14]);
            mx = fmaxf(fmaxf(mx_a, mx_b), s[15]);
          } else if constexpr (g == 2) {
            mx = dead ? seed : mx;  // a dead block has no live key
            if constexpr (NEXT) {
              ref_cur = next_new ? kNegInf : ref_cur;
              thr = next_new ? kNegInf : thr;
            }
            mv = move_ref(mx, ref_cur, thr, out.ref);
          } else if constexpr (g == 3) {
            // reference of the exponent: +inf makes a dead block's probabilities 0
            ref_exp = dead ? __builtin_huge_valf() : (TCAUSAL && ref_cur == kNegInf) ? 0.f : ref_cur;
            moved[SRC] = mv;
            if constexpr (!NEXT) {
              lmax = mx;
            } else {
              lmax_next = mx;
              lmax = (has_next && !next_new) ? mx : lmax;
            }
            l0 = 0.f;
            l1 = 0.f;
          } else if constexpr (g < 12) {
            constexpr int r = 2 * (g - 4);
            out.p[r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[r], sl2, -ref_exp));
            out.p[r >> 3][(r & 7) + 1] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -ref_exp));
          } else {
            constexpr int h = g - 12;
            const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
            float& acc_l = h ? l1 : l0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc_l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{out.p[h][2 * e], out.p[h][2 * e + 1]}, ones, acc_l, false);
            if constexpr (h == 1) out.lsum = l0 + l1;
          }
        };
        constexpr int NSTAGE = 14;
        constexpr int SPS = (NSTAGE + NOPS - 1) / NOPS;  // stages per MFMA slot
        static_for<NOPS>([&](auto kc) {
          constexpr int k = decltype(kc)::value, q = j * NOPS + k;
          if constexpr (q + AHEAD < 2 * NOPS) rd(std::integral_constant<int, ord(q + AHEAD)>{});
          mm(std::integral_constant<int, ord(q)>{});
          static_for<SPS>([&](auto uc) {
            constexpr int g = k * SPS + decltype(uc)::value;
            if constexpr (g < NSTAGE) stage(std::integral_constant<int, g>{});
          });
          if constexpr (k < LPS / 2) {
            loader.template issue<false, j * LPS / 2 + k, j * LPS / 2 + k + 1>(gK, srcK, kfree, wave);
            loader.template issue<false, j * LPS / 2 + k, j * LPS / 2 + k + 1>(gV, srcV, vfree, wave);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        // keep the section's vector results in this section (they are consumed one
        // section later)
        asm volatile("" : "+v"(out.p[0]), "+v"(out.p[1]), "+v"(out.lsum), "+v"(out.ref), "+v"(ref_cur));
      });
    };
    for (int t = 0; t < n_tiles; t += 2) {
      tile(t, std::integral_constant<int, 0>{});
      if (t + 1 < n_tiles) tile(t + 1, std::integral_constant<int, 1>{});
    }

    wait_vm();
    __syncthreads();
    if (!full) {
      while (cur_chunk < a.c1) flush_chunk(cur_chunk++, (float*)sK0, (float*)sV0);
    } else {
      const int ln = opaque(lane), h2 = ln >> 5;
      float m, l_row;
      true_max();
      merge_halves<D, BLK>(st, m, l_row, (float*)sK0, (float*)sV0, rg, kh, ln);
      const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
      if (kh == 0) {
        bf16* op = (bf16*)a.o + bh_base + (int64_t)qrow * a.ss;
#pragma unroll
        for (int d = 0; d < ND; ++d)
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
    if (dyn) {
      if (tid == 0) {
        if (n_tiles == 0) next_pos = queue_take(a.dyn_ctr, p_end);  // (else taken during the first tile)
        sQueuePos = next_pos;
      }
      __syncthreads();  // (every wave read the previous position before this item's barriers)
      pos = __builtin_amdgcn_readfirstlane(sQueuePos);
    } else {
      ++pos;
    }
  }
  if (dyn && tid == 0) queue_finish(a.dyn_ctr);
}

// Q-block pairs (S a multiple of 128): an item is the two Q-blocks 2p and 2p+1
// of one (batch, head), 256 query rows, so each K/V tile staged in LDS feeds
// twice the queries of a single-block item.  Wave w owns the 32 rows 32*(w%4)
// of Q-block 2p + w/4 and all four 32-key blocks of every tile, so no key
// halves are merged.  The tile list is the union of both mask rows; a 32-key
// block that has no live key for a Q-block (a tile live for the other row only,
// or, STRIPED, a dead group of a striped chunk's tile) is a dead block for that
// Q-block's waves (its probabilities are 0; its MFMAs still run).
//
// Each wave's block stream has four blocks per tile, pipelined as in the
// single-block kernel: the S MFMAs of block b+2 and the P V MFMAs of block b
// issue while the vector units take block b+1's softmax.  A tile is worked in
// two halves with a workgroup barrier before each.  The first half (P V of
// blocks 0-1) takes the S of blocks 2-3 from this tile's K and loads the next
// tile's V into the V buffer the previous tile used; the second half (P V of
// blocks 2-3) takes the S of the next tile's blocks 0-1 from the next K and
// loads K of the tile after next into this tile's K buffer, which the first
// half was the last to read.  TCAUSAL: token-level causality as in the
// single-block kernel.
template <int D, bool STRIPED, bool TCAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_pair_kernel(FwdArgs a) {
  constexpr int BLK = 128;
  using SH = Shape<D, BLK>;
  constexpr int ND = SH::ND, NKS = SH::NKS;
  static_assert(SH::NW * 64 == 512, "launch bounds");
  constexpr int NOPS = NKS + 2 * ND;  // MFMAs of one section: S of one block and P V of one block
  static_assert(NKS == 2 * ND, "a section alternates S and P V MFMAs one for one");
  constexpr int AHEAD = 6;            // operands read this many MFMAs ahead (4 measured 1% slower)
  constexpr int LPS = SH::IPW;        // load instructions of one K or V tile per wave
  static_assert(LPS % 2 == 0 && LPS / 2 <= NOPS, "a half-tile's loads spread over its two sections");
  __shared__ __attribute__((aligned(1024))) bf16 sK0[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[SH::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[SH::TILE];
  __shared__ int sList[kMaxTilesPerRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, rg = wave & 3;  // Q-block of the pair, row group within it
  const bool full = a.o != nullptr;
  constexpr int LAYOUT = STRIPED ? SA_LAYOUT_STRIPED : SA_LAYOUT_CONTIGUOUS;
  // 32-key blocks per liveness group: one group per striped chunk's slice of a KV block, one
  // per tile for contiguous chunks (whose code bits are all set together)
  const int kb_div = STRIPED ? SH::NKB / a.n_chunks : SH::NKB;
  const int kstep = STRIPED ? a.n_chunks : 1;  // token distance of consecutive keys of a tile
  TileLoader<D, BLK> loader;
  loader.init(wave, lane);
  loader.set_stride(STRIPED ? (int)(a.ss * a.n_chunks) : (int)a.ss);
  OperandLanes<D, true> ol;
  ol.init(lane, 0);
  const bf16* __restrict__ gQ = (const bf16*)a.q;
  const bf16* __restrict__ gK = (const bf16*)a.k;
  const bf16* __restrict__ gV = (const bf16*)a.v;
  const int bin = blockIdx.x;
  const float sl2 = a.scale_log2;   // > 0
  const float inv_sl2 = 1.f / sl2;
  // the workgroup's items: its bin's list, or positions taken from the run-time queue
  const bool dyn = a.dyn_items != nullptr;
  __shared__ int sQueuePos;
  int pos = 0, p_end = 0, next_pos = 0;
  if (dyn) {
    p_end = a.bin_ptr[a.num_bins];
    if (tid == 0) sQueuePos = queue_take(a.dyn_ctr, p_end);
    __syncthreads();
    pos = __builtin_amdgcn_readfirstlane(sQueuePos);
  } else {
    pos = a.bin_ptr[bin];
    p_end = a.bin_ptr[bin + 1];
  }

  while (pos < p_end) {
    const int64_t t_start = realtime_now();
    const int item = dyn ? a.dyn_items[pos] : a.items[pos];
    const int pr = item % a.nI;
    const int bh = item / a.nI;
    const int b = bh / a.H, h = bh % a.H;
    const int64_t bh_base = (int64_t)b * a.sb + (int64_t)h * a.sh;
    const int qa = 2 * pr;              // first Q-block of the pair
    const int qb = qa + half;           // this wave's Q-block
    const bool absent = qb >= a.nQ;     // second half of the last pair of an odd nQ: computes, never stores
    const int qrow = qb * BLK + rg * 32 + (lane & 31);

    bf16x8 qf[NKS];
    {
      const bf16* qp = gQ + bh_base + (int64_t)(absent ? qrow - BLK : qrow) * a.ss + 8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    }

    __syncthreads();  // every wave is done with the previous item's list and tiles
    const int n_tiles = build_pair_tile_list(a.mask + ((int64_t)bh * a.nQ + qa) * a.nK, qa + 1 < a.nQ, a.nK,
                                             a.n_chunks, LAYOUT, a.c0, a.c1, sList, wave == 0);
    __syncthreads();

    RowState<ND> st;  // acc and l relative to st.m_ref (the reference of the last consumed block)
    reset(st);
    int cur_chunk = a.c0;
    // Row maxima are kept per lane, over the lane's own keys and in raw score units (the
    // scale is positive): lmax for the accumulation in progress, lmax_next for one that starts
    // with the next tile (partial mode).  A row's true max (both half-waves) is formed only
    // where it is needed: when a reference may move, and when a partial is written.
    float lmax = kNegInf, lmax_next = kNegInf;

    // Writes chunk `chunk`'s partial of this wave's rows (O unnormalised, m, l in the
    // true-max basis) and resets the state.  D = 128: the O rows go through `stage`, a
    // 4 KiB LDS region of this wave alone (its own slice of a tile buffer that no wave
    // reads meanwhile), one head-dim block at a time, so that every store instruction
    // writes eight whole 128-byte row segments; otherwise straight from the registers.
    auto flush_partial = [&](int chunk, float* stage) {
      const int ln = opaque(lane), l32 = ln & 31, h2 = ln >> 5;
      const float m_true = fmaxf(lmax, other_half(lmax)) * sl2;  // the row's true max, log2 units
      const bool any = m_true != kNegInf;
      const float corr = any ? __builtin_amdgcn_exp2f(st.m_ref - m_true) : 0.f;
      const float l_row = (st.l + other_half(st.l)) * corr;
      if (!absent) {
        const int64_t prow0 = ((int64_t)(chunk - a.c0) * a.B * a.H + bh) * a.S + (int64_t)qb * BLK + rg * 32;
        if (D == 128 && !__builtin_amdgcn_ballot_w64(any)) {
          // no row of the wave has a key in this chunk: zeros, row segments written whole
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              *(f32x4*)(a.o_part + (prow0 + 8 * i + (ln >> 3)) * D + d * 32 + 4 * (ln & 7)) = z;
        } else if constexpr (D == 128) {
          // stage layout: row r (32 floats) at 32 r, its 16-byte chunk c at physical chunk
          // c ^ ((r >> 1) & 7), so that both the column-wise writes and the row-wise reads
          // touch 16 different chunks of 16 bytes per 256 bytes
#pragma unroll
          for (int d = 0; d < ND; ++d) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v4 = {st.acc[d][4 * g] * corr, st.acc[d][4 * g + 1] * corr,
                                st.acc[d][4 * g + 2] * corr, st.acc[d][4 * g + 3] * corr};
              *(f32x4*)(stage + l32 * 32 + 4 * ((2 * g + h2) ^ ((l32 >> 1) & 7))) = v4;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 8 * i + (ln >> 3), c = ln & 7;
              const f32x4 v4 = *(const f32x4*)(stage + r * 32 + 4 * (c ^ ((r >> 1) & 7)));
              *(f32x4*)(a.o_part + (prow0 + r) * D + d * 32 + 4 * c) = v4;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          }
        } else {
          float* const op = a.o_part + (prow0 + l32) * D + 4 * h2;
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v4 = {st.acc[d][4 * g] * corr, st.acc[d][4 * g + 1] * corr,
                                st.acc[d][4 * g + 2] * corr, st.acc[d][4 * g + 3] * corr};
              *(f32x4*)(op + d * 32 + 8 * g) = v4;
            }
        }
        if (h2 == 0) {
          a.m_part[prow0 + l32] = any ? m_true * kLn2 : kNegInf;
          a.l_part[prow0 + l32] = l_row;
        }
      }
      reset(st);
      lmax = kNegInf;
    };
    // this wave's slice of a tile buffer (the slots its own tile loads write), as staging
    auto stage_of = [&](bf16* buf) { return (float*)(buf + wave * SH::IPW * 64 * 8); };
    auto src_of = [&](int desc) {  // (the group codes cleared, the tile index and chunk kept)
      return tile_source(desc & ~(0xFF << kPairCodeShift), bh_base, a.ss, a.S, LAYOUT, a.n_chunks, BLK);
    };
    auto chunk_of = [&](int desc) { return (desc >> kDescChunkShift) & 63; };
    // 32-key block j of the tile of `desc` has no live key for this wave's Q-block
    auto dead_of = [&](int desc, int j) { return !((desc >> (kPairCodeShift + 4 * half + j / kb_div)) & 1); };
    // token position of the first key of block j of the tile of `desc` (striped chunk c's
    // compacted position p is token c + C p)
    auto kpos_of = [&](int desc, int j) {
      const int key = (desc & kPairTileMask) * BLK + j * 32;
      return STRIPED ? chunk_of(desc) + a.n_chunks * key : key;
    };
    // key block j of the tile of `desc` has a key after the wave's first query
    auto diag_of = [&](int desc, int j) {
      return TCAUSAL && kpos_of(desc, j) + kstep * 31 > qb * BLK + rg * 32;
    };

    f32x16 sc[2];        // scores of the next two blocks of the stream (by block parity)
    PBlock pb[2];        // probabilities waiting for their P V product (by block parity)
    uint64_t moved[2];   // rows whose reference moved with that block
    float ref_cur = kNegInf;  // reference of the latest block exponentiated (log2 units)
    float thr = kNegInf;      // raw score above which that reference moves: (ref_cur + slack) / scale
    // A row's reference moves when its running max (both half-waves) exceeds thr: the lanes
    // compare their own maxima, and only a ballot with a lane above thr forms the row maxima.
    // A block's PBlock::ref is written only then (it is read only for a block whose ballot
    // of moved rows is not empty).
    auto move_ref = [&](float mx, float& ref, float& th, float& pref) {
      uint64_t mv = 0;
      if (__builtin_amdgcn_ballot_w64(mx > th)) {
        const float rm = fmaxf(mx, other_half(mx));
        const bool up = rm > th;
        ref = up ? rm * sl2 : ref;
        th = up ? (ref + kRescaleSlack) * inv_sl2 : th;
        pref = ref;
        mv = __builtin_amdgcn_ballot_w64(up);
      }
      return mv;
    };
    if (n_tiles > 0) {
      const int d0 = __builtin_amdgcn_readfirstlane(sList[0]);
      loader.template issue<false>(gK, src_of(d0), sK0, wave);
      loader.template issue<false>(gV, src_of(d0), sV0, wave);
      if (n_tiles > 1) loader.template issue<false>(gK, src_of(__builtin_amdgcn_readfirstlane(sList[1])), sK1, wave);
      wait_vm();
      __syncthreads();
      tile_scores<D, BLK, false>(sK0, qf, ol, 0, sc);  // blocks 0 and 1 of tile 0
      if (diag_of(d0, 0)) drop_future(sc[0], qrow, kpos_of(d0, 0), kstep, lane >> 5);
      const bool dead = dead_of(d0, 0);
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
      lmax_next = dead ? kNegInf : mx;
      moved[0] = move_ref(lmax_next, ref_cur, thr, pb[0].ref);
      float l0 = 0.f, l1 = 0.f;
      tile_probs(sc[0], sl2, dead ? __builtin_huge_valf() : (ref_cur == kNegInf ? 0.f : ref_cur), pb[0].p, l0, l1);
      pb[0].lsum = l0 + l1;
    }

    // Adds block p to the state; st.m_ref changes only with a moved reference.
    auto consume = [&](const PBlock& p, uint64_t mv) {
      if (mv) {
        const float alpha = (TCAUSAL && st.m_ref == p.ref) ? 1.f : __builtin_amdgcn_exp2f(st.m_ref - p.ref);
        st.l *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d) st.acc[d] *= alpha;
        st.m_ref = p.ref;
      }
      st.l += p.lsum;
    };

    // Half H of tile t (parity P = t % 2): sections j = 2H, 2H+1 of the tile.
    // MFMA operands in flight; the first half of a tile also reads the second half's first
    // operands (K of the next tile and V of this one, both complete since the first half's wait)
    bf16x8 fr[2 * NOPS];
    auto halftile = [&](int t, auto parity, auto hc) {
      constexpr int P = decltype(parity)::value;
      constexpr int H = decltype(hc)::value;
      const bf16* const Kt = P ? sK1 : sK0;  // K of tile t
      const bf16* const Kn = P ? sK0 : sK1;  // K of tile t+1
      const bf16* const Vt = P ? sV1 : sV0;  // V of tile t
      bf16* const lfree = H == 0 ? (P ? sV0 : sV1) : (P ? sK1 : sK0);  // V of t+1, or K of t+2
      const int desc = __builtin_amdgcn_readfirstlane(sList[t]);
      const bool has_next = t + 1 < n_tiles;
      const int desc1 = has_next ? __builtin_amdgcn_readfirstlane(sList[t + 1]) : desc;
      // the next tile starts a new accumulation (a chunk of its own in partial mode)
      const bool next_new = !full && has_next && chunk_of(desc1) != chunk_of(desc);

      // The first half reads V of this tile, loaded during the previous tile's first half:
      // wait for this wave's loads, then the barrier makes every wave's visible (and frees the
      // V buffer of the previous tile).  The second half reads only data that the first
      // half's wait covered (K of the next tile, V of this one); its barrier just frees this
      // tile's K buffer, whose reads the first half's MFMAs have consumed, so it waits for no
      // memory operation and the loads and partial stores issued meanwhile keep draining
      // (waiting for the stores of a chunk flush here took 1.6% of the partial forward).
      if constexpr (H == 0) {
        wait_vm();
        __syncthreads();
        // (thread 0) the position of the workgroup's next item, taken from the run-time queue
        // here, right after a wait for every load in flight: the next such wait is a tile away
        if (dyn && t == 0 && tid == 0) next_pos = queue_take(a.dyn_ctr, p_end);
      } else {
        barrier_only();
      }
      if constexpr (H == 0) {
        bool fresh = t == 0;  // block 0 of this tile opens an accumulation
        if (!full && cur_chunk < chunk_of(desc)) {
          // the V buffer of the previous tile is free until this half's loads go out
          while (cur_chunk < chunk_of(desc)) flush_partial(cur_chunk++, stage_of(lfree));
          fresh = true;
        }
        if (fresh) lmax = lmax_next;
      }
      const TileSrc src = H == 0 ? src_of(desc1) : src_of(__builtin_amdgcn_readfirstlane(sList[min(t + 2, n_tiles - 1)]));
      const bf16* const gsrc = H == 0 ? gV : gK;

      // operand of op i of half HH of this tile
      auto rd = [&](auto hh, auto ic) {
        constexpr int HH = decltype(hh)::value;
        constexpr int i = decltype(ic)::value;
        constexpr int jj = i / NOPS, k = i % NOPS;
        if constexpr (k < NKS)
          fr[i] = ol.k_frag(HH == 0 ? Kt : Kn, HH == 0 ? jj + 2 : jj, k);
        else
          fr[i] = ol.v_frag(Vt, 2 * HH + jj, (k - NKS) / ND, (k - NKS) % ND);
      };
      auto mm = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int jj = i / NOPS, k = i % NOPS;
        if constexpr (k < NKS) {
          sc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], qf[k], k == 0 ? f32x16{} : sc[jj], 0, 0, 0);
        } else {
          constexpr int hf = (k - NKS) / ND, d = (k - NKS) % ND;
          st.acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], pb[jj].p[hf], st.acc[d], 0, 0, 0);
        }
      };
      // slot q of a section runs op ord(q): its S and P V MFMAs alternate, so that the
      // S chain (eight MFMAs into one accumulator) never has two links back to back
      auto ord = [](int q) constexpr {
        return (q / NOPS) * NOPS + ((q % NOPS) % 2 == 0 ? (q % NOPS) / 2 : NKS + (q % NOPS) / 2);
      };
      if constexpr (H == 0)
        static_for<AHEAD>([&](auto ic) {
          rd(std::integral_constant<int, 0>{}, std::integral_constant<int, ord(decltype(ic)::value)>{});
        });

      static_for<2>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        constexpr int j = 2 * H + jj;          // section of the tile: P V of block j
        constexpr bool NEXT = j == 3;          // its softmax is block 0 of the next tile
        consume(pb[jj], moved[jj]);
        constexpr int SRC = 1 - jj;            // parity of block j + 1
        const f32x16& s = sc[SRC];
        PBlock& out = pb[SRC];
        const int sdesc = NEXT ? desc1 : desc;
        constexpr int sblk = NEXT ? 0 : j + 1;
        const bool dead = dead_of(sdesc, sblk);  // uniform
        float mx_a, mx_b, mx, seed, ref_exp, lsum;
        uint64_t mv;
        auto stage = [&](auto sc_) {
          constexpr int g = decltype(sc_)::value;
          if constexpr (g == 0) {
            if constexpr (TCAUSAL)
              if (diag_of(sdesc, sblk)) drop_future(sc[SRC], qrow, kpos_of(sdesc, sblk), kstep, lane >> 5);
            // the running max this block folds into (a new accumulation starts empty)
            seed = (NEXT && next_new) ? kNegInf : lmax;
            mx_a = fmaxf(fmaxf(seed, s[0]), s[1]);
            mx_a = fmaxf(fmaxf(mx_a, s[2]), s[3]);
            mx_a = fmaxf(fmaxf(mx_a, s[4]), s[5]);
          } else if constexpr (g == 1) {
            mx_b = fmaxf(fmaxf(s[6], s[7]), s[8]);
            mx_b = fmaxf(fmaxf(mx_b, s[9]), s[10]);
            mx_b = fmaxf(fmaxf(mx_b, s[11]), s[12]);
            mx_b = fmaxf(fmaxf(mx_b, s[13]), s[14]);
            mx = fmaxf(fmaxf(mx_a, mx_b), s[15]);
          } else if constexpr (g == 2) {
            mx = dead ? seed : mx;  // a dead block has no live key
            if constexpr (NEXT) {
              ref_cur = next_new ? kNegInf : ref_cur;
              thr = next_new ? kNegInf : thr;
            }
            mv = move_ref(mx, ref_cur, thr, out.ref);
          } else if constexpr (g == 3) {
            // reference of the exponent: +inf makes a dead block's probabilities 0
            ref_exp = dead ? __builtin_huge_valf() : (TCAUSAL && ref_cur == kNegInf) ? 0.f : ref_cur;
            moved[SRC] = mv;
            if constexpr (!NEXT) {
              lmax = mx;
            } else {
              lmax_next = mx;
              lmax = (has_next && !next_new) ? mx : lmax;
            }
            lsum = 0.f;
          } else if constexpr (g < 12) {
            constexpr int r = 2 * (g - 4);
            out.p[r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[r], sl2, -ref_exp));
            out.p[r >> 3][(r & 7) + 1] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -ref_exp));
          } else {
            constexpr int hh = g - 12;
            const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{out.p[hh][2 * e], out.p[hh][2 * e + 1]}, ones, lsum, false);
            if constexpr (hh == 1) out.lsum = lsum;
          }
        };
        constexpr int NSTAGE = 14;
        constexpr int SPS = (NSTAGE + NOPS - 1) / NOPS;  // stages per MFMA slot
        static_for<NOPS>([&](auto kc) {
          constexpr int k = decltype(kc)::value, q = jj * NOPS + k;
          if constexpr (q + AHEAD < 2 * NOPS)
            rd(std::integral_constant<int, H>{}, std::integral_constant<int, ord(q + AHEAD)>{});
          else if constexpr (H == 0)
            rd(std::integral_constant<int, 1>{}, std::integral_constant<int, ord(q + AHEAD - 2 * NOPS)>{});
          mm(std::integral_constant<int, ord(q)>{});
          static_for<SPS>([&](auto uc) {
            constexpr int g = k * SPS + decltype(uc)::value;
            if constexpr (g < NSTAGE) stage(std::integral_constant<int, g>{});
          });
          if constexpr (k < LPS / 2)
            loader.template issue<false, jj * LPS / 2 + k, jj * LPS / 2 + k + 1>(gsrc, src, lfree, wave);
          __builtin_amdgcn_sched_barrier(0);
        });
        // keep the section's vector results in this section (they are consumed one
        // section later)
        asm volatile("" : "+v"(out.p[0]), "+v"(out.p[1]), "+v"(out.lsum), "+v"(out.ref), "+v"(ref_cur));
      });
    };
    for (int t = 0; t < n_tiles; t += 2) {
      halftile(t, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      halftile(t, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      if (t + 1 < n_tiles) {
        halftile(t + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
        halftile(t + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
      }
    }

    wait_vm();  // the last half's loads land before the next item loads into the same buffers
    if (!full) {
      // the buffer the last tile's first half loaded into (the next tile's V, of which there
      // is none) is read by no wave; with no tile, no wave reads any buffer in this item
      bf16* const spare = n_tiles > 0 ? (((n_tiles - 1) & 1) ? sV0 : sV1) : sV0;
      while (cur_chunk < a.c1) flush_partial(cur_chunk++, stage_of(spare));
    } else {
      const int ln = opaque(lane), h2 = ln >> 5;
      const float l_row = st.l + other_half(st.l);
      const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
      if (!absent) {
        bf16* op = (bf16*)a.o + bh_base + (int64_t)(qb * BLK + rg * 32 + (ln & 31)) * a.ss + 4 * h2;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const bf16x4 v4 = {(bf16)(st.acc[d][4 * g] * inv), (bf16)(st.acc[d][4 * g + 1] * inv),
                               (bf16)(st.acc[d][4 * g + 2] * inv), (bf16)(st.acc[d][4 * g + 3] * inv)};
            *(bf16x4*)(op + d * 32 + 8 * g) = v4;
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
    if (dyn) {
      if (tid == 0) {
        if (n_tiles == 0) next_pos = queue_take(a.dyn_ctr, p_end);  // (else taken during the first tile)
        sQueuePos = next_pos;
      }
      __syncthreads();  // (every wave read the previous position before this item's barriers)
      pos = __builtin_amdgcn_readfirstlane(sQueuePos);
    } else {
      ++pos;
    }
  }
  if (dyn && tid == 0) queue_finish(a.dyn_ctr);
}

template <int D, int BLK>
hipError_t launch_variant(const FwdArgs& a, hipStream_t stream) {
  const bool general = a.layout == SA_LAYOUT_STRIPED || a.S % BLK != 0;
  const dim3 grid(a.num_bins), block(Shape<D, BLK>::NW * 64);
  if constexpr (BLK == 128) {
    // Q-block pairs (S a multiple of the block; checked by the plan)
    if (a.q_pairs) {
      if (a.layout == SA_LAYOUT_STRIPED) {
        if (a.token_causal)
          hipLaunchKernelGGL((attn_bf16_pair_kernel<D, true, true>), grid, block, 0, stream, a);
        else
          hipLaunchKernelGGL((attn_bf16_pair_kernel<D, true, false>), grid, block, 0, stream, a);
      } else if (a.token_causal) {
        hipLaunchKernelGGL((attn_bf16_pair_kernel<D, false, true>), grid, block, 0, stream, a);
      } else {
        hipLaunchKernelGGL((attn_bf16_pair_kernel<D, false, false>), grid, block, 0, stream, a);
      }
      return hipGetLastError();
    }
    // striped chunks (S is then a multiple of block * n_chunks) without token-level causality
    if (a.layout == SA_LAYOUT_STRIPED) {
      if (a.token_causal)
        hipLaunchKernelGGL((attn_bf16_pipe_kernel<D, true, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((attn_bf16_pipe_kernel<D, true, false>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if (general)
    hipLaunchKernelGGL((attn_bf16_kernel<D, BLK, true, false>), grid, block, 0, stream, a);
  else if constexpr (BLK == 128) {
    if (a.token_causal)
      hipLaunchKernelGGL((attn_bf16_pipe_kernel<D, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_bf16_pipe_kernel<D, false, false>), grid, block, 0, stream, a);
  } else if (a.token_causal)
    hipLaunchKernelGGL((attn_bf16_kernel<D, BLK, false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, BLK, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int attn_bf16_wg_per_cu(int block) { return block >= 128 ? Shape<128, 128>::WG_PER_CU : Shape<128, 64>::WG_PER_CU; }

hipError_t launch_attn_bf16(const FwdArgs& a, int D, int block, hipStream_t stream) {
  if (D == 128 && block == 128) return launch_variant<128, 128>(a, stream);
  if (D == 64 && block == 128) return launch_variant<64, 128>(a, stream);
  if (D == 128 && block == 64) return launch_variant<128, 64>(a, stream);
  if (D == 64 && block == 64) return launch_variant<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
