// Top-k indexer of DeepSeek Sparse Attention (6D-parallel notes, section 7.1):
// a low-rank importance I[i, j] = <Q'_i, K'_j> with Q' = Q Wq and K' = K Wk
// (rank 32), and per query the top_k keys by importance (ties to the lower key
// index; with a causal mask the candidates of query i are j <= i and a query
// with fewer candidates than top_k takes all of them).
//
// 1. proj_kernel: Q' and K' in bf16 (fp32 sums over the head dimension in
//    index order, rounded to nearest-even), the precision the selection is
//    defined in.
// 2. select_kernel: one workgroup per 32 consecutive queries of a (batch,
//    head).  Importance tiles of 32 keys x 32 queries come from two
//    v_mfma_f32_32x32x16_bf16 (fp32 accumulate; the bf16 products are exact).
//    Each row's selection is a threshold K on a unique 64-bit key
//    key(j) = ord(I[i, j]) << 32 | (0xFFFF - j), ord being the order-preserving
//    map of fp32 onto uint32, so "larger key" means "higher importance, then
//    lower index" and exactly top_k keys lie above the right threshold.  A
//    counting pass streams all candidate keys of the 32 rows and appends those
//    above each row's threshold to the row's LDS buffer (kCap entries); while
//    the threshold's index part is all ones, a plain compare of the importance
//    with the threshold's float decides each key.  The threshold is first
//    estimated as a normal quantile (Abramowitz & Stegun 26.2.23) from the mean
//    and deviation of the row's importances over the block's key prefix, which
//    come from prefix sums of K' and K' K'^T in groups of kMomGroup keys
//    (moments_group_kernel, moments_scan_kernel), with no pass over the keys;
//    a pass that collects fewer than top_k or more than kCap keys moves it (by the normal-model distance between the observed and
//    the target count, then by bisection of the key space, which ends because
//    one more unit of the threshold removes at most one key).  Finally a wave
//    per row picks the exact top_k from its buffer: a radix select of the
//    top_k-th largest importance bits, 8 bits per round from the highest bit in
//    which the entries differ (a histogram of the next byte among the entries
//    that match the bits fixed so far), stopping once the boundary digit's whole
//    bin is taken, then, for ties, bisection on the key index.  The order of
//    the indices within a row's list is unspecified.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "internal.h"
#include "kernel_common.h"

namespace sa {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRank = 32;
constexpr int kRows = 32;          // queries per workgroup
constexpr int kWaves = 16;         // 4 per SIMD: the key stream is latency-bound
constexpr int kCap = 768;          // candidate buffer entries per row
constexpr int kPrefetch = 4;       // key blocks whose K' loads each wave keeps in flight
constexpr int kModelSteps = 6;     // threshold corrections from the normal model before bisection
constexpr int kMaxPasses = 80;     // kModelSteps + at most 64 bisections suffice
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint32_t ord_of(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of_ord(uint32_t o) {
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// Threshold that keeps exactly the importances strictly above t.
__device__ __forceinline__ uint64_t key_above(float t) { return ((uint64_t)ord_of(t) << 32) | 0xFFFFFFFFull; }

// Upper-tail normal quantile: z with P(N(0,1) > z) = p (Abramowitz & Stegun 26.2.23, |error| < 4.5e-4).
__device__ float normal_upper_quantile(float p) {
  const bool lower = p > 0.5f;
  const float pp = lower ? 1.f - p : p;
  const float t = sqrtf(-2.f * logf(fmaxf(pp, 1e-30f)));
  const float z = t - (2.515517f + t * (0.802853f + t * 0.010328f)) /
                          (1.f + t * (1.432788f + t * (0.189269f + t * 0.001308f)));
  return lower ? -z : z;
}

// ---------------------------------------------------------------------------
// Projections: Xp[row][r] = bf16(sum_d X[row][d] * W[d][r]), the sum an fp32 fma chain in
// index order.  Thread (g, r) of a 256-thread block keeps column r of W in registers (as
// fp32) and takes rows g, g + 8, ... of each chunk of kProjRows rows, which the block first
// stages in LDS as fp32 (one conversion per element; the 32 lanes of a group then read the
// same row, a broadcast).  The block strides over the chunks, so W is read once per block.
constexpr int kProjRows = 64;
constexpr int kProjBlocks = 1024;
template <int D>
__global__ __launch_bounds__(256) void proj_kernel(const bf16* __restrict__ X, const bf16* __restrict__ W,
                                                   bf16* __restrict__ Xp, int B, int H, int S, int64_t sb,
                                                   int64_t sh, int64_t ss) {
  constexpr int LD = D + 4;  // row stride in floats: rows of one wave's two groups fall on other banks
  __shared__ __attribute__((aligned(16))) float xs[kProjRows * LD];
  const int r = threadIdx.x & 31, g = threadIdx.x >> 5;
  float w[D];
#pragma unroll
  for (int d = 0; d < D; ++d) w[d] = (float)W[d * kRank + r];
  const int64_t rows = (int64_t)B * H * S;
  const int64_t n_chunks = (rows + kProjRows - 1) / kProjRows;
  constexpr int NL = kProjRows * (D / 8) / 256;  // 16-byte row pieces per thread and chunk
  static_assert(NL * 256 == kProjRows * (D / 8), "a chunk's pieces cover the block evenly");
  // piece c of a chunk: row c / (D/8), elements (c % (D/8)) * 8 .. +7; a piece past the last
  // row is zero (and never stored)
  auto load_chunk = [&](int64_t chunk, bf16x8 (&v)[NL]) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int c = threadIdx.x + 256 * k;
      const int64_t row = chunk * kProjRows + c / (D / 8);
      v[k] = bf16x8{};
      if (row < rows) {
        const int i = (int)(row % S);
        const int bh = (int)(row / S);
        v[k] = *(const bf16x8*)(X + (int64_t)(bh / H) * sb + (int64_t)(bh % H) * sh + (int64_t)i * ss +
                                (c % (D / 8)) * 8);
      }
    }
  };
  // the next chunk's rows are loaded into registers while the current one is computed
  bf16x8 nxt[NL];
  if (blockIdx.x < n_chunks) load_chunk(blockIdx.x, nxt);
  for (int64_t chunk = blockIdx.x; chunk < n_chunks; chunk += gridDim.x) {
    const int64_t row0 = chunk * kProjRows;
    __syncthreads();  // the previous chunk's rows are consumed
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int c = threadIdx.x + 256 * k;
      float* dst = xs + (c / (D / 8)) * LD + (c % (D / 8)) * 8;
      const bf16x8 v = nxt[k];
      *(float4*)dst = float4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
      *(float4*)(dst + 4) = float4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
    }
    __syncthreads();
    if (chunk + gridDim.x < n_chunks) load_chunk(chunk + gridDim.x, nxt);
    for (int rr = g; rr < kProjRows; rr += 8) {
      const int64_t row = row0 + rr;
      if (row >= rows) break;
      const float* x = xs + rr * LD;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 xv = *(const float4*)(x + d);
        acc = fmaf(xv.x, w[d], acc);
        acc = fmaf(xv.y, w[d + 1], acc);
        acc = fmaf(xv.z, w[d + 2], acc);
        acc = fmaf(xv.w, w[d + 3], acc);
      }
      Xp[row * kRank + r] = (bf16)acc;
    }
  }
}

// ---------------------------------------------------------------------------
struct RowCtl {
  uint64_t K, lo, hi;  // threshold; largest known with too many keys above; smallest known with too few
  float mean, sd;
  int n, need, done, found;  // candidates, keys to select, finished, keys in the buffer once finished
};

struct SelShared {
  float score[kRows][kCap];
  uint16_t key[kRows][kCap];
  int cnt[kRows];
  RowCtl ctl[kRows];
  int active;
};

// K' operand of key block kb: lane holds K'[kb*32 + lane%32][8*(lane/32) .. +7] and the
// same 8 ranks + 16 (rows beyond S repeat the last row; they are masked below).
struct KFrag {
  bf16x8 k0, k1;
};
__device__ __forceinline__ KFrag load_kfrag(const bf16* __restrict__ kp, int kb, int S, int lane) {
  const bf16* p = kp + (int64_t)min(kb * 32 + (lane & 31), S - 1) * kRank + 8 * (lane >> 5);
  return KFrag{*(const bf16x8*)p, *(const bf16x8*)(p + 16)};
}

// Importance tile of key block kb: element r holds key kb*32 + 8*(r/4) + 4*(lane/32) + r%4
// of query i (= i0 + lane%32); when `edge` (the block crosses the diagonal or the end of the
// sequence) invalid pairs are set to -inf.
__device__ __forceinline__ f32x16 tile_scores(const KFrag& kf, const bf16x8 (&qf)[2], int kb, int S, int i,
                                              bool causal, bool edge, int lane) {
  f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.k0, qf[0], f32x16{}, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.k1, qf[1], acc, 0, 0, 0);
  // wave-uniform, and rare (diagonal and last blocks): a branch, not predicated code
  if (__builtin_expect(__builtin_amdgcn_readfirstlane((int)edge) != 0, 0)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (j >= S || i >= S || (causal && j > i)) acc[r] = kNegInf;
    }
  }
  return acc;
}

// Prefix moments of K' for the threshold estimate: entry g of a (batch, head) holds the sum
// of K'_j (kRank floats) and of K'_j K'_j^T (kRank x kRank, row-major) over the keys
// [0, min(kMomGroup g, S)).  moments_group_kernel writes group g's own sums into entry g + 1
// (and zeroes entry 0); moments_scan_kernel turns entries 1.. into running sums.
__global__ __launch_bounds__(256) void moments_group_kernel(const bf16* __restrict__ kp, float* __restrict__ mom,
                                                            int S, int n_groups) {
  __shared__ float ks[kMomGroup][kRank + 1];
  const int bh = blockIdx.x / n_groups, g = blockIdx.x % n_groups;
  const int nk = min(kMomGroup, S - g * kMomGroup);
  const bf16* src = kp + ((int64_t)bh * S + (int64_t)g * kMomGroup) * kRank;
  for (int c = threadIdx.x; c < kMomGroup * kRank / 8; c += 256) {
    const int j = c / (kRank / 8), r8 = (c % (kRank / 8)) * 8;
    bf16x8 v = {};
    if (j < nk) v = *(const bf16x8*)(src + (int64_t)j * kRank + r8);
#pragma unroll
    for (int e = 0; e < 8; ++e) ks[j][r8 + e] = (float)v[e];
  }
  __syncthreads();
  float* dst = mom + ((int64_t)bh * (n_groups + 1) + g + 1) * kMomEntry;
  // thread t: row t / 8 of K'K'^T, columns 4 (t % 8) .. +3
  const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < kMomGroup; ++j) {
    const float x = ks[j][r];
    a0 = fmaf(x, ks[j][c0], a0);
    a1 = fmaf(x, ks[j][c0 + 1], a1);
    a2 = fmaf(x, ks[j][c0 + 2], a2);
    a3 = fmaf(x, ks[j][c0 + 3], a3);
  }
  *(float4*)(dst + kRank + r * kRank + c0) = float4{a0, a1, a2, a3};
  if (threadIdx.x < kRank) {
    float t = 0.f;
    for (int j = 0; j < kMomGroup; ++j) t += ks[j][threadIdx.x];
    dst[threadIdx.x] = t;
  }
  if (g == 0)
    for (int e = threadIdx.x; e < kMomEntry; e += 256) mom[(int64_t)bh * (n_groups + 1) * kMomEntry + e] = 0.f;
}

__global__ __launch_bounds__(256) void moments_scan_kernel(float* __restrict__ mom, int n_bh, int n_groups) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)n_bh * kMomEntry) return;
  const int bh = (int)(t / kMomEntry), e = (int)(t % kMomEntry);
  float* col = mom + (int64_t)bh * (n_groups + 1) * kMomEntry + e;
  constexpr int CH = 32;  // entries loaded together
  float run = 0.f;
  for (int g0 = 1; g0 <= n_groups; g0 += CH) {
    float v[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) v[k] = g0 + k <= n_groups ? col[(int64_t)(g0 + k) * kMomEntry] : 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      run += v[k];
      if (g0 + k <= n_groups) col[(int64_t)(g0 + k) * kMomEntry] = run;
    }
  }
}

__device__ __forceinline__ int wave_count(bool pred) { return __builtin_popcountll(__ballot(pred)); }

__global__ __launch_bounds__(kWaves * 64) void select_kernel(IndexerArgs a) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int blocks_per_bh = (a.S + kRows - 1) / kRows;
  // each XCD takes whole heads in turn, so the head's K' blocks that every query block
  // streams stay in that XCD's L2
  const int blk = xcd_contiguous(blockIdx.x, gridDim.x, a.n_xcd);
  const int bh = blk / blocks_per_bh;
  const int i0 = (blk % blocks_per_bh) * kRows;
  const bool causal = a.causal != 0;
  const bf16* qp = a.qp + (int64_t)bh * a.S * kRank;
  const bf16* kp = a.kp + (int64_t)bh * a.S * kRank;
  const int i = i0 + l32;  // this lane's query

  // Q'^T operand: lane holds Q'[i][8*h2 .. +7] (k-step 0) and Q'[i][16 + 8*h2 .. +7] (k-step 1).
  bf16x8 qf[2];
  {
    const bf16* p = qp + (int64_t)min(i, a.S - 1) * kRank + 8 * h2;
    qf[0] = *(const bf16x8*)p;
    qf[1] = *(const bf16x8*)(p + 16);
  }
  const int i_last = min(i0 + kRows - 1, a.S - 1);
  // key blocks that need masking: those reaching past the first query of the block (causal)
  // or past the end of the sequence, and all of them when the block has rows beyond S
  const int first_edge_kb = i0 + kRows > a.S ? 0 : (causal ? i0 / 32 : (a.S - 1) / 32);
  const int n_max = causal ? i_last + 1 : a.S;  // most candidates of any row of the block
  const int nkb = (n_max + 31) / 32;

  if (tid < kRows) {
    const int ir = i0 + tid;
    RowCtl& c = sh.ctl[tid];
    c.n = ir < a.S ? (causal ? ir + 1 : a.S) : 0;
    c.need = min(a.top_k, c.n);
    c.lo = 0;
    c.hi = ~0ull;
    c.K = 0;  // every candidate is above key 0
    c.done = c.n == 0;
    c.found = 0;
    c.mean = 0.f;
    c.sd = 0.f;
  }

  // Threshold estimate for rows with more candidates than the buffer holds: the mean and
  // deviation of the row's importances over the keys of the block's moment prefix, from the
  // prefix sums of K' and of K' K'^T (mean = q.K1 / N, second moment = q^T K2 q / N).
  if (n_max > kCap) {
    const int n_groups = (a.S + kMomGroup - 1) / kMomGroup;
    const int gsel = causal ? (i0 + 1) / kMomGroup : n_groups;  // keys [0, min(kMomGroup gsel, S))
    const float n_mom = (float)min(gsel * kMomGroup, a.S);
    const float* me = a.mom + ((int64_t)bh * (n_groups + 1) + gsel) * kMomEntry;
    // wave w takes rows 2w (lanes 0-31) and 2w + 1 (lanes 32-63); lane l32 holds rank l32
    const int row = 2 * wave + h2;
    const int ir = min(i0 + row, a.S - 1);
    float q[kRank];
#pragma unroll
    for (int v = 0; v < kRank / 8; ++v) {
      const bf16x8 x = *(const bf16x8*)(qp + (int64_t)ir * kRank + 8 * v);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[8 * v + e] = (float)x[e];
    }
    float y = 0.f;  // (K2 q)[l32]
#pragma unroll
    for (int v = 0; v < kRank / 4; ++v) {
      const float4 k2 = *(const float4*)(me + kRank + l32 * kRank + 4 * v);
      y = fmaf(k2.x, q[4 * v], y);
      y = fmaf(k2.y, q[4 * v + 1], y);
      y = fmaf(k2.z, q[4 * v + 2], y);
      y = fmaf(k2.w, q[4 * v + 3], y);
    }
    float qr = q[0];
#pragma unroll
    for (int r = 1; r < kRank; ++r) qr = l32 == r ? q[r] : qr;  // q[l32]
    float s1 = qr * me[l32], s2 = qr * y;
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1) {
      s1 += __shfl_xor(s1, w);
      s2 += __shfl_xor(s2, w);
    }
    __syncthreads();  // the rows' control entries are initialised
    if (l32 == 0 && i0 + row < a.S) {
      RowCtl& c = sh.ctl[row];
      c.mean = n_mom > 0.f ? s1 / n_mom : 0.f;
      c.sd = n_mom > 0.f ? sqrtf(fmaxf(s2 / n_mom - c.mean * c.mean, 0.f)) : 0.f;
      if (c.n > kCap) {
        const float target = 0.5f * (float)(c.need + kCap);
        c.K = key_above(c.mean + c.sd * normal_upper_quantile(target / (float)c.n));
      }
    }
  }
  __syncthreads();

  // Counting passes until every row has between need and kCap keys above its threshold.
  for (int pass = 0; pass < kMaxPasses; ++pass) {
    if (tid < kRows) {
      if (!sh.ctl[tid].done) sh.cnt[tid] = 0;
      if (tid == 0) sh.active = 0;
    }
    __syncthreads();
    const RowCtl& c = sh.ctl[l32];
    const bool live = !c.done;
    const uint64_t K = live ? c.K : ~0ull;
    const uint32_t k_hi = (uint32_t)(K >> 32);
    const float t_filter = !live ? __builtin_huge_valf() : (k_hi == 0 ? kNegInf : float_of_ord(k_hi));
    // A threshold whose index part is all ones (every threshold but those of the bisection
    // fallback) keeps exactly the importances strictly above t_filter: then one compare per
    // key decides, with no tie test.  Wave-uniform.
    const bool plain = __ballot(!(K == 0 || (uint32_t)K == 0xFFFFFFFFu)) == 0;
    auto process_plain = [&](const f32x16& sc, int kb) {
      bool sel[16];
      int c = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sel[r] = sc[r] > t_filter;
        c += sel[r] ? 1 : 0;
      }
      if (__ballot(c > 0) == 0) return;
      int pos = 0;
      if (c > 0) pos = atomicAdd(&sh.cnt[l32], c);  // one claim per lane
      const int kbase = kb * 32 + 4 * h2;
      if (__builtin_expect(__ballot(pos + c > kCap) == 0, 1)) {
        // the common case: every claimed slot is inside the buffer; the stores are unrolled
        // over the 16 scores, each under its compare's lane mask (no dynamic register index)
        float* ps = &sh.score[l32][pos];
        uint16_t* pk = &sh.key[l32][pos];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (sel[r]) {
            *ps++ = sc[r];
            *pk++ = (uint16_t)(kbase + 8 * (r >> 2) + (r & 3));
          }
      } else {
        // the buffer overflows (the pass is repeated): keep the slots that fit
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (sel[r]) {
            if (pos < kCap) {
              sh.score[l32][pos] = sc[r];
              sh.key[l32][pos] = (uint16_t)(kbase + 8 * (r >> 2) + (r & 3));
            }
            ++pos;
          }
      }
    };
    auto process = [&](const f32x16& sc, int kb) {
      float m = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, sc[r]);
      const bool maybe = m != kNegInf && m >= t_filter;
      if (__ballot(maybe)) {
        if (maybe) {
          // which of the 16 keys lie above the threshold (importance above t_filter, or equal
          // to it with the index part of the key deciding)
          uint32_t bits = 0;
          bool tie = false;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            bits |= (sc[r] > t_filter ? 1u : 0u) << r;
            tie |= sc[r] == t_filter;
          }
          // exact ties with the threshold are rare: branch on the whole wave, so that the key
          // compares below do not run (predicated) for every block
          if (__builtin_expect(__ballot(tie) != 0, 0) && tie) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = kb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
              const uint64_t key = ((uint64_t)ord_of(sc[r]) << 32) | (uint32_t)(0xFFFF - j);
              if (sc[r] == t_filter && sc[r] != kNegInf && key > K) bits |= 1u << r;
            }
          }
          if (bits) {
            int pos = atomicAdd(&sh.cnt[l32], __builtin_popcount(bits));  // one claim per lane
            while (bits) {
              const int r = __builtin_ctz(bits);
              bits &= bits - 1;
              if (pos < kCap) {
                sh.score[l32][pos] = sc[r];
                sh.key[l32][pos] = (uint16_t)(kb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3));
              }
              ++pos;
            }
          }
        }
      }
    };
    // key blocks wave, wave + kWaves, ...: each wave keeps kPrefetch blocks' K' loads in
    // flight.  A slot is refilled once its MFMAs have read it, into the same registers, and
    // every round issues the same loads (past the last block they repeat it, a cache hit), so
    // that each block waits only for its own loads (conditional loads, or a refill while the
    // old operand is still live, made the compiler wait for all of them at every round's end).
    KFrag ring[kPrefetch];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
      ring[p] = load_kfrag(kp, min(wave + p * kWaves, nkb - 1), a.S, lane);
      // issue order = use order (the first slot's wait then counts only the later slots)
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int kb0 = wave; kb0 < nkb; kb0 += kPrefetch * kWaves) {
#pragma unroll
      for (int p = 0; p < kPrefetch; ++p) {
        const int kb = kb0 + p * kWaves;
        const f32x16 sc = tile_scores(ring[p], qf, kb, a.S, i, causal, kb >= first_edge_kb, lane);
        ring[p] = load_kfrag(kp, min(kb + kPrefetch * kWaves, nkb - 1), a.S, lane);
        if (kb < nkb) {
          if (plain)
            process_plain(sc, kb);
          else
            process(sc, kb);
        }
      }
    }
    __syncthreads();
    if (tid < kRows) {
      RowCtl& cc = sh.ctl[tid];
      if (!cc.done) {
        const int n = sh.cnt[tid];
        if (n >= cc.need && n <= kCap) {
          cc.done = 1;
          cc.found = n;
        } else {
          if (n > kCap)
            cc.lo = cc.K;
          else
            cc.hi = cc.K;
          uint64_t next = cc.lo + (cc.hi - cc.lo) / 2;
          if (pass < kModelSteps && cc.sd > 0.f) {
            // move by the normal-model distance between the observed and the target count
            const float t = float_of_ord((uint32_t)(cc.K >> 32));
            const float nn = (float)cc.n;
            const float target = 0.5f * (float)(cc.need + kCap);
            const float seen = fminf(fmaxf((float)n, 0.5f), nn - 0.5f);
            const uint64_t kk = key_above(t + cc.sd * (normal_upper_quantile(target / nn) -
                                                       normal_upper_quantile(seen / nn)));
            if (kk > cc.lo && kk < cc.hi) next = kk;
          }
          cc.K = next;
          atomicAdd(&sh.active, 1);
        }
      }
    }
    __syncthreads();
    const int still_active = sh.active;
    __syncthreads();  // everyone has read it before the next pass resets it
    if (still_active == 0) break;
  }

  // Exact top-need of each row's buffer: wave w takes rows w, w + 4, ...
  constexpr int kPer = (kCap + 63) / 64;
  for (int row = wave; row < kRows; row += kWaves) {
    const int ir = i0 + row;
    if (ir >= a.S) break;
    const int n = sh.ctl[row].found;
    const int need = sh.ctl[row].need;
    uint32_t o[kPer];
    int jj[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int p = e * 64 + lane;
      o[e] = p < n ? ord_of(sh.score[row][p]) : 0u;
      jj[e] = p < n ? (int)sh.key[row][p] : 0x7FFFFFFF;
    }
    auto count_if = [&](auto pred) {
      int c = 0;
#pragma unroll
      for (int e = 0; e < kPer; ++e) c += wave_count(e * 64 + lane < n && pred(o[e], jj[e]));
      return c;
    };
    uint32_t t_ord = 0;   // selected: ord > t_ord, plus ord == t_ord with index <= t_j
    int t_j = -1;
    if (n > need) {
      // Radix select of the need-th largest ord, 8 bits at a time from the first bit in which
      // the entries differ (the buffered keys are the row's largest, so their leading bits
      // mostly agree, and a histogram of a shared digit would also put every lane's atomic
      // add on one bin): a histogram
      // of the next digit among the entries that match the digits fixed so far, then the
      // digit where the count from the top reaches the keys still needed.  The histogram
      // lives in this row's score buffer, whose entries are now in registers (a wave's LDS
      // accesses complete in order, so the reads above precede these writes).
      uint32_t* hist = (uint32_t*)sh.score[row];
      // the entries' common leading bits need no round: the first digit window ends at the
      // highest bit in which they differ
      uint32_t o_lo = 0xFFFFFFFFu, o_hi = 0u;
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (e * 64 + lane < n) {
          o_lo = min(o_lo, o[e]);
          o_hi = max(o_hi, o[e]);
        }
#pragma unroll
      for (int w = 32; w >= 1; w >>= 1) {
        o_lo = min(o_lo, (uint32_t)__shfl_xor((int)o_lo, w));
        o_hi = max(o_hi, (uint32_t)__shfl_xor((int)o_hi, w));
      }
      const uint32_t diff = o_lo ^ o_hi;  // n > need >= 1, so both are entries
      const int top = diff ? 31 - __builtin_clz(diff) : 0;
      const int shift0 = max(top - 7, 0);
      uint32_t pmask = shift0 + 8 >= 32 ? 0u : ~0u << (shift0 + 8);
      uint32_t prefix = o_hi & pmask;
      int remaining = need;  // keys still to take among the entries matching prefix
      bool whole_bin = false;  // every entry matching prefix is taken: no lower digit decides
      for (int shift = shift0; ; shift = max(shift - 8, 0)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) hist[q * 64 + lane] = 0u;
#pragma unroll
        for (int e = 0; e < kPer; ++e)
          if (e * 64 + lane < n && (o[e] & pmask) == prefix) atomicAdd(&hist[(o[e] >> shift) & 255u], 1u);
        // lane L holds digits 4L .. 4L+3; counts of larger digits come from the lanes above
        const uint32_t cnt[4] = {hist[4 * lane], hist[4 * lane + 1], hist[4 * lane + 2], hist[4 * lane + 3]};
        const uint32_t mine = cnt[0] + cnt[1] + cnt[2] + cnt[3];
        uint32_t above = mine;  // inclusive suffix sum over lanes >= this one
#pragma unroll
        for (int w = 1; w < 64; w <<= 1) {
          const uint32_t v = (uint32_t)__shfl_down((int)above, w);
          if (lane + w < 64) above += v;
        }
        above -= mine;  // entries with a digit above this lane's four
        // find the digit d with count(> d) < remaining <= count(>= d); exactly one lane has it
        int found = -1;
        uint32_t gt_found = 0, n_found = 0;
        uint32_t ge = above;
#pragma unroll
        for (int k = 3; k >= 0; --k) {
          const uint32_t gt = ge;
          ge += cnt[k];
          if (found < 0 && gt < (uint32_t)remaining && ge >= (uint32_t)remaining) {
            found = 4 * lane + k;
            gt_found = gt;
            n_found = cnt[k];
          }
        }
        const uint64_t who = __ballot(found >= 0);
        const int src = __builtin_ctzll(who);
        const int digit = __shfl(found, src);
        const uint32_t gt_d = (uint32_t)__shfl((int)gt_found, src);
        const uint32_t n_d = (uint32_t)__shfl((int)n_found, src);
        prefix |= (uint32_t)digit << shift;
        pmask |= 255u << shift;
        remaining -= (int)gt_d;
        // the digit's whole bin is taken (its smallest entry is the need-th largest): the
        // selection is every entry at or above prefix, whatever the lower bits
        if (n_d == (uint32_t)remaining) {
          whole_bin = true;
          break;
        }
        if (shift == 0) break;
      }
      const uint32_t hi = prefix;  // the need-th largest ord, or with whole_bin a lower bound of the taken bin
      const int c_hi = need - remaining;  // entries strictly above it
      t_ord = hi;
      const int ties_needed = need - c_hi;
      if (whole_bin) {
        t_j = 0xFFFF;  // ord > hi, or ord == hi with any index
      } else if (count_if([&](uint32_t ov, int) { return ov == hi; }) == ties_needed) {
        t_j = 0xFFFF;  // every tied key is taken (the usual case: the tie is the need-th key alone)
      } else {
        // smallest index bound taking ties_needed of the tied keys (lowest indices first)
        int jlo = -1, jhi = 0xFFFF;
        while (jhi - jlo > 1) {
          const int mid = (jlo + jhi) / 2;
          if (count_if([&](uint32_t ov, int jv) { return ov == hi && jv <= mid; }) >= ties_needed)
            jhi = mid;
          else
            jlo = mid;
        }
        t_j = jhi;
      }
    }
    int32_t* out = a.idx + ((int64_t)bh * a.S + ir) * a.top_k;
    int base = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const bool sel = e * 64 + lane < n && (n <= need || o[e] > t_ord || (o[e] == t_ord && jj[e] <= t_j));
      const uint64_t bits = __ballot(sel);
      const int pos = base + __builtin_popcountll(bits & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
      if (sel && pos < a.top_k) out[pos] = jj[e];
      base += __builtin_popcountll(bits);
    }
    if (lane == 0) a.count[(int64_t)bh * a.S + ir] = min(base, need);
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream) {
  if (a.rank != kRank || a.top_k < 1 || a.top_k > kIndexerMaxTopK || a.S > 65536 || (a.D != 64 && a.D != 128))
    return hipErrorInvalidValue;
  const int64_t rows = (int64_t)a.B * a.H * a.S;
  const dim3 pg((unsigned)std::min<int64_t>((rows + kProjRows - 1) / kProjRows, kProjBlocks));
  auto proj = [&](const void* x, const void* w, bf16* xp) {
    if (a.D == 128)
      hipLaunchKernelGGL(proj_kernel<128>, pg, dim3(256), 0, stream, (const bf16*)x, (const bf16*)w, xp, a.B, a.H,
                         a.S, a.sb, a.sh, a.ss);
    else
      hipLaunchKernelGGL(proj_kernel<64>, pg, dim3(256), 0, stream, (const bf16*)x, (const bf16*)w, xp, a.B, a.H,
                         a.S, a.sb, a.sh, a.ss);
  };
  proj(a.q, a.wq, a.qp);
  proj(a.k, a.wk, a.kp);
  const int n_groups = (a.S + kMomGroup - 1) / kMomGroup;
  const int n_bh = a.B * a.H;
  hipLaunchKernelGGL(moments_group_kernel, dim3((unsigned)(n_bh * n_groups)), dim3(256), 0, stream, a.kp, a.mom, a.S,
                     n_groups);
  hipLaunchKernelGGL(moments_scan_kernel, dim3((unsigned)((n_bh * kMomEntry + 255) / 256)), dim3(256), 0, stream,
                     a.mom, n_bh, n_groups);
  const int blocks = a.B * a.H * ((a.S + kRows - 1) / kRows);
  hipLaunchKernelGGL(select_kernel, dim3(blocks), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
