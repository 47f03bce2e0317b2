// Internal declarations shared by the host runtime and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "sparse_attn.h"

namespace sa {

// Limits of the compiled kernels (checked before any launch).
constexpr int kMaxTilesPerRow = 2048;  // nK <= 2048: per-item tile list lives in LDS
constexpr int kMaxChunks = 64;
constexpr int kDevicePlanMaxItems = 16384;  // B*H*nQ of a plan made on the device (LDS sort buffer)
constexpr int kDevicePlanMaxBins = 1024;    // one bin key per thread of the planning workgroup
constexpr int kMaxMergeParts = 64;

// Tile descriptor packed in an int32 (per-item tile list):
//   bits  0..19 tile index (contiguous: KV block j; striped: compacted tile t)
//   bits 20..23 live 32-key-group code (striped; all ones for contiguous)
//   bits 24..29 chunk index
constexpr int kDescCodeShift = 20;
constexpr int kDescChunkShift = 24;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;        // full mode output (problem dtype), nullptr in partial mode
  float* o_part;  // partial mode: [n][B][H][S][D]
  float* m_part;  // [n][B][H][S]
  float* l_part;
  const uint8_t* mask;    // [B][H][nQ][nK]
  const int32_t* items;   // work list of this launch
  const int32_t* bin_ptr; // [num_bins + 1]
  // run-time queue (SA_ORDER_LPT_DYNAMIC), null otherwise: items in LPT order and two
  // counters (next position, finished workgroups) that the last workgroup resets
  const int32_t* dyn_items;
  int32_t* dyn_ctr;
  int64_t* trace;         // nullable
  int32_t B, H, S, nQ, nK, n_chunks, layout, c0, c1;
  int32_t num_bins;
  int32_t token_causal;  // also drop keys after the query inside live tiles
  int32_t q_pairs;       // items are Q-block pairs (2p, 2p+1): item = (b*H + h)*nI + p
  int32_t nI;            // items per (batch, head): nQ, or ceil(nQ / 2) with q_pairs
  int64_t sb, sh, ss;
  float scale;        // natural-log softmax scale
  float scale_log2;   // scale * log2(e)
};

struct GatherArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* idx;    // [B][H][S][top_k]
  const int32_t* count;  // [B][H][S]
  int32_t B, H, S, D, top_k;
  int64_t sb, sh, ss;
  float scale_log2;
};

// The indexer's per-row candidate buffer leaves room above the selection size.
constexpr int kIndexerMaxTopK = 512;
// Keys per group of the indexer's prefix moments, and floats per moment entry (rank 32: the
// sum of K' and the sum of K' K'^T).
// counters per list of the run-time queue: one next position per XCD, finished workgroups
constexpr int kQueueCtrs = 16;
constexpr int kMomGroup = 128;
constexpr int kMomEntry = 32 + 32 * 32;

struct IndexerArgs {
  const void* q;
  const void* k;
  const void* wq;  // [D][rank] bf16
  const void* wk;
  __bf16* qp;      // [B][H][S][rank] projections (plan scratch)
  __bf16* kp;
  float* mom;      // [B][H][S/128 + 1][rank + rank*rank] prefix moments of K' (plan scratch)
  int32_t* idx;    // [B][H][S][top_k]
  int32_t* count;  // [B][H][S]
  int32_t B, H, S, D, rank, top_k, causal;
  int64_t sb, sh, ss;
  int32_t n_xcd;  // L2 domains of the device (workgroups are dealt to them round-robin)
};

struct MergeArgs {
  const float* o[kMaxMergeParts];
  const float* m[kMaxMergeParts];
  const float* l[kMaxMergeParts];
  void* out;
  float* lse;
  int64_t rows;
  int32_t n_parts;
};

// Kernel launchers (defined in the .hip files).  Return hipSuccess or the launch error.
// Row, column and per-chunk row counts of the block mask; with prow/pcrow also the union counts
// of Q-block pairs (2p, 2p+1): prow [BH*nP], pcrow [BH][C][nP], nP = ceil(nQ/2).
hipError_t launch_popcount(const uint8_t* mask, int BH, int nQ, int nK, int n_chunks, int layout,
                           int32_t* row, int32_t* col, int32_t* crow, hipStream_t stream,
                           int32_t* prow = nullptr, int32_t* pcrow = nullptr);
// Round-based LPT of the lists of a block plan on the device: list 0 from row, list 1 + c
// from chunk c of crow.  Lists [list0, list0 + n_lists) are made (n_lists < 0: through list
// C), list list0 + s written to slot s of items [.][BH*nQ], bin_ptr [.][m+1], bin_load [.][m]
// and stats [.][4] = (load sum, max item load, makespan, lower bound).
// order (nullable): each list's items in LPT order; dyn_ctr (nullable): kQueueCtrs counters
// per list, zeroed (the run-time queue of SA_ORDER_LPT_DYNAMIC)
hipError_t launch_plan_rounds(const int32_t* row, const int32_t* crow, int BH, int nQ, int C, int m, int32_t* items,
                              int32_t* bin_ptr, int64_t* bin_load, int64_t* stats, hipStream_t stream,
                              int list0 = 0, int n_lists = -1, int32_t* order = nullptr,
                              int32_t* dyn_ctr = nullptr);
hipError_t launch_attn_bf16(const FwdArgs& a, int D, int block, hipStream_t stream);
int attn_bf16_wg_per_cu(int block);  // workgroups the bf16 kernel keeps resident per CU
hipError_t launch_attn_f32(const FwdArgs& a, int D, int block, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int D, int out_dtype, hipStream_t stream);
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);
hipError_t launch_gather_attn(const GatherArgs& a, hipStream_t stream);

// Host helpers of the C ABI (api.cpp), shared by the entry points in other files.
sa_status set_error(sa_status st, const char* fmt, ...);       // records the last-error text
sa_status validate_block_problem(const sa_problem* p);          // as for a block plan
int default_num_bins(const sa_problem& p, int device);          // one bin per resident workgroup
float softmax_scale(const sa_problem& p);                       // scale, or 1/sqrt(D) when <= 0

// Host LPT / round-robin (lpt.cpp).  Items are 0..n-1 with loads[i] >= 0.
//   LPT: sort by (load desc, id asc); each item goes to the least-loaded bin,
//   ties to the lowest bin index; each bin keeps assignment order.
//   NAIVE: item i goes to bin i mod m, in id order.
void assign(const int64_t* loads, int n, int m, int order, int32_t* items_out, int32_t* bin_ptr_out,
            int64_t* bin_load_out);
// Two-level LPT: heads to bin groups (bins b with b mod groups == g), then each group's
// items to its bins (lpt.cpp).  n = n_heads * per_head items, item id = head * per_head + q.
void assign_grouped(const int64_t* loads, int n_heads, int per_head, int m, int groups, int32_t* items_out,
                    int32_t* bin_ptr_out, int64_t* bin_load_out);

}  // namespace sa
