/*
 * sparse_attn.h — C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * What it computes.  Multi-head attention in which each head carries a block
 * mask: rows are Q-blocks, columns are KV-blocks, and only the non-zero
 * ("dense") entries are computed (db-SP post on load balancing sparse-attention
 * head and sequence parallelism, scenario 2).  For every live tile the library
 * runs a flash-attention tile; KV is visited in chunks, each chunk being one
 * ring-attention step's KV shard, and the per-chunk partial softmax states
 * (O, m, l) are combined by the online-softmax merge of the 6D-parallel
 * attention notes, section 2.1.  Work items (one per (batch, head, Q-block))
 * are ordered by the LPT greedy of the db-SP post so that the persistent
 * kernel's workgroups carry equal numbers of live tiles.  A second sparsity
 * kind follows the same notes' section 7.1 (DSA): a rank-r indexer picks the
 * top-k keys of every query and attention runs over those keys only.
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers unless the comment says (host).
 *  - Q, K, V and O are indexed [b, h, s, d] through the element strides
 *    sb, sh, ss of sa_problem; d is contiguous (stride 1).  Q, K, V, O share
 *    one stride set.  bf16 data is IEEE bfloat16, f32 is IEEE binary32.
 *  - Per-chunk partials are dense fp32: O_part [n][B][H][S][D], m_part and
 *    l_part [n][B][H][S], where n = chunk_end - chunk_begin.  O_part is the
 *    UNNORMALISED sum of exp(s - m) v, m is the row max of the scaled scores in
 *    natural-log units, l = sum exp(s - m).  A row with no live key in a chunk
 *    gets (O, m, l) = (0, -inf, 0).
 *  - A row with no live key at all gets O = 0 (and lse = -inf).
 *  - Every call is asynchronous on the given stream unless stated otherwise;
 *    no call allocates device memory except sparse_attn_plan (which takes its
 *    buffers from the library's cache of destroyed plans' buffers first).
 *  - Errors are negative sa_status codes; no C++ exception crosses the ABI.
 *    Arguments are validated before anything is launched.  On SA_ERR_HIP the
 *    HIP error text is available from sa_last_error() (thread-local).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID = -1,     /* bad pointer, shape, stride or range */
  SA_ERR_UNSUPPORTED = -2, /* valid request outside the compiled kernel variants */
  SA_ERR_HIP = -3,         /* a HIP runtime call failed; see sa_last_error() */
  SA_ERR_NOMEM = -4        /* device or host allocation failed (plan only) */
} sa_status;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;
/* Work order of a block plan (db-SP post, LPT paragraph).
 *  SA_ORDER_LPT:     one LPT pass over all (b, h, Q-block) items onto the bins.
 *  SA_ORDER_NAIVE:   item i to bin i mod num_bins (round-robin in id order).
 *  SA_ORDER_LPT_XCD: two-level LPT for L2 locality (the post's "stay-home" bonus
 *                    re-read for one chip): heads to the chip's XCDs by LPT on
 *                    head loads, then each XCD's items by LPT onto its bins (bin b
 *                    runs on XCD b mod #XCDs).  Plain LPT when num_bins is not a
 *                    multiple of the XCD count.
 *  SA_ORDER_LPT_DEVICE: round-based LPT made on the GPU, for runtime masks (the
 *                    post notes that they add planning overhead): items in LPT
 *                    order are handed out num_bins per round, the round's j-th
 *                    item to the j-th least-loaded bin (lower index on ties).
 *                    Block plans only; at most 16384 work items (b, h, Q-block
 *                    or, with q_pairs, Q-block pair) and
 *                    1024 bins (else SA_ERR_UNSUPPORTED).  The plan call then
 *                    never waits for the device: popcount and every list
 *                    (full range and each chunk) are made on `stream`, and
 *                    sparse_attn_plan_info waits for them to read the statistics.
 *  SA_ORDER_LPT_DYNAMIC: the LPT rule in its list-scheduling form: the items in
 *                    LPT order (load descending, id ascending) form a queue, and
 *                    each persistent workgroup takes a new item whenever it is
 *                    free, so work goes to the compute unit that becomes free first
 *                    at run time rather than by the loads alone.  Queue position i
 *                    belongs to XCD i mod 8 (workgroup b runs on XCD b mod 8): a
 *                    workgroup takes its XCD's next position, and another XCD's once
 *                    its own are all taken.  The plan is made on the GPU as for
 *                    SA_ORDER_LPT_DEVICE (same limits; its bin lists are also made
 *                    and exported) plus the queue of each list (SA_PLAN_LPT_ORDER)
 *                    and 16 counters per list, which the forward's last workgroup
 *                    returns to zero.  bf16 block-128
 *                    kernels (single Q-blocks without a partial last block, and
 *                    Q-block pairs) take the queue; the other kernels use the bin
 *                    lists.  Forward calls with one such plan are serialised (each
 *                    waits for the plan's earlier calls on other streams). */
typedef enum {
  SA_ORDER_LPT = 0,
  SA_ORDER_NAIVE = 1,
  SA_ORDER_LPT_XCD = 2,
  SA_ORDER_LPT_DEVICE = 3,
  SA_ORDER_LPT_DYNAMIC = 4
} sa_order;
typedef enum { SA_LAYOUT_CONTIGUOUS = 0, SA_LAYOUT_STRIPED = 1 } sa_layout;
typedef enum { SA_KIND_BLOCK = 0, SA_KIND_TOPK = 1, SA_KIND_INDEX = 2 } sa_kind;

/* Shape of one attention problem (self-attention: Q and KV have length S).
 *  block     Q-block = KV-block size in tokens.  bf16: 64 or 128; f32: 64.
 *            nK = ceil(S/block) <= 2048.
 *  D         head dim.  bf16: 64 or 128; f32: 64 or 128.
 *  n_chunks  number of KV chunks (ring steps).  Contiguous layout: chunk c is
 *            KV blocks [c*nK/C, (c+1)*nK/C) and nK % C == 0, nK = ceil(S/block);
 *            the last block may be partial (S % block != 0).  Striped layout
 *            (striped attention, 6D notes section 2.3): chunk c holds tokens
 *            j with j % C == c; requires S % (block*C) == 0 and block/C a
 *            multiple of 32.
 *  scale     softmax scale; <= 0 selects 1/sqrt(D).
 *  q_pairs   non-zero: a work item is the Q-block pair (2p, 2p+1) of one
 *            (batch, head) instead of one Q-block, so every K/V tile the kernel
 *            stages feeds 256 query rows; the pair visits the union of its two
 *            mask rows' live tiles (a tile live for one row only is computed
 *            with zero probabilities for the other), and the LPT loads are
 *            those union counts.  Block plans, bf16, block 128, S % 128 == 0
 *            (else SA_ERR_UNSUPPORTED); both layouts.  Worth it where adjacent
 *            mask rows share most tiles (causal, banded masks).
 *  sb,sh,ss  element strides of the b, h and s axes of Q, K, V and O. */
typedef struct {
  int32_t B, H, S, D;
  int32_t block;
  int32_t n_chunks;
  int32_t layout; /* sa_layout */
  int32_t dtype;  /* sa_dtype */
  float scale;
  int32_t token_causal; /* non-zero: inside live tiles, key j is also dropped for query i when
                           j > i (token positions; striped chunks use each key's original
                           position), i.e. causal attention at token granularity */
  int32_t q_pairs;      /* non-zero: work items are Q-block pairs (see above) */
  int64_t sb, sh, ss;
} sa_problem;

/* Sparsity description handed to sparse_attn_plan.
 *  SA_KIND_BLOCK: mask  uint8 [B][H][nQ][nK], contiguous; non-zero = live.
 *                 Copied into the plan, so the caller may free it afterwards.
 *  SA_KIND_TOPK:  q, k  (problem layout and dtype); wq, wk [D][rank] row-major,
 *                 problem dtype (bf16 only).  The indexer (6D notes, section
 *                 7.1) computes I = (Q wq)(K wk)^T with the projections rounded
 *                 to bf16 and fp32 accumulation, and keeps, per query i,
 *                 the min(top_k, #candidates) keys that come first in the
 *                 order (I desc, key asc); candidates are j <= i when causal,
 *                 else all j.  rank == 32, top_k <= 512, S <= 65536.  The
 *                 order of the keys within a query's list is unspecified.
 *  SA_KIND_INDEX: idx int32 [B][H][S][top_k] key indices, count int32
 *                 [B][H][S] (0 <= count <= top_k); copied into the plan.  Every
 *                 idx[b,h,i,t], t < count, must lie in [0, S) (checked on the
 *                 host copy; the plan call is synchronous for this kind). */
typedef struct {
  int32_t kind; /* sa_kind */
  int32_t rank, top_k, causal;
  const uint8_t* mask;
  const void* q;
  const void* k;
  const void* wq;
  const void* wk;
  const int32_t* idx;
  const int32_t* count;
} sa_sparsity;

typedef struct sa_plan sa_plan; /* opaque; owned by the library */

typedef struct {
  int32_t kind, num_bins, order, n_chunks;
  int32_t nQ, nK, n_items, top_k;
  int64_t total_live;   /* BLOCK: live (Q-block, KV-block) tiles; TOPK/INDEX: selected pairs */
  int64_t load_sum;     /* sum of the full-range item loads (= total_live for BLOCK without
                           q_pairs; with q_pairs the sum of the pairs' union counts) */
  int64_t makespan;     /* max bin load of the full-range list */
  int64_t lower_bound;  /* max(max item load, ceil(load_sum / num_bins)) */
                        /* (SA_ORDER_LPT_DEVICE: the call waits for the plan to read these) */
  int32_t groups;       /* bin groups of SA_ORDER_LPT_XCD (XCDs), 1 otherwise */
  int32_t reserved;
} sa_plan_info;

/* Arrays that sparse_attn_plan_copy can export to host memory. */
typedef enum {
  SA_PLAN_ROW = 0,      /* int32 [B][H][nQ]   live tiles per Q-block (mask row sums)      */
  SA_PLAN_COL = 1,      /* int32 [B][H][nK]   live tiles per KV-block (mask column sums)  */
  SA_PLAN_CROW = 2,     /* int32 [B][H][C][nQ] per-chunk row counts (striped: = row)      */
  SA_PLAN_ITEMS = 3,    /* int32 [n_items]    item ids (b*H + h)*nQ + q, bins concatenated;
                                             q_pairs: (b*H + h)*nP + p, nP = ceil(nQ/2) */
  SA_PLAN_BIN_PTR = 4,  /* int32 [num_bins+1] offsets of each bin's list in ITEMS          */
  SA_PLAN_BIN_LOAD = 5, /* int64 [num_bins]   sum of item loads per bin                    */
  SA_PLAN_TOPK_IDX = 6, /* int32 [B][H][S][top_k] selected keys (TOPK/INDEX)              */
  SA_PLAN_TOPK_COUNT = 7, /* int32 [B][H][S]  number of selected keys                     */
  SA_PLAN_PAIR_ROW = 8,   /* int32 [B][H][nP]  q_pairs: live tiles of the union of rows 2p, 2p+1 */
  SA_PLAN_PAIR_CROW = 9,  /* int32 [B][H][C][nP] q_pairs: the same per chunk (striped: = PAIR_ROW) */
  SA_PLAN_LPT_ORDER = 10  /* int32 [n_items] SA_ORDER_LPT_DYNAMIC: the queue, items in LPT order      */
} sa_plan_array;

/* Build a plan.
 *  BLOCK: counts live tiles per mask row, column and per-chunk row on the GPU
 *  (row/column sums of the db-SP post, scenario 2), copies the row counts to
 *  the host and runs the LPT greedy of the same post (longest item to the
 *  least-loaded bin; ties: lower item id first, lower bin index) — or
 *  round-robin for SA_ORDER_NAIVE — over the full chunk range, and uploads
 *  the list for the persistent kernel.  The list of a single chunk c (used by
 *  sparse_attn_fwd over [c, c+1), one ring step) is built from the same counts
 *  on its first use (that forward call, which then waits for its upload once,
 *  or sparse_attn_plan_copy).  This kind synchronises the stream once, except
 *  with SA_ORDER_LPT_DEVICE, where every list is made on the GPU behind the
 *  popcount and the call returns without waiting.
 *  TOPK: runs the indexer and top-k selection on the GPU; asynchronous.
 *  All kinds: the plan's device arrays are written on `stream`; sparse_attn_fwd
 *  makes its own stream wait for them, so a plan may be built on a side stream
 *  (for instance the next step's plan while the current step computes).
 *  num_bins: persistent workgroups; 0 picks one per resident workgroup slot
 *  (bf16: 1 per compute unit for block 128, 2 for block 64; f32: 1).
 *  out (host): receives the plan.  Returns SA_ERR_NOMEM if the plan's device
 *  buffers cannot be allocated. */
sa_status sparse_attn_plan(const sa_problem* prob, const sa_sparsity* sp, int32_t num_bins,
                           int32_t order, sa_plan** out, hipStream_t stream);

/* Run attention under a plan over KV chunks [chunk_begin, chunk_end).
 *  Full mode (o != NULL): O = softmax-weighted sum over the live keys of the
 *  chunk range, normalised, written in the problem dtype through the strides.
 *  Partial mode (o == NULL): writes one fp32 (O, m, l) partial per chunk of
 *  the range (see the conventions above); o_part, m_part, l_part must all be
 *  non-NULL.  This is the ring step's flash_attention of the 6D notes,
 *  section 2.1.  TOPK/INDEX plans: full mode only, chunk range [0, 1).
 *  trace (nullable): int64 [n_items_of_list][4] = {start, end, (xcc_id << 32)
 *  | hw_id, (bin << 32) | item}, timestamps from the 100 MHz real-time clock,
 *  in list order.  The list is the full-range one, or the chunk's own list
 *  when the range is a single chunk.  Allocates nothing. */
sa_status sparse_attn_fwd(const sa_plan* plan, const void* q, const void* k, const void* v,
                          int32_t chunk_begin, int32_t chunk_end, void* o, float* o_part,
                          float* m_part, float* l_part, int64_t* trace, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 *  tight serving loops, harnesses that forbid allocation): plan and forward in
 *  one call that allocates nothing.  The result equals that of
 *  sparse_attn_plan(prob, SA_KIND_BLOCK mask, num_bins, SA_ORDER_LPT_DEVICE)
 *  followed by sparse_attn_fwd over [chunk_begin, chunk_end) with the same o or
 *  (o_part, m_part, l_part).  The counts and the work list are kept in a
 *  2 MiB device array of the library, one per GPU, held until the process
 *  ends; calls that overlap on one GPU (other streams, other host threads)
 *  race on it, calls ordered on one stream do not.  All launches go to
 *  `stream`; the call never waits for the device.
 *  mask: uint8 [B][H][nQ][nK] as for a block plan, 16-byte aligned, read on
 *  the stream (keep it alive until the work is done); it is not copied.
 *  Limits: at most 16384 work items (B*H*nQ, or B*H*ceil(nQ/2) with q_pairs)
 *  and num_bins <= 1024 (as for SA_ORDER_LPT_DEVICE), and the counts and list
 *  must fit the array (about B*H*nQ*(n_chunks + 3)*4 bytes, half as much
 *  again with q_pairs); beyond them SA_ERR_UNSUPPORTED.  Other arguments as for
 *  sparse_attn_plan and sparse_attn_fwd. */
sa_status sparse_attn_fwd_noalloc(const sa_problem* prob, const uint8_t* mask, int32_t num_bins, const void* q,
                                  const void* k, const void* v, int32_t chunk_begin, int32_t chunk_end, void* o,
                                  float* o_part, float* m_part, float* l_part, hipStream_t stream);

/* Online-softmax merge of n_parts partials (6D notes, section 2.1): per row,
 *  the parts are taken in order into one running (O, m, l); at each step the
 *  running maximum becomes the larger of m and m_p and both sides' O and l are
 *  scaled by exp(their maximum - the new maximum) before they are added; the
 *  result is O / l.  Parts with m_p = -inf add nothing and their O_p is not read.
 *  o_parts, m_parts, l_parts (host arrays of n_parts device pointers): O_p is
 *  fp32 [rows][D], m_p and l_p fp32 [rows].  o_out: [rows][D] dense in out_dtype.
 *  lse_out (nullable): fp32 [rows], m + log(l), -inf for empty rows.
 *  1 <= n_parts <= 64, D in {64, 128}.  Allocates nothing. */
sa_status chunk_merge(int32_t n_parts, const float* const* o_parts, const float* const* m_parts,
                      const float* const* l_parts, int64_t rows, int32_t D, void* o_out,
                      int32_t out_dtype, float* lse_out, hipStream_t stream);

/* Summary of a plan (host output). */
sa_status sparse_attn_plan_info(const sa_plan* plan, sa_plan_info* out);

/* Copy one of the plan's arrays to host memory dst (n_elems elements of the
 * array's type).  chunk selects the list for ITEMS / BIN_PTR / BIN_LOAD /
 * LPT_ORDER: -1 is the full-range list, c in [0, C) the list of chunk c.
 * Synchronous. */
sa_status sparse_attn_plan_copy(const sa_plan* plan, int32_t what, int32_t chunk, void* dst,
                                int64_t n_elems);

/* Host-only LPT / round-robin assignment, the same code the plan uses.
 *  loads (host) [n] non-negative; items_out (host) [n]; bin_ptr_out (host)
 *  [m+1]; bin_load_out (host, nullable) [m].  Touches no GPU. */
sa_status sparse_attn_assign_host(const int64_t* loads, int32_t n, int32_t m, int32_t order,
                                  int32_t* items_out, int32_t* bin_ptr_out, int64_t* bin_load_out);

/* Host-only two-level LPT (SA_ORDER_LPT_XCD), the same code the plan uses:
 *  loads (host) [n_heads * items_per_head], item i = head * items_per_head + q;
 *  heads go to `groups` bin groups (bins b with b mod groups == g), then each
 *  group's items (its heads in assignment order, then q) to its bins by LPT.
 *  Plain LPT when groups <= 1 or m is not a multiple of groups.  Outputs as in
 *  sparse_attn_assign_host.  Touches no GPU. */
sa_status sparse_attn_assign_host_grouped(const int64_t* loads, int32_t n_heads, int32_t items_per_head, int32_t m,
                                          int32_t groups, int32_t* items_out, int32_t* bin_ptr_out,
                                          int64_t* bin_load_out);

/* Free a plan.  NULL is a no-op.  Does not wait for the device: the plan's
 *  device buffers go to a per-device cache of the library together with events
 *  that mark the end of the plan's own construction and of the last
 *  sparse_attn_fwd call on every stream that used it; a later plan that takes a
 *  buffer makes its stream wait for those events, so buffers are reused only
 *  after every kernel that read them has finished (no host synchronisation; a
 *  step that re-plans a runtime mask allocates nothing once the cache is warm).
 *  The call waits only for the plan's own construction work to finish (it
 *  frees the host arrays that work may read from).  The plan must not be used
 *  afterwards; kernels already enqueued with it may still be running. */
void sparse_attn_plan_destroy(sa_plan* plan);

/* Static description of a status code. */
const char* sa_status_string(int32_t status);

/* Text of the last error raised on this thread ("" if none). */
const char* sa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H */
