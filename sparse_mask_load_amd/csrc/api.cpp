// Host side of the C ABI: validation, the plan object, launches, error mapping.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"
#include "sparse_attn.h"

struct sa_plan {
  sa_problem prob{};
  int32_t kind = SA_KIND_BLOCK;
  int32_t num_bins = 0;
  int32_t order = SA_ORDER_LPT;
  int32_t groups = 1;  // bin groups of SA_ORDER_LPT_XCD (one per XCD), else 1
  int32_t nQ = 0, nK = 0, n_items = 0, top_k = 0, rank = 0, causal = 0;
  int32_t nI = 0;        // items per (batch, head): nQ, or the pair count ceil(nQ/2) with q_pairs
  bool q_pairs = false;  // items are Q-block pairs
  int device = 0;
  int32_t n_xcd = 1;  // L2 domains (XCDs) of the device
  // BLOCK
  uint8_t* d_mask = nullptr;         // [B][H][nQ][nK] copy of the caller's mask
  int32_t* d_row = nullptr;          // [B*H*nQ]
  int32_t* d_col = nullptr;          // [B*H*nK]
  int32_t* d_crow = nullptr;         // [B*H*C*nQ]
  int32_t* d_prow = nullptr;         // q_pairs: [B*H*nI] union counts of each pair
  int32_t* d_pcrow = nullptr;        // q_pairs: [B*H*C*nI] the same per chunk
  int32_t* d_items = nullptr;        // [(C+1)][n_items]: list 0 = full range, list 1+c = chunk c
  int32_t* d_bin_ptr = nullptr;      // [(C+1)][num_bins+1]
  // SA_ORDER_LPT_DEVICE: every list is made on the device; loads and statistics stay there
  bool device_lists = false;
  int64_t* d_bin_load = nullptr;     // [(C+1)][num_bins]
  int64_t* d_stats = nullptr;        // [(C+1)][4]: load sum, max item load, makespan, lower bound
  std::vector<int32_t> h_items, h_bin_ptr;
  std::vector<int64_t> h_bin_load;   // [(C+1)][num_bins]
  // The full-range list is built by the plan call; the list of chunk c (used by forward calls
  // over that chunk alone, as in one ring step) is built on first use from the host counts.
  std::vector<int32_t> h_crow;       // [B*H*C*nI] per-chunk item loads (row or pair counts)
  std::unique_ptr<std::once_flag[]> list_once;
  std::unique_ptr<bool[]> list_uploaded;
  std::mutex upload_mutex;
  int64_t total_live = 0, load_sum = 0, makespan = 0, lower_bound = 0;
  // TOPK / INDEX
  // SA_ORDER_LPT_DYNAMIC: each list's queue (items in LPT order) and its two counters
  int32_t* d_lpt_order = nullptr;    // [(C+1)][n_items]
  int32_t* d_dyn_ctr = nullptr;      // [(C+1)][sa::kQueueCtrs]
  int32_t* d_idx = nullptr;          // [B][H][S][top_k]
  int32_t* d_count = nullptr;        // [B][H][S]
  __bf16* d_qp = nullptr;            // [B][H][S][rank]
  __bf16* d_kp = nullptr;
  float* d_mom = nullptr;            // [B][H][S/128 + 1][rank + rank^2]
  // recorded on the plan's stream once its device arrays are complete; every forward call
  // makes its own stream wait for it, so a plan may be built on a side stream
  hipEvent_t ready = nullptr;
  // device buffers of the plan (pointer, capacity in bytes), returned to the buffer cache
  std::vector<std::pair<void*, size_t>> allocs;
  // one event per stream that ran a forward call with the plan, re-recorded after each call
  std::mutex use_mutex;
  std::mutex queue_mutex;  // SA_ORDER_LPT_DYNAMIC: held by a forward call from its waits to its use record
  std::vector<std::pair<hipStream_t, hipEvent_t>> uses;
};

namespace {

thread_local std::string g_last_error;

sa_status fail(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sa_status hip_fail(hipError_t e, const char* what) {
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define SA_HIP(call)                                   \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return hip_fail(e_, #call);  \
  } while (0)

int max_tiles_per_row(int) { return sa::kMaxTilesPerRow; }

sa_status validate_problem(const sa_problem* p, bool block_kind) {
  if (!p) return fail(SA_ERR_INVALID, "problem is NULL");
  if (p->B <= 0 || p->H <= 0 || p->S <= 0 || p->D <= 0)
    return fail(SA_ERR_INVALID, "B, H, S, D must be positive (got %d, %d, %d, %d)", p->B, p->H, p->S, p->D);
  if (p->dtype != SA_F32 && p->dtype != SA_BF16) return fail(SA_ERR_INVALID, "unknown dtype %d", p->dtype);
  if (p->D != 64 && p->D != 128) return fail(SA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", p->D);
  if (p->sb <= 0 || p->sh <= 0 || p->ss < p->D)
    return fail(SA_ERR_INVALID, "strides must be positive with ss >= D (got %lld, %lld, %lld)",
                (long long)p->sb, (long long)p->sh, (long long)p->ss);
  if ((p->ss % 8) || (p->sh % 8) || (p->sb % 8))
    return fail(SA_ERR_UNSUPPORTED, "strides must be multiples of 8 elements (16-byte rows)");
  if (!block_kind) {
    if (p->token_causal)
      return fail(SA_ERR_INVALID, "token_causal applies to block plans (top-k and index plans take causality "
                                  "from their key selection)");
    if (p->q_pairs) return fail(SA_ERR_INVALID, "q_pairs applies to block plans");
    return SA_OK;
  }
  if (p->dtype == SA_BF16 && p->block != 64 && p->block != 128)
    return fail(SA_ERR_UNSUPPORTED, "bf16 block %d (supported: 64, 128)", p->block);
  if (p->dtype == SA_F32 && p->block != 64)
    return fail(SA_ERR_UNSUPPORTED, "f32 block %d (supported: 64)", p->block);
  const int nK = (p->S + p->block - 1) / p->block;
  if (nK > max_tiles_per_row(p->block))
    return fail(SA_ERR_UNSUPPORTED, "S/block = %d exceeds %d tiles per row", nK, max_tiles_per_row(p->block));
  if (p->n_chunks < 1 || p->n_chunks > sa::kMaxChunks)
    return fail(SA_ERR_INVALID, "n_chunks %d outside [1, %d]", p->n_chunks, sa::kMaxChunks);
  if (nK % p->n_chunks) return fail(SA_ERR_INVALID, "nK = %d not divisible by n_chunks %d", nK, p->n_chunks);
  if (p->layout == SA_LAYOUT_STRIPED) {
    if (p->S % (p->block * p->n_chunks))
      return fail(SA_ERR_INVALID, "striped layout needs S %% (block * n_chunks) == 0");
    if ((p->block / p->n_chunks) % 32 || p->block % p->n_chunks)
      return fail(SA_ERR_UNSUPPORTED, "striped layout needs block / n_chunks to be a multiple of 32");
  } else if (p->layout != SA_LAYOUT_CONTIGUOUS) {
    return fail(SA_ERR_INVALID, "unknown layout %d", p->layout);
  }
  if (p->q_pairs && (p->dtype != SA_BF16 || p->block != 128 || p->S % 128))
    return fail(SA_ERR_UNSUPPORTED, "q_pairs needs bf16, block 128 and S %% 128 == 0");
  return SA_OK;
}

float effective_scale(const sa_problem& p) { return p.scale > 0.f ? p.scale : 1.f / std::sqrt((float)p.D); }

// Device buffers of destroyed plans, kept per device for reuse by later plans (a step that
// re-plans a runtime mask then allocates nothing once the cache holds its buffers).  A buffer
// goes back with the events that mark the end of every use its plan made of it: the plan's
// own construction (its ready event) and the last forward call on each stream.  A plan that
// takes the buffer makes its stream wait for those events first, so reuse is ordered on the
// device and neither destroying nor re-planning waits on the host.
struct UseEvents {
  std::vector<hipEvent_t> ev;
  ~UseEvents() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};
struct CachedBuf {
  int device;
  void* ptr;
  size_t bytes;
  std::shared_ptr<UseEvents> uses;
};
constexpr size_t kCacheMaxBytes = size_t(2) << 30;  // beyond this, returned buffers are freed
constexpr size_t kCacheMaxBufs = 512;
struct BufCache {
  std::mutex mu;
  std::vector<CachedBuf> bufs;
  size_t bytes = 0;
};
BufCache& buf_cache() {
  static BufCache* c = new BufCache();  // never destroyed: no HIP calls during process teardown
  return *c;
}

// Device buffer of at least n elements for plan P, from the cache (ordered after its previous
// users on `stream`) or from hipMalloc.
template <typename T>
sa_status dalloc(sa_plan* P, T** ptr, size_t n, hipStream_t stream) {
  *ptr = nullptr;
  const size_t need = ((std::max<size_t>(n, 1) * sizeof(T)) + 255) & ~size_t(255);
  CachedBuf hit{-1, nullptr, 0, nullptr};
  {
    BufCache& c = buf_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    size_t best = SIZE_MAX;
    for (size_t i = 0; i < c.bufs.size(); ++i) {
      const CachedBuf& b = c.bufs[i];
      if (b.device == P->device && b.bytes >= need && b.bytes <= 2 * need + 4096 &&
          (best == SIZE_MAX || b.bytes < c.bufs[best].bytes))
        best = i;
    }
    if (best != SIZE_MAX) {
      hit = c.bufs[best];
      c.bufs[best] = c.bufs.back();
      c.bufs.pop_back();
      c.bytes -= hit.bytes;
    }
  }
  if (hit.ptr) {
    P->allocs.emplace_back(hit.ptr, hit.bytes);
    for (hipEvent_t e : hit.uses->ev) {
      const hipError_t err = hipStreamWaitEvent(stream, e, 0);
      if (err != hipSuccess) return hip_fail(err, "hipStreamWaitEvent on a reused plan buffer");
    }
    *ptr = (T*)hit.ptr;
    return SA_OK;
  }
  hipError_t e = hipMalloc((void**)ptr, need);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *ptr = nullptr;
    return fail(SA_ERR_NOMEM, "hipMalloc of %zu bytes failed: %s", need, hipGetErrorString(e));
  }
  P->allocs.emplace_back((void*)*ptr, need);
  return SA_OK;
}

// Frees a plan without waiting for the device: its buffers go to the cache together with
// the events of their last uses (buffers beyond the cache's limits are freed once those
// events have completed).
void free_plan(sa_plan* p) {
  if (!p) return;
  auto uses = std::make_shared<UseEvents>();
  if (p->ready) {
    // host copies the plan uploaded from are freed below: let its own work finish first
    (void)hipEventSynchronize(p->ready);
    uses->ev.push_back(p->ready);
  }
  for (auto& u : p->uses) uses->ev.push_back(u.second);
  std::vector<std::pair<void*, size_t>> spill;
  {
    BufCache& c = buf_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    for (auto& a : p->allocs) {
      if (c.bytes + a.second <= kCacheMaxBytes && c.bufs.size() < kCacheMaxBufs) {
        c.bufs.push_back(CachedBuf{p->device, a.first, a.second, uses});
        c.bytes += a.second;
      } else {
        spill.push_back(a);
      }
    }
  }
  if (!spill.empty()) {
    for (hipEvent_t e : uses->ev) (void)hipEventSynchronize(e);
    for (auto& a : spill) (void)hipFree(a.first);
  }
  delete p;
}

int default_bins(const sa_problem& p, int device) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
    cus = 256;
  // one bin per resident workgroup: the bf16 kernel keeps 1 (block 128) or 2 (block 64) per CU
  return p.dtype == SA_BF16 ? cus * sa::attn_bf16_wg_per_cu(p.block) : cus;
}

// One work list of a block plan from per-item loads, in the plan's order.
void assign_list(const sa_plan* P, const int64_t* loads, int32_t* items, int32_t* bin_ptr, int64_t* bin_load) {
  const int m = P->num_bins, n = P->n_items;
  if (P->order == SA_ORDER_LPT_XCD)
    sa::assign_grouped(loads, n / P->nI, P->nI, m, P->groups, items, bin_ptr, bin_load);
  else
    sa::assign(loads, n, m, P->order, items, bin_ptr, bin_load);
}

// Number of XCDs (L2 domains) of the device; the persistent workgroups are dispatched to
// them round-robin, so workgroup b runs on XCD b mod this count.
int xcd_count(int device) {
  int x = 0;
  if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, device) != hipSuccess || x <= 0) x = 1;
  return x;
}

sa_status plan_block(sa_plan* P, const sa_sparsity* sp, hipStream_t stream) {
  const sa_problem& pr = P->prob;
  const int BH = pr.B * pr.H, C = pr.n_chunks;
  P->nQ = P->nK = (pr.S + pr.block - 1) / pr.block;
  const int nQ = P->nQ, nK = P->nK;
  P->q_pairs = pr.q_pairs != 0;
  P->nI = P->q_pairs ? (nQ + 1) / 2 : nQ;
  const int nI = P->nI;
  P->n_items = BH * nI;
  if (!sp->mask) return fail(SA_ERR_INVALID, "mask is NULL");
  const size_t mask_bytes = (size_t)BH * nQ * nK;
  sa_status st;
  if ((st = dalloc(P, &P->d_mask, mask_bytes, stream)) || (st = dalloc(P, &P->d_row, (size_t)BH * nQ, stream)) ||
      (st = dalloc(P, &P->d_col, (size_t)BH * nK, stream)) || (st = dalloc(P, &P->d_crow, (size_t)BH * C * nQ, stream)) ||
      (st = dalloc(P, &P->d_items, (size_t)(C + 1) * P->n_items, stream)) ||
      (st = dalloc(P, &P->d_bin_ptr, (size_t)(C + 1) * (P->num_bins + 1), stream)))
    return st;
  if (P->q_pairs && ((st = dalloc(P, &P->d_prow, (size_t)BH * nI, stream)) ||
                     (st = dalloc(P, &P->d_pcrow, (size_t)BH * C * nI, stream))))
    return st;
  SA_HIP(hipMemcpyAsync(P->d_mask, sp->mask, mask_bytes, hipMemcpyDeviceToDevice, stream));
  SA_HIP(sa::launch_popcount(P->d_mask, BH, nQ, nK, C, pr.layout, P->d_row, P->d_col, P->d_crow, stream, P->d_prow,
                             P->d_pcrow));
  // item loads: mask row counts, or the union counts of Q-block pairs
  const int32_t* d_load = P->q_pairs ? P->d_prow : P->d_row;
  const int32_t* d_cload = P->q_pairs ? P->d_pcrow : P->d_crow;
  if (P->order == SA_ORDER_LPT_DEVICE || P->order == SA_ORDER_LPT_DYNAMIC) {
    // every list on the device, right behind the popcount: nothing waits for the host
    if ((st = dalloc(P, &P->d_bin_load, (size_t)(C + 1) * P->num_bins, stream)) ||
        (st = dalloc(P, &P->d_stats, (size_t)(C + 1) * 4, stream)))
      return st;
    const bool dyn = P->order == SA_ORDER_LPT_DYNAMIC;
    if (dyn && ((st = dalloc(P, &P->d_lpt_order, (size_t)(C + 1) * P->n_items, stream)) ||
                (st = dalloc(P, &P->d_dyn_ctr, (size_t)(C + 1) * sa::kQueueCtrs, stream))))
      return st;
    SA_HIP(sa::launch_plan_rounds(d_load, d_cload, BH, nI, C, P->num_bins, P->d_items, P->d_bin_ptr,
                                  P->d_bin_load, P->d_stats, stream, 0, -1, P->d_lpt_order, P->d_dyn_ctr));
    P->device_lists = true;
    return SA_OK;
  }
  std::vector<int32_t> row((size_t)BH * nI), crow((size_t)BH * C * nI), qrow;
  SA_HIP(hipMemcpyAsync(row.data(), d_load, row.size() * 4, hipMemcpyDeviceToHost, stream));
  SA_HIP(hipMemcpyAsync(crow.data(), d_cload, crow.size() * 4, hipMemcpyDeviceToHost, stream));
  if (P->q_pairs) {
    qrow.resize((size_t)BH * nQ);
    SA_HIP(hipMemcpyAsync(qrow.data(), P->d_row, qrow.size() * 4, hipMemcpyDeviceToHost, stream));
  }
  SA_HIP(hipStreamSynchronize(stream));

  const int m = P->num_bins, n = P->n_items;
  P->h_items.assign((size_t)(C + 1) * n, 0);
  P->h_bin_ptr.assign((size_t)(C + 1) * (m + 1), 0);
  P->h_bin_load.assign((size_t)(C + 1) * m, 0);
  P->h_crow = std::move(crow);
  P->list_once.reset(new std::once_flag[C + 1]);
  P->list_uploaded.reset(new bool[C + 1]());
  {
    std::vector<int64_t> loads(row.begin(), row.end());
    assign_list(P, loads.data(), P->h_items.data(), P->h_bin_ptr.data(), P->h_bin_load.data());
  }
  std::call_once(P->list_once[0], [] {});  // list 0 is built
  int64_t sum = 0, pmax = 0;
  for (int i = 0; i < n; ++i) {
    sum += row[i];
    pmax = std::max<int64_t>(pmax, row[i]);
  }
  P->load_sum = sum;
  P->total_live = sum;  // every live tile belongs to exactly one Q-block row
  if (P->q_pairs) {
    P->total_live = 0;
    for (int32_t x : qrow) P->total_live += x;
  }
  P->makespan = *std::max_element(P->h_bin_load.begin(), P->h_bin_load.begin() + m);
  P->lower_bound = std::max<int64_t>(pmax, (sum + m - 1) / m);
  SA_HIP(hipMemcpyAsync(P->d_items, P->h_items.data(), (size_t)n * 4, hipMemcpyHostToDevice, stream));
  SA_HIP(hipMemcpyAsync(P->d_bin_ptr, P->h_bin_ptr.data(), (size_t)(m + 1) * 4, hipMemcpyHostToDevice, stream));
  P->list_uploaded[0] = true;
  return SA_OK;
}

// Host lists of chunk `list - 1` (LPT or round-robin over the chunk's row counts), once.
void build_chunk_list(sa_plan* P, int list) {
  std::call_once(P->list_once[list], [P, list] {
    const int C = P->prob.n_chunks, nI = P->nI, n = P->n_items, m = P->num_bins, c = list - 1;
    std::vector<int64_t> loads(n);
    for (int i = 0; i < n; ++i) loads[i] = P->h_crow[((size_t)(i / nI) * C + c) * nI + i % nI];
    assign_list(P, loads.data(), P->h_items.data() + (size_t)list * n, P->h_bin_ptr.data() + (size_t)list * (m + 1),
                P->h_bin_load.data() + (size_t)list * m);
  });
}

// Device copy of list `list` (built on the host first if needed), ordered on `stream`.
sa_status ensure_list_on_device(sa_plan* P, int list, hipStream_t stream) {
  if (P->device_lists) return SA_OK;  // made on the device by the plan call
  build_chunk_list(P, list);
  std::lock_guard<std::mutex> lock(P->upload_mutex);
  if (P->list_uploaded[list]) return SA_OK;
  const int n = P->n_items, m = P->num_bins;
  SA_HIP(hipMemcpyAsync(P->d_items + (size_t)list * n, P->h_items.data() + (size_t)list * n, (size_t)n * 4,
                        hipMemcpyHostToDevice, stream));
  SA_HIP(hipMemcpyAsync(P->d_bin_ptr + (size_t)list * (m + 1), P->h_bin_ptr.data() + (size_t)list * (m + 1),
                        (size_t)(m + 1) * 4, hipMemcpyHostToDevice, stream));
  // later calls on other streams must not race the copy: wait for it here (first use only)
  SA_HIP(hipStreamSynchronize(stream));
  P->list_uploaded[list] = true;
  return SA_OK;
}

// Marks the end of a forward call's use of the plan's buffers on `stream` (the plan's cache
// entry waits for it before the buffers serve another plan).
sa_status note_use(const sa_plan* cP, hipStream_t stream) {
  sa_plan* P = const_cast<sa_plan*>(cP);  // logically const: only the use bookkeeping changes
  std::lock_guard<std::mutex> lock(P->use_mutex);
  hipEvent_t ev = nullptr;
  for (auto& u : P->uses)
    if (u.first == stream) ev = u.second;
  if (!ev) {
    SA_HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    P->uses.emplace_back(stream, ev);
  }
  SA_HIP(hipEventRecord(ev, stream));
  return SA_OK;
}

sa_status plan_topk(sa_plan* P, const sa_sparsity* sp, hipStream_t stream) {
  const sa_problem& pr = P->prob;
  if (pr.dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "top-k kinds are bf16 only");
  if (sp->top_k <= 0 || sp->top_k > 2048) return fail(SA_ERR_UNSUPPORTED, "top_k %d outside [1, 2048]", sp->top_k);
  P->top_k = sp->top_k;
  P->causal = sp->causal ? 1 : 0;
  const size_t rows = (size_t)pr.B * pr.H * pr.S;
  P->n_items = (int32_t)rows;
  sa_status st;
  if ((st = dalloc(P, &P->d_idx, rows * P->top_k, stream)) || (st = dalloc(P, &P->d_count, rows, stream))) return st;
  if (P->kind == SA_KIND_INDEX) {
    if (!sp->idx || !sp->count) return fail(SA_ERR_INVALID, "idx or count is NULL");
    std::vector<int32_t> idx(rows * P->top_k), cnt(rows);
    SA_HIP(hipMemcpyAsync(idx.data(), sp->idx, idx.size() * 4, hipMemcpyDeviceToHost, stream));
    SA_HIP(hipMemcpyAsync(cnt.data(), sp->count, cnt.size() * 4, hipMemcpyDeviceToHost, stream));
    SA_HIP(hipStreamSynchronize(stream));
    int64_t tot = 0;
    for (size_t r = 0; r < rows; ++r) {
      if (cnt[r] < 0 || cnt[r] > P->top_k) return fail(SA_ERR_INVALID, "count[%zu] = %d outside [0, top_k]", r, cnt[r]);
      for (int t = 0; t < cnt[r]; ++t) {
        const int32_t j = idx[r * P->top_k + t];
        if (j < 0 || j >= pr.S) return fail(SA_ERR_INVALID, "idx[%zu][%d] = %d outside [0, S)", r, t, j);
      }
      tot += cnt[r];
    }
    P->total_live = P->load_sum = tot;
    SA_HIP(hipMemcpyAsync(P->d_idx, sp->idx, idx.size() * 4, hipMemcpyDeviceToDevice, stream));
    SA_HIP(hipMemcpyAsync(P->d_count, sp->count, cnt.size() * 4, hipMemcpyDeviceToDevice, stream));
    SA_HIP(hipStreamSynchronize(stream));
    return SA_OK;
  }
  if (!sp->q || !sp->k || !sp->wq || !sp->wk) return fail(SA_ERR_INVALID, "q, k, wq or wk is NULL");
  if (sp->rank != 32) return fail(SA_ERR_UNSUPPORTED, "indexer rank %d (supported: 32)", sp->rank);
  if (P->top_k > sa::kIndexerMaxTopK)
    return fail(SA_ERR_UNSUPPORTED, "indexer top_k %d above %d", P->top_k, sa::kIndexerMaxTopK);
  if (pr.S > 65536) return fail(SA_ERR_UNSUPPORTED, "indexer sequence length %d above 65536", pr.S);
  P->rank = sp->rank;
  const size_t mom = (size_t)pr.B * pr.H * ((size_t)(pr.S + sa::kMomGroup - 1) / sa::kMomGroup + 1) * sa::kMomEntry;
  if ((st = dalloc(P, &P->d_qp, rows * P->rank, stream)) || (st = dalloc(P, &P->d_kp, rows * P->rank, stream)) ||
      (st = dalloc(P, &P->d_mom, mom, stream)))
    return st;
  sa::IndexerArgs a{};
  a.q = sp->q; a.k = sp->k; a.wq = sp->wq; a.wk = sp->wk;
  a.qp = P->d_qp; a.kp = P->d_kp; a.mom = P->d_mom; a.idx = P->d_idx; a.count = P->d_count;
  a.B = pr.B; a.H = pr.H; a.S = pr.S; a.D = pr.D; a.rank = P->rank; a.top_k = P->top_k; a.causal = P->causal;
  a.sb = pr.sb; a.sh = pr.sh; a.ss = pr.ss;
  a.n_xcd = P->n_xcd;
  SA_HIP(sa::launch_indexer(a, stream));
  // selected pairs are known in closed form: min(top_k, #candidates) per query
  int64_t tot = 0;
  for (int i = 0; i < pr.S; ++i) tot += std::min<int64_t>(P->top_k, P->causal ? i + 1 : pr.S);
  P->total_live = P->load_sum = tot * pr.B * pr.H;
  return SA_OK;
}

}  // namespace

namespace sa {

sa_status set_error(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
sa_status validate_block_problem(const sa_problem* p) { return validate_problem(p, true); }
int default_num_bins(const sa_problem& p, int device) { return default_bins(p, device); }
float softmax_scale(const sa_problem& p) { return effective_scale(p); }

}  // namespace sa

extern "C" {

sa_status sparse_attn_plan(const sa_problem* prob, const sa_sparsity* sp, int32_t num_bins, int32_t order,
                           sa_plan** out, hipStream_t stream) {
  if (!out) return fail(SA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!sp) return fail(SA_ERR_INVALID, "sparsity is NULL");
  if (sp->kind != SA_KIND_BLOCK && sp->kind != SA_KIND_TOPK && sp->kind != SA_KIND_INDEX)
    return fail(SA_ERR_INVALID, "unknown sparsity kind %d", sp->kind);
  sa_status st = validate_problem(prob, sp->kind == SA_KIND_BLOCK);
  if (st) return st;
  if (order != SA_ORDER_LPT && order != SA_ORDER_NAIVE && order != SA_ORDER_LPT_XCD && order != SA_ORDER_LPT_DEVICE &&
      order != SA_ORDER_LPT_DYNAMIC)
    return fail(SA_ERR_INVALID, "unknown order %d", order);
  const bool device_order = order == SA_ORDER_LPT_DEVICE || order == SA_ORDER_LPT_DYNAMIC;
  if (order == SA_ORDER_LPT_DYNAMIC && sp->kind != SA_KIND_BLOCK)
    return fail(SA_ERR_INVALID, "the run-time order exists only for block plans");
  if (num_bins < 0) return fail(SA_ERR_INVALID, "num_bins %d < 0", num_bins);
  if (device_order && sp->kind == SA_KIND_BLOCK) {
    const int64_t nQ = (prob->S + prob->block - 1) / prob->block;
    const int64_t n_items = (int64_t)prob->B * prob->H * (prob->q_pairs ? (nQ + 1) / 2 : nQ);
    if (n_items > sa::kDevicePlanMaxItems || num_bins > sa::kDevicePlanMaxBins)
      return fail(SA_ERR_UNSUPPORTED, "device planning takes at most %d items and %d bins (got %lld, %d)",
                  sa::kDevicePlanMaxItems, sa::kDevicePlanMaxBins, (long long)n_items, num_bins);
  }
  sa_plan* P = new (std::nothrow) sa_plan();
  if (!P) return fail(SA_ERR_NOMEM, "host allocation of the plan failed");
  P->prob = *prob;
  P->kind = sp->kind;
  P->order = order;
  if (hipGetDevice(&P->device) != hipSuccess) {
    delete P;
    return fail(SA_ERR_HIP, "hipGetDevice failed");
  }
  P->num_bins = num_bins ? num_bins : default_bins(*prob, P->device);
  P->n_xcd = xcd_count(P->device);
  if (device_order && sp->kind == SA_KIND_BLOCK && P->num_bins > sa::kDevicePlanMaxBins) {
    delete P;  // the default bin count of this device is above the planner's limit
    return fail(SA_ERR_UNSUPPORTED, "device planning takes at most %d bins (default here: %d)",
                sa::kDevicePlanMaxBins, P->num_bins);
  }
  if (order == SA_ORDER_LPT_XCD) {
    P->groups = xcd_count(P->device);
    if (P->num_bins % P->groups != 0) P->groups = 1;  // groups must split the bins evenly
  }
  st = sp->kind == SA_KIND_BLOCK ? plan_block(P, sp, stream) : plan_topk(P, sp, stream);
  if (!st) {
    hipError_t e = hipEventCreateWithFlags(&P->ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(P->ready, stream);
    if (e != hipSuccess) st = hip_fail(e, "plan completion event");
  }
  if (st) {
    std::string keep = g_last_error;
    free_plan(P);
    g_last_error = keep;
    return st;
  }
  *out = P;
  return SA_OK;
}

sa_status sparse_attn_fwd(const sa_plan* P, const void* q, const void* k, const void* v, int32_t chunk_begin,
                          int32_t chunk_end, void* o, float* o_part, float* m_part, float* l_part, int64_t* trace,
                          hipStream_t stream) {
  if (!P) return fail(SA_ERR_INVALID, "plan is NULL");
  if (!q || !k || !v) return fail(SA_ERR_INVALID, "q, k or v is NULL");
  const sa_problem& pr = P->prob;
  if (P->ready) SA_HIP(hipStreamWaitEvent(stream, P->ready, 0));  // the plan may come from another stream
  if (P->kind != SA_KIND_BLOCK) {
    if (!o) return fail(SA_ERR_INVALID, "top-k plans support full mode only (o must be non-NULL)");
    if (chunk_begin != 0 || chunk_end != 1) return fail(SA_ERR_INVALID, "top-k plans take the chunk range [0, 1)");
    sa::GatherArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.idx = P->d_idx; a.count = P->d_count;
    a.B = pr.B; a.H = pr.H; a.S = pr.S; a.D = pr.D; a.top_k = P->top_k;
    a.sb = pr.sb; a.sh = pr.sh; a.ss = pr.ss;
    a.scale_log2 = effective_scale(pr) * 1.4426950408889634f;
    SA_HIP(sa::launch_gather_attn(a, stream));
    return note_use(P, stream);
  }
  if (chunk_begin < 0 || chunk_end > pr.n_chunks || chunk_begin >= chunk_end)
    return fail(SA_ERR_INVALID, "chunk range [%d, %d) not inside [0, %d)", chunk_begin, chunk_end, pr.n_chunks);
  if (!o && (!o_part || !m_part || !l_part))
    return fail(SA_ERR_INVALID, "partial mode needs o_part, m_part and l_part");
  const int list = (chunk_end - chunk_begin == 1) ? 1 + chunk_begin : 0;
  if (list > 0) {
    const sa_status st = ensure_list_on_device(const_cast<sa_plan*>(P), list, stream);
    if (st) return st;
  }
  sa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.o_part = o ? nullptr : o_part;
  a.m_part = o ? nullptr : m_part;
  a.l_part = o ? nullptr : l_part;
  a.mask = P->d_mask;
  a.items = P->d_items + (size_t)list * P->n_items;
  a.bin_ptr = P->d_bin_ptr + (size_t)list * (P->num_bins + 1);
  std::unique_lock<std::mutex> queue_lock;
  if (P->order == SA_ORDER_LPT_DYNAMIC) {
    // the queue's counters are shared by every call with this plan: calls on other streams
    // finish first (a call on this stream follows the previous one anyway).  The queue lock is
    // held until this call's use is recorded, so that two host threads cannot both launch
    // before either has recorded its use
    queue_lock = std::unique_lock<std::mutex>(const_cast<sa_plan*>(P)->queue_mutex);
    std::lock_guard<std::mutex> lock(const_cast<sa_plan*>(P)->use_mutex);
    for (const auto& u : P->uses)
      if (u.first != stream) SA_HIP(hipStreamWaitEvent(stream, u.second, 0));
    a.dyn_items = P->d_lpt_order + (size_t)list * P->n_items;
    a.dyn_ctr = P->d_dyn_ctr + sa::kQueueCtrs * list;
  }
  a.trace = trace;
  a.B = pr.B; a.H = pr.H; a.S = pr.S; a.nQ = P->nQ; a.nK = P->nK; a.n_chunks = pr.n_chunks;
  a.layout = pr.layout; a.c0 = chunk_begin; a.c1 = chunk_end; a.num_bins = P->num_bins;
  a.token_causal = pr.token_causal ? 1 : 0;
  a.q_pairs = P->q_pairs ? 1 : 0;
  a.nI = P->nI;
  a.sb = pr.sb; a.sh = pr.sh; a.ss = pr.ss;
  a.scale = effective_scale(pr);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  hipError_t e = pr.dtype == SA_BF16 ? sa::launch_attn_bf16(a, pr.D, pr.block, stream)
                                     : sa::launch_attn_f32(a, pr.D, pr.block, stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return note_use(P, stream);
}

sa_status chunk_merge(int32_t n_parts, const float* const* o_parts, const float* const* m_parts,
                      const float* const* l_parts, int64_t rows, int32_t D, void* o_out, int32_t out_dtype,
                      float* lse_out, hipStream_t stream) {
  if (n_parts < 1 || n_parts > sa::kMaxMergeParts)
    return fail(SA_ERR_INVALID, "n_parts %d outside [1, %d]", n_parts, sa::kMaxMergeParts);
  if (!o_parts || !m_parts || !l_parts || !o_out) return fail(SA_ERR_INVALID, "NULL pointer argument");
  if (rows < 0) return fail(SA_ERR_INVALID, "rows %lld < 0", (long long)rows);
  if (D != 64 && D != 128) return fail(SA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", D);
  if (out_dtype != SA_F32 && out_dtype != SA_BF16) return fail(SA_ERR_INVALID, "unknown dtype %d", out_dtype);
  if (rows == 0) return SA_OK;
  sa::MergeArgs a{};
  for (int p = 0; p < n_parts; ++p) {
    if (!o_parts[p] || !m_parts[p] || !l_parts[p]) return fail(SA_ERR_INVALID, "part %d has a NULL pointer", p);
    a.o[p] = o_parts[p];
    a.m[p] = m_parts[p];
    a.l[p] = l_parts[p];
  }
  a.out = o_out;
  a.lse = lse_out;
  a.rows = rows;
  a.n_parts = n_parts;
  SA_HIP(sa::launch_merge(a, D, out_dtype, stream));
  return SA_OK;
}

sa_status sparse_attn_plan_info(const sa_plan* P, sa_plan_info* out) {
  if (!P || !out) return fail(SA_ERR_INVALID, "NULL argument");
  std::memset(out, 0, sizeof(*out));
  out->kind = P->kind;
  out->num_bins = P->num_bins;
  out->order = P->order;
  out->n_chunks = P->prob.n_chunks;
  out->nQ = P->nQ;
  out->nK = P->nK;
  out->n_items = P->n_items;
  out->top_k = P->top_k;
  out->total_live = P->total_live;
  out->load_sum = P->load_sum;
  out->makespan = P->makespan;
  out->lower_bound = P->lower_bound;
  if (P->device_lists) {  // statistics of list 0 live on the device: wait for the plan, then read them
    int64_t s[4];
    SA_HIP(hipEventSynchronize(P->ready));
    SA_HIP(hipMemcpy(s, P->d_stats, sizeof(s), hipMemcpyDeviceToHost));
    out->total_live = out->load_sum = s[0];
    if (P->q_pairs) {  // the list loads are union counts; the live tiles are the row sums
      std::vector<int32_t> row((size_t)P->prob.B * P->prob.H * P->nQ);
      SA_HIP(hipMemcpy(row.data(), P->d_row, row.size() * 4, hipMemcpyDeviceToHost));
      out->total_live = 0;
      for (int32_t x : row) out->total_live += x;
    }
    out->makespan = s[2];
    out->lower_bound = s[3];
  }
  out->groups = P->groups;
  return SA_OK;
}

sa_status sparse_attn_plan_copy(const sa_plan* P, int32_t what, int32_t chunk, void* dst, int64_t n_elems) {
  if (!P || !dst) return fail(SA_ERR_INVALID, "NULL argument");
  const sa_problem& pr = P->prob;
  const int C = pr.n_chunks;
  const int64_t BH = (int64_t)pr.B * pr.H;
  const bool block = P->kind == SA_KIND_BLOCK;
  if (what == SA_PLAN_ITEMS || what == SA_PLAN_BIN_PTR || what == SA_PLAN_BIN_LOAD) {
    if (!block) return fail(SA_ERR_INVALID, "work lists exist only for block plans");
    if (chunk < -1 || chunk >= C) return fail(SA_ERR_INVALID, "chunk %d outside [-1, %d)", chunk, C);
  }
  const int list = chunk + 1;
  if (block && !P->device_lists && list > 0 &&
      (what == SA_PLAN_ITEMS || what == SA_PLAN_BIN_PTR || what == SA_PLAN_BIN_LOAD))
    build_chunk_list(const_cast<sa_plan*>(P), list);
  const void* src = nullptr;
  bool device = true;
  int64_t count = 0;
  size_t esize = 4;
  switch (what) {
    case SA_PLAN_ROW: src = P->d_row; count = block ? BH * P->nQ : 0; break;
    case SA_PLAN_COL: src = P->d_col; count = block ? BH * P->nK : 0; break;
    case SA_PLAN_CROW: src = P->d_crow; count = block ? BH * C * P->nQ : 0; break;
    case SA_PLAN_PAIR_ROW: src = P->d_prow; count = P->q_pairs ? BH * P->nI : 0; break;
    case SA_PLAN_PAIR_CROW: src = P->d_pcrow; count = P->q_pairs ? BH * C * P->nI : 0; break;
    case SA_PLAN_ITEMS:
      device = P->device_lists;
      src = device ? (const void*)(P->d_items + (size_t)list * P->n_items)
                   : (const void*)(P->h_items.data() + (size_t)list * P->n_items);
      count = P->n_items;
      break;
    case SA_PLAN_BIN_PTR:
      device = P->device_lists;
      src = device ? (const void*)(P->d_bin_ptr + (size_t)list * (P->num_bins + 1))
                   : (const void*)(P->h_bin_ptr.data() + (size_t)list * (P->num_bins + 1));
      count = P->num_bins + 1;
      break;
    case SA_PLAN_BIN_LOAD:
      device = P->device_lists;
      src = device ? (const void*)(P->d_bin_load + (size_t)list * P->num_bins)
                   : (const void*)(P->h_bin_load.data() + (size_t)list * P->num_bins);
      count = P->num_bins;
      esize = 8;
      break;
    case SA_PLAN_LPT_ORDER:
      if (chunk < -1 || chunk >= C) return fail(SA_ERR_INVALID, "chunk %d outside [-1, %d)", chunk, C);
      src = P->d_lpt_order ? (const void*)(P->d_lpt_order + (size_t)list * P->n_items) : nullptr;
      count = P->d_lpt_order ? P->n_items : 0;
      break;
    case SA_PLAN_TOPK_IDX: src = P->d_idx; count = block ? 0 : BH * pr.S * P->top_k; break;
    case SA_PLAN_TOPK_COUNT: src = P->d_count; count = block ? 0 : BH * pr.S; break;
    default: return fail(SA_ERR_INVALID, "unknown plan array %d", what);
  }
  if (count == 0 || !src) return fail(SA_ERR_INVALID, "array %d does not exist for this plan kind", what);
  if (n_elems != count) return fail(SA_ERR_INVALID, "array %d has %lld elements, caller asked for %lld", what,
                                    (long long)count, (long long)n_elems);
  if (device) {
    if (P->ready) SA_HIP(hipEventSynchronize(P->ready));  // the plan's arrays are complete
    SA_HIP(hipMemcpy(dst, src, (size_t)count * esize, hipMemcpyDeviceToHost));
  } else {
    std::memcpy(dst, src, (size_t)count * esize);
  }
  return SA_OK;
}

sa_status sparse_attn_assign_host(const int64_t* loads, int32_t n, int32_t m, int32_t order, int32_t* items_out,
                                  int32_t* bin_ptr_out, int64_t* bin_load_out) {
  if (n < 0 || m <= 0) return fail(SA_ERR_INVALID, "need n >= 0 and m > 0 (got %d, %d)", n, m);
  if ((n > 0 && (!loads || !items_out)) || !bin_ptr_out) return fail(SA_ERR_INVALID, "NULL argument");
  if (order != SA_ORDER_LPT && order != SA_ORDER_NAIVE) return fail(SA_ERR_INVALID, "unknown order %d", order);
  for (int i = 0; i < n; ++i)
    if (loads[i] < 0) return fail(SA_ERR_INVALID, "loads[%d] = %lld < 0", i, (long long)loads[i]);
  sa::assign(loads, n, m, order, items_out, bin_ptr_out, bin_load_out);
  return SA_OK;
}

sa_status sparse_attn_assign_host_grouped(const int64_t* loads, int32_t n_heads, int32_t items_per_head, int32_t m,
                                          int32_t groups, int32_t* items_out, int32_t* bin_ptr_out,
                                          int64_t* bin_load_out) {
  if (n_heads < 0 || items_per_head <= 0 || m <= 0 || groups <= 0)
    return fail(SA_ERR_INVALID, "need n_heads >= 0, items_per_head > 0, m > 0, groups > 0");
  const int64_t n = (int64_t)n_heads * items_per_head;
  if (n > INT32_MAX) return fail(SA_ERR_INVALID, "too many items");
  if ((n > 0 && (!loads || !items_out)) || !bin_ptr_out) return fail(SA_ERR_INVALID, "NULL argument");
  for (int64_t i = 0; i < n; ++i)
    if (loads[i] < 0) return fail(SA_ERR_INVALID, "loads[%lld] = %lld < 0", (long long)i, (long long)loads[i]);
  sa::assign_grouped(loads, n_heads, items_per_head, m, groups, items_out, bin_ptr_out, bin_load_out);
  return SA_OK;
}

void sparse_attn_plan_destroy(sa_plan* P) { free_plan(P); }

const char* sa_status_string(int32_t status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID: return "SA_ERR_INVALID: invalid argument";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: outside the compiled kernel variants";
    case SA_ERR_HIP: return "SA_ERR_HIP: HIP runtime error";
    case SA_ERR_NOMEM: return "SA_ERR_NOMEM: allocation failed";
    default: return "unknown sa_status";
  }
}

const char* sa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
