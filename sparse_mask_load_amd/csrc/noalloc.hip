// Block-sparse attention in one call that allocates nothing, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// It does, on the caller's stream, what a plan made with SA_ORDER_LPT_DEVICE
// followed by sparse_attn_fwd does: the mask popcount, the round-based LPT
// list the forward call would use (the full-range list, or the chunk's own
// list for a one-chunk range), and the attention kernel.  The counts and the
// work list live in a file-scope device array instead of plan buffers.  Every
// call on a GPU uses that GPU's one copy of the array, so calls that overlap
// on one GPU (on different streams, or from different host threads) race;
// calls ordered on one stream do not.  Nothing in the array needs clearing:
// each call writes every entry it reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "sparse_attn.h"

namespace {

constexpr size_t kScratchBytes = size_t(2) << 20;  // per GPU
constexpr int kMaxDevices = 64;

// Counts and work list of the allocation-free path.  In host code this name
// is not a device address: host code uses the per-device address taken below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
unsigned char* g_scratch[kMaxDevices];  // device address of `scratch` on each GPU, once known

// Address of this GPU's copy of the array (looked up once per device, with that device current).
sa_status scratch_of(int device, unsigned char** out) {
  if (device < 0 || device >= kMaxDevices) return sa::set_error(SA_ERR_UNSUPPORTED, "device %d beyond %d", device, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return sa::set_error(SA_ERR_HIP, "hipGetSymbolAddress of the work-list array: %s", hipGetErrorString(e));
    g_scratch[device] = (unsigned char*)p;
  }
  *out = g_scratch[device];
  return SA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Byte offsets of the arrays in the scratch array.
struct Layout {
  size_t row, col, crow, prow, pcrow, items, bin_ptr, bin_load, stats, end;
};

// nI: items per (batch, head) (nQ, or the pair count with Q-block pairs; then nP = nI)
Layout layout_for(int64_t BH, int64_t nQ, int64_t nK, int64_t C, int64_t m, int64_t nI, bool pairs) {
  Layout L;
  L.row = 0;
  L.col = align256(L.row + (size_t)(BH * nQ) * 4);
  L.crow = align256(L.col + (size_t)(BH * nK) * 4);
  L.prow = align256(L.crow + (size_t)(BH * C * nQ) * 4);
  L.pcrow = align256(L.prow + (pairs ? (size_t)(BH * nI) * 4 : 0));
  L.items = align256(L.pcrow + (pairs ? (size_t)(BH * C * nI) * 4 : 0));
  L.bin_ptr = align256(L.items + (size_t)(BH * nI) * 4);
  L.bin_load = align256(L.bin_ptr + (size_t)(m + 1) * 4);
  L.stats = align256(L.bin_load + (size_t)m * 8);
  L.end = L.stats + 4 * 8;
  return L;
}

}  // namespace

extern "C" sa_status sparse_attn_fwd_noalloc(const sa_problem* prob, const uint8_t* mask, int32_t num_bins,
                                             const void* q, const void* k, const void* v, int32_t chunk_begin,
                                             int32_t chunk_end, void* o, float* o_part, float* m_part,
                                             float* l_part, hipStream_t stream) {
  sa_status st = sa::validate_block_problem(prob);
  if (st) return st;
  const sa_problem& pr = *prob;
  if (!mask || !q || !k || !v) return sa::set_error(SA_ERR_INVALID, "mask, q, k or v is NULL");
  if ((uintptr_t)mask % 16) return sa::set_error(SA_ERR_INVALID, "mask must be 16-byte aligned");
  if (chunk_begin < 0 || chunk_end > pr.n_chunks || chunk_begin >= chunk_end)
    return sa::set_error(SA_ERR_INVALID, "chunk range [%d, %d) not inside [0, %d)", chunk_begin, chunk_end,
                         pr.n_chunks);
  if (!o && (!o_part || !m_part || !l_part))
    return sa::set_error(SA_ERR_INVALID, "partial mode needs o_part, m_part and l_part");
  if (num_bins < 0) return sa::set_error(SA_ERR_INVALID, "num_bins %d < 0", num_bins);
  const int64_t nQ = (pr.S + pr.block - 1) / pr.block, nK = nQ, BH = (int64_t)pr.B * pr.H, C = pr.n_chunks;
  const bool pairs = pr.q_pairs != 0;
  const int64_t nI = pairs ? (nQ + 1) / 2 : nQ;  // items per (batch, head)
  // size limits first (before any HIP call), with the most bins the planner takes when the
  // default count is asked for
  auto limits = [&](int m) -> sa_status {
    if (BH * nI > sa::kDevicePlanMaxItems || m > sa::kDevicePlanMaxBins)
      return sa::set_error(SA_ERR_UNSUPPORTED, "the allocation-free path plans at most %d work items on "
                                               "at most %d bins (got %lld, %d)",
                           sa::kDevicePlanMaxItems, sa::kDevicePlanMaxBins, (long long)(BH * nI), m);
    const Layout L = layout_for(BH, nQ, nK, C, m, nI, pairs);
    if (L.end > kScratchBytes)
      return sa::set_error(SA_ERR_UNSUPPORTED, "the allocation-free path's counts and list need %zu bytes, above its "
                                               "%zu-byte work array (B*H*n_chunks*nQ too large)",
                           L.end, kScratchBytes);
    return SA_OK;
  };
  if ((st = limits(num_bins ? num_bins : sa::kDevicePlanMaxBins))) return st;
  int device = 0;
  const hipError_t de = hipGetDevice(&device);
  if (de != hipSuccess) return sa::set_error(SA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(de));
  const int m = num_bins ? num_bins : sa::default_num_bins(pr, device);
  if ((st = limits(m))) return st;
  const Layout L = layout_for(BH, nQ, nK, C, m, nI, pairs);
  unsigned char* base = nullptr;
  if ((st = scratch_of(device, &base))) return st;
  int32_t* row = (int32_t*)(base + L.row);
  int32_t* col = (int32_t*)(base + L.col);
  int32_t* crow = (int32_t*)(base + L.crow);
  int32_t* prow = pairs ? (int32_t*)(base + L.prow) : nullptr;
  int32_t* pcrow = pairs ? (int32_t*)(base + L.pcrow) : nullptr;
  int32_t* items = (int32_t*)(base + L.items);
  int32_t* bin_ptr = (int32_t*)(base + L.bin_ptr);
  int64_t* bin_load = (int64_t*)(base + L.bin_load);
  int64_t* stats = (int64_t*)(base + L.stats);
  hipError_t e =
      sa::launch_popcount(mask, (int)BH, (int)nQ, (int)nK, (int)C, pr.layout, row, col, crow, stream, prow, pcrow);
  if (e != hipSuccess) return sa::set_error(SA_ERR_HIP, "popcount launch: %s", hipGetErrorString(e));
  // the list the forward call of a plan would use: one chunk's own list, else the full-range one
  const int list = (chunk_end - chunk_begin == 1) ? 1 + chunk_begin : 0;
  e = sa::launch_plan_rounds(pairs ? prow : row, pairs ? pcrow : crow, (int)BH, (int)nI, (int)C, m, items, bin_ptr,
                             bin_load, stats, stream, list, 1);
  if (e != hipSuccess) return sa::set_error(SA_ERR_HIP, "planning launch: %s", hipGetErrorString(e));
  sa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.o_part = o ? nullptr : o_part;
  a.m_part = o ? nullptr : m_part;
  a.l_part = o ? nullptr : l_part;
  a.mask = mask;
  a.items = items;
  a.bin_ptr = bin_ptr;
  a.trace = nullptr;
  a.B = pr.B; a.H = pr.H; a.S = pr.S; a.nQ = (int)nQ; a.nK = (int)nK; a.n_chunks = pr.n_chunks;
  a.layout = pr.layout; a.c0 = chunk_begin; a.c1 = chunk_end; a.num_bins = m;
  a.token_causal = pr.token_causal ? 1 : 0;
  a.q_pairs = pairs ? 1 : 0;
  a.nI = (int)nI;
  a.sb = pr.sb; a.sh = pr.sh; a.ss = pr.ss;
  a.scale = sa::softmax_scale(pr);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  e = pr.dtype == SA_BF16 ? sa::launch_attn_bf16(a, pr.D, pr.block, stream) : sa::launch_attn_f32(a, pr.D, pr.block, stream);
  if (e != hipSuccess) return sa::set_error(SA_ERR_HIP, "attention kernel launch: %s", hipGetErrorString(e));
  return SA_OK;
}
