// Kernel launchers replaced for the host-only check build: that build compiles the C ABI's host
// code (validation, the plan object, the host LPT planner) without device code, under address
// and undefined-behaviour sanitizers, so that the host entry points can be exercised on a
// machine without a GPU.  Every launcher reports that no kernel is available.
#include "internal.h"

namespace sa {

hipError_t launch_popcount(const uint8_t*, int, int, int, int, int, int32_t*, int32_t*, int32_t*, hipStream_t, int32_t*,
                           int32_t*) {
  return hipErrorNotSupported;
}
hipError_t launch_plan_rounds(const int32_t*, const int32_t*, int, int, int, int, int32_t*, int32_t*, int64_t*,
                              int64_t*, hipStream_t, int, int, int32_t*, int32_t*) {
  return hipErrorNotSupported;
}
hipError_t launch_attn_bf16(const FwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
int attn_bf16_wg_per_cu(int block) { return block >= 128 ? 1 : 2; }
hipError_t launch_attn_f32(const FwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_merge(const MergeArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_indexer(const IndexerArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gather_attn(const GatherArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace sa
