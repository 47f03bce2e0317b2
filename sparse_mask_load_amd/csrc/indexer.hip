// DSA-style indexer (6D-parallel notes, section 7.1): placeholder until the
// top-k selection kernel lands; the plan reports SA_ERR_HIP (not supported).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sa {

hipError_t launch_indexer(const IndexerArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace sa
