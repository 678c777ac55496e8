// Fused LM-head selected logprob (matrix-core path). Not implemented yet: the entry point
// reports an error instead of running anything else.
#include "common.h"

namespace drift {

size_t lmhead_ws_bytes(int64_t T, int64_t V) { return 256 + align_up((size_t)T * 16, 256) + 0 * V; }

hipError_t launch_lmhead(const LmheadParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace drift
