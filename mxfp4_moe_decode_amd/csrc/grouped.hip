// Grouped (prefill) path.  Not built yet: reports no workspace, so the entry
// point returns MOE_ERR_UNSUPPORTED.
#include "internal.h"

namespace mxmoe {

size_t grouped_ws_bytes(const moe_layer_t&, int) { return 0; }

hipError_t launch_grouped(const moe_layer_t&, const uint16_t*, int, const uint16_t*, uint16_t*, void*,
                          hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace mxmoe
