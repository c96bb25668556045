// Batched causal prefill (gfx950).  The matrix-core kernel is not in this
// build yet; the launcher reports the call as unsupported.
#include "pa_internal.h"

namespace pa {

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
