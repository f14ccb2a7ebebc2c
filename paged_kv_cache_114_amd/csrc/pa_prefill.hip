// Variable-length causal prefill over the paged KV cache (bf16 MFMA).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
