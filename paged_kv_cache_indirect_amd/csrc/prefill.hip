// Chunked causal prefill (bf16 MFMA). Placeholder launcher until the kernel lands.
#include "launch.h"

namespace pa {

hipError_t LaunchPrefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
