// kda_chunked.hip - chunk-parallel KDA prefill (placeholder until the MFMA
// kernel lands: every call is routed to the token-by-token kernel).
#include "kda_internal.h"

namespace kda {

bool chunked_supported(const PrefillArgs&) { return false; }

size_t chunked_workspace_bytes(int, int, int, int, int, bool) { return 0; }

hipError_t launch_chunked(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
