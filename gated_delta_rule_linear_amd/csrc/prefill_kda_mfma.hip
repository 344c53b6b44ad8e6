// Chunked prefill for Kimi Delta Attention on bf16 matrix cores (not built yet: the
// entry points below report the shape as unsupported, so the fp32 VALU path serves
// every KDA prefill).
#include "la_internal.h"

namespace la {

bool kda_mfma_supported(int, int, bool) { return false; }

size_t kda_mfma_workspace_bytes(const Problem&) { return 0; }

hipError_t launch_prefill_kda_mfma(const Problem&) { return hipErrorInvalidValue; }

}  // namespace la
