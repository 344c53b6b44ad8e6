// Chunked prefill for the diagonal-transition variants (KATH, GLA) on bf16 MFMA.
#include "common.hpp"
#include "la_internal.h"

namespace la {

bool diag_mfma_supported(int, int, int, bool) { return false; }
size_t diag_mfma_workspace_bytes(const Problem&) { return 0; }
int diag_mfma_auto_segments(const Problem&) { return 1; }
hipError_t launch_prefill_diag_mfma(const Problem&) { return hipErrorInvalidValue; }

}  // namespace la
