// Chunked prefill for the gated delta rule on bf16 MFMA.
#include "common.hpp"
#include "la_internal.h"

namespace la {

bool gdn_mfma_supported(int, int, bool) { return false; }
hipError_t launch_prefill_gdn_mfma(const Problem&) { return hipErrorInvalidValue; }

}  // namespace la
