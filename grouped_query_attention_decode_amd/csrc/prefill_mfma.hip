// Placeholder until the kernel lands: reports no supported shapes.
#include "gqa_internal.h"

namespace gqa {

bool prefill_mfma_supports(const AttnArgs &) { return false; }

hipError_t launch_prefill_mfma(const AttnArgs &, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace gqa
