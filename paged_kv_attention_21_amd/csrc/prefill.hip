// Paged prefill attention for gfx950 (placeholder until the MFMA kernel lands).
#include "launch.h"

namespace pka {

bool prefill_supported(bool, int, int) { return false; }

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pka
