// Chunked-prefill tiles on MFMA: not yet enabled; mixed steps route every query row through the
// decode-partition kernel until this path is in place.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

bool prefill_supported(int, int, int) { return false; }
int prefill_rows_per_tile(int group) { return group > 0 && group <= kPrefillPairs ? kPrefillPairs / group : 1; }
hipError_t launch_plan(const AttnArgs&, int32_t*, int32_t*, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prefill(const AttnArgs&, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pa
