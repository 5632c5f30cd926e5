// Host-side helpers of the C ABI: argument validation, the calling thread's error detail and shared
// constants. Nothing here needs HIP, so the host checkers (pa_host.cpp) and the host scheduler also build with
// a plain C++ compiler (the sanitizer build of the host code).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Tokens per decode tile: one wave processes 16 consecutive context tokens per step.
constexpr int kTileTokens = 16;
// Largest context partition (keys) one work item handles.
constexpr int kMaxPartitionTokens = 1024;

// The calling thread's error detail (pa_last_error_detail), kDetailBytes long.
constexpr size_t kDetailBytes = 256;
char* error_detail();
// Sets the calling thread's detail to `what` and returns st.
pa_status fail(pa_status st, const char* what);
// Host scalars of pa_params: PA_OK, or the status of the first violated range (with its detail).
pa_status validate_params(const pa_params* p);

}  // namespace pa
