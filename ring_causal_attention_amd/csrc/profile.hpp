// Opt-in per-kernel timing: when enabled, every kernel launch of the library is bracketed by
// two HIP events recorded on the launch stream; lwm_profile_get() resolves them.
#pragma once

#include <hip/hip_runtime.h>

namespace lwm {

// Returns a token for prof_end(), or -1 when timing is off.
int prof_begin(const char* kernel, hipStream_t stream);
void prof_end(int token, hipStream_t stream);

// Launch a kernel bracketed by the timing events (no-ops when timing is off).
#define LWM_LAUNCH(name, kernel, grid, block, stream, ...)                             \
  do {                                                                                 \
    const int lwm_prof_token_ = ::lwm::prof_begin(name, stream);                       \
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                   \
    ::lwm::prof_end(lwm_prof_token_, stream);                                          \
  } while (0)

}  // namespace lwm
