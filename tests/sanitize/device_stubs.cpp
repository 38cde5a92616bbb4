// Stand-ins for the library's device-side entry points, linked into the
// sanitizer build of the host code (pa_host.cpp, pa_alloc.cpp), which is
// compiled by the host compiler alone.  A call that reaches one of them has
// passed every host check; each answers as a launch does on a machine
// without a usable GPU, so the host code takes its error path.

#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

int split_wgs_per_cu(int, int, int, int) { return 1; }

hipError_t launch_decode(const DecodeParams&, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorNoDevice; }

hipError_t launch_scatter(const uint8_t*, int32_t, uint8_t*, uint8_t*, int32_t, int32_t, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}

hipError_t launch_append_encode(const AppendLaunch&, hipStream_t) { return hipErrorNoDevice; }

hipError_t launch_read_probe(const void*, size_t, uint32_t*, int32_t, int32_t, bool, bool, hipStream_t) {
  return hipErrorNoDevice;
}

void* scratch_buffer(int32_t* st) {
  *st = -5;  // PA_ERR_HIP
  return nullptr;
}

hipError_t launch_gather(const uint8_t*, int32_t, const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t,
                         uint8_t*, int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace pa
