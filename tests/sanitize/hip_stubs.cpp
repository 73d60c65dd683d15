// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// the C ABI (api.cpp) links against, so that the planner (plan.cpp) and the
// host paths of the ABI build with a plain host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer. A plan made without a
// device workspace, and every argument check, make no HIP call; each stand-in
// therefore reports the call and aborts, so a host path that reaches the
// runtime fails the sanitizer test instead of passing silently.
#include <hip/hip_runtime_api.h>

#include <stdio.h>
#include <stdlib.h>

#include "../../include/fa.h"
#include "../../paged_kv_cache_fa_amd/csrc/kernels.h"

namespace {
[[noreturn]] void reached(const char* what) {
  fprintf(stderr, "host-only build: %s was called\n", what);
  fflush(stderr);
  abort();
}
}  // namespace

extern "C" {
const char* hipGetErrorString(hipError_t) { reached("hipGetErrorString"); }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus*) {
  reached("hipStreamIsCapturing");
}
hipError_t hipEventSynchronize(hipEvent_t) { reached("hipEventSynchronize"); }
hipError_t hipMemsetAsync(void*, int, size_t, hipStream_t) { reached("hipMemsetAsync"); }
hipError_t hipPointerGetAttributes(hipPointerAttribute_t*, const void*) {
  reached("hipPointerGetAttributes");
}
hipError_t hipGetLastError(void) { reached("hipGetLastError"); }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  reached("hipMemcpyAsync");
}
hipError_t hipEventCreateWithFlags(hipEvent_t*, unsigned) { reached("hipEventCreateWithFlags"); }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { reached("hipEventRecord"); }
hipError_t hipEventDestroy(hipEvent_t) { reached("hipEventDestroy"); }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) {
  reached("hipStreamWaitEvent");
}
hipError_t hipStreamSynchronize(hipStream_t) { reached("hipStreamSynchronize"); }
// A heap read at index i of a 4-element array: out of bounds for i >= 4. The
// sanitizer test calls it with i = 4 to show that the build is instrumented.
int pkfa_sanitizer_canary(int i) {
  int* a = static_cast<int*>(malloc(4 * sizeof(int)));
  for (int k = 0; k < 4; ++k) a[k] = k;
  const int v = a[i];
  free(a);
  return v;
}
// the no-allocation decode keeps its static device array in a HIP source
fa_status fa_decode_noalloc(const fa_geometry*, const int32_t*, const int32_t*, int32_t,
                            const void*, const void*, const void*, int64_t, int64_t, int64_t,
                            const int32_t*, const int32_t*, const int32_t*, float, void*, float*,
                            void*) {
  reached("fa_decode_noalloc");
}
// the streaming-read probe lives with its kernel in a HIP source
fa_status fa_probe_stream_read(const void*, int64_t, uint32_t*, int32_t, void*) {
  reached("fa_probe_stream_read");
}
}

namespace pkfa {
hipError_t launch_decode(const AttnParams&, int, bool, int, int, hipStream_t) {
  reached("launch_decode");
}
hipError_t launch_append(const AttnParams&, int, int, int, hipStream_t) { reached("launch_append"); }
hipError_t launch_pod(const AttnParams&, int, const AttnParams&, int, int, int, bool,
                      hipStream_t) {
  reached("launch_pod");
}
int upload_grid(int64_t) { return 1; }
hipError_t launch_upload(uint32_t*, const uint32_t*, int64_t, uint32_t*, uint32_t, hipStream_t) {
  reached("launch_upload");
}
hipError_t launch_merge_state(const void*, const float*, const void*, const float*, void*, float*,
                              int64_t, int, int, int, hipStream_t) {
  reached("launch_merge_state");
}
hipError_t launch_cascade_merge(const int32_t*, const int32_t*, const float*, const float*,
                                const void*, const float*, const void*, const float*, void*,
                                float*, const int32_t*, int64_t, int, int, int, int, int,
                                hipStream_t) {
  reached("launch_cascade_merge");
}
hipError_t launch_merge_states(const void*, const float*, int64_t, int, int, int, int, void*,
                               float*, hipStream_t) {
  reached("launch_merge_states");
}
}  // namespace pkfa
