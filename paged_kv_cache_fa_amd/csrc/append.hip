// Paged-KV append / prefill kernel for gfx950 (MFMA). Placeholder until the
// MFMA kernel lands: reports "not supported".
#include "device_common.h"
#include "kernels.h"

namespace pkfa {

hipError_t launch_append(const AttnParams&, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pkfa
