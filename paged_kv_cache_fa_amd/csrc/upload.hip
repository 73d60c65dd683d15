// Plan upload: a small copy kernel that reads the plan image straight out of
// pinned (device-visible) host memory. Queued on the caller's stream right
// before the attention kernel, it avoids the DMA-engine round trip of a
// host-to-device copy, which on this GPU costs more than the copy itself.
// Each workgroup then stores a sequence number into a word of the host
// workspace, which tells the host that the image may be rewritten; a HIP
// event recorded between this kernel and the attention kernel would delay
// the latter by several microseconds.
#include "device_common.h"
#include "kernels.h"
#include "plan_internal.h"

namespace pkfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void upload_kernel(uint32_t* __restrict__ dst,
                                                     const uint32_t* __restrict__ src,
                                                     int64_t n_words, uint32_t* flags,
                                                     uint32_t seq) {
  const int64_t n16 = n_words >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
  const int64_t tail = n16 * 4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (tail < n_words && blockIdx.x == 0 && threadIdx.x < 4) dst[tail] = src[tail];
  if (flags) {
    // Every thread's loads have returned (its store consumed them) before the
    // barrier; then the workgroup reports that it no longer reads the host
    // image. A system-scope store, so the host sees the word without waiting
    // for the end of the kernel.
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(flags + blockIdx.x, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace

int upload_grid(int64_t n_words) {
  const int64_t blocks = ((n_words >> 2) + 255) / 256;
  return (int)(blocks < 1 ? 1 : (blocks > kUploadMaxGrid ? kUploadMaxGrid : blocks));
}

hipError_t launch_upload(uint32_t* dst, const uint32_t* src, int64_t n_words, uint32_t* flags,
                         uint32_t seq, hipStream_t s) {
  if (n_words <= 0) return hipSuccess;
  hipLaunchKernelGGL(upload_kernel, dim3(upload_grid(n_words)), dim3(256), 0, s, dst, src, n_words,
                     flags, seq);
  return hipGetLastError();
}

}  // namespace pkfa
