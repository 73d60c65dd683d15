// Streaming-read probe for gfx950: the HBM read bandwidth a plain kernel
// attains on this device. It is a measurement utility beside the attention
// path (the benchmark reports the decode's bandwidth against it), not a step
// of that path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "plan_internal.h"

namespace pkfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread per pass

// Workgroup g reads its own contiguous share of the 16-byte words, 256 x 8
// words (32 KB) per pass, with the non-temporal cache policy, and folds them
// by XOR; the fold is stored only if it equals a value no input makes likely,
// which keeps the loads without adding write traffic. (Contiguous shares
// measured 6.9-7.05 TB/s from 512 to 16384 workgroups on MI355X; a grid-wide
// stride 5.5-6.3 TB/s.)
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* src, int64_t n16,
                                                                     uint32_t key, uint32_t* flag) {
  const int64_t share = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * share;
  const int64_t end = min(n16, beg + share);
  int64_t i = beg + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
    u32x4 w[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      w[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= w[u][0] ^ w[u][1] ^ w[u][2] ^ w[u][3];
  }
  for (; i < end; i += kProbeThreads) {
    const u32x4 w = __builtin_nontemporal_load(src + i);
    acc ^= w[0] ^ w[1] ^ w[2] ^ w[3];
  }
  if (acc == key) *flag = 1u;
}

}  // namespace
}  // namespace pkfa

extern "C" fa_status fa_probe_stream_read(const void* src, int64_t bytes, uint32_t* flag,
                                          int32_t workgroups, void* stream) {
  if (!src || !flag || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) ||
      workgroups <= 0) {
    pkfa::set_error("stream-read probe: NULL pointer, size not a positive multiple of 16, "
                    "source not 16-byte aligned or no workgroups");
    return FA_ERR_INVALID;
  }
  hipLaunchKernelGGL(pkfa::stream_read_kernel, dim3(workgroups), dim3(pkfa::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const pkfa::u32x4*>(src),
                     bytes / 16, 0x9e3779b9u, flag);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    pkfa::set_error("stream-read probe launch: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}
