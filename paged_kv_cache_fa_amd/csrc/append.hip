// Paged-KV append / prefill kernel for gfx950 (see append_dev.h for what it
// computes and how).
#include "append_dev.h"

namespace pkfa {
namespace {

constexpr int kWaves = 8;  // one 512-thread workgroup per CU, 2 waves per SIMD
constexpr int kThreads = 64 * kWaves;

template <int DT, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void append_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * app::VLayout::kBufElems];
  __shared__ int s_flag;
  app::append_worker<DT, G, 4, kWaves>(p, (int)blockIdx.x, (int)gridDim.x, smem, s_flag);
}

template <int DT>
hipError_t launch_dt(const AttnParams& p, int group, int grid, hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL((append_kernel<DT, 1>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((append_kernel<DT, 2>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL((append_kernel<DT, 4>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL((append_kernel<DT, 8>), dim3(grid), dim3(kThreads), 0, s, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AttnParams& p, int dtype, int group, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int grid = (max_tiles + kAppendBins - 1) / kAppendBins * kAppendBins;
  return dtype == FA_BF16 ? launch_dt<FA_BF16>(p, group, grid, s)
                          : launch_dt<FA_F16>(p, group, grid, s);
}

}  // namespace pkfa
