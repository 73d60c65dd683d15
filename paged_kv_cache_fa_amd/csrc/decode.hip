// Paged-KV decode kernel for gfx950: one launch of worker waves (see
// decode_dev.h for what it computes and how).
#include "decode_dev.h"

namespace pkfa {
namespace {

using dec::decode_worker;

template <int DT, int G, int NBUF, bool KV8>
__global__ __launch_bounds__(256, 1) void decode_kernel(AttnParams p) {
  decode_worker<DT, G, NBUF, KV8>(
      p, (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)));
}

// Ring depth per group size: 16-bit pages keep 2 pages (16 KB per wave) in
// flight for G <= 4 (1 for G = 8, whose 8 heads of accumulators fill the
// registers); E4M3 pages are half the size, so the ring is deeper.
template <int DT, bool KV8>
hipError_t launch_dt(const AttnParams& p, int group, int grid, hipStream_t s) {
  constexpr int R = KV8 ? 5 : 3;
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<DT, 1, R, KV8>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<DT, 2, R, KV8>), dim3(grid), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<DT, 4, R, KV8>), dim3(grid), dim3(256), 0, s, p); break;
    case 8:
      hipLaunchKernelGGL((decode_kernel<DT, 8, KV8 ? 3 : 2, KV8>), dim3(grid), dim3(256), 0, s, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnParams& p, int dtype, bool kv_e4m3, int group, int workers,
                         hipStream_t s) {
  const int grid = (workers + 3) / 4;
  if (grid <= 0) return hipSuccess;
  if (kv_e4m3)
    return dtype == FA_BF16 ? launch_dt<FA_BF16, true>(p, group, grid, s)
                            : launch_dt<FA_F16, true>(p, group, grid, s);
  return dtype == FA_BF16 ? launch_dt<FA_BF16, false>(p, group, grid, s)
                          : launch_dt<FA_F16, false>(p, group, grid, s);
}

}  // namespace pkfa
