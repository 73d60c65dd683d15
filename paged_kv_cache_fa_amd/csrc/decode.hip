// Paged-KV decode kernel for gfx950: one launch of worker waves (see
// decode_dev.h for what it computes and how).
#include "decode_dev.h"

namespace pkfa {
namespace {

using dec::decode_worker;

template <int DT, int G, int NBUF, bool KV8, bool MPV>
__global__ __launch_bounds__(256, 1) void decode_kernel(AttnParams p) {
  // per-wave LDS page of the matrix-core path (unused by the VALU path)
  constexpr int kWaveBytes = MPV ? dec::kVPageBytes : 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kWaveBytes];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  decode_worker<DT, G, NBUF, KV8, MPV>(p, (int)blockIdx.x * 4 + wave, lds + wave * kWaveBytes);
}

// Ring depth and path per group size. 16-bit pages keep 2 pages (16 KB per
// wave) in flight; E4M3 pages are half the size, so the ring is deeper.
// G >= 4 takes the matrix-core path (MPV); batch-64 lengths, 8 kv heads:
// G = 4 108 -> 102 us, G = 8 138 -> 103 us, E4M3 G = 4 73 -> 60 us. G <= 2
// keeps the VALU path (G = 1: 99 against 100 us, E4M3 G = 1: 55 against
// 58 us; the single-request decode 11.4 against 13.4 us).
template <int DT, bool KV8>
hipError_t launch_dt(const AttnParams& p, int group, int grid, hipStream_t s) {
  constexpr int R = KV8 ? 5 : 3;
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<DT, 1, R, KV8, false>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<DT, 2, R, KV8, false>), dim3(grid), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<DT, 4, R, KV8, true>), dim3(grid), dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<DT, 8, R, KV8, true>), dim3(grid), dim3(256), 0, s, p); break;
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
