// Paged-KV decode kernel for gfx950: one launch of worker waves (see
// decode_dev.h for what it computes and how).
#include "decode_dev.h"

namespace pkfa {
namespace {

using dec::decode_worker;

template <int DT, int G, int NBUF, bool KV8, bool MQK>
__global__ __launch_bounds__(256, 1) void decode_kernel(AttnParams p) {
  // per-wave rows for the matrix-core score exchange (unused otherwise)
  __shared__ float sc[MQK ? 4 * dec::kScoreFloats : 1];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  decode_worker<DT, G, NBUF, KV8, MQK>(p, (int)blockIdx.x * 4 + wave,
                                       MQK ? sc + wave * dec::kScoreFloats : nullptr);
}

// Ring depth and score path per group size. 16-bit pages keep 2 pages (16 KB
// per wave) in flight; E4M3 pages are half the size, so the ring is deeper.
// G = 8, and G = 4 over E4M3 pages, compute their scores on the matrix cores
// (MQK): on the VALU their dot products would need most of the vector peak at
// HBM speed (twice the products per byte of 16-bit G = 4), and the q
// operands shrink to 16 registers. Batch-64 lengths, 8 kv heads: G = 8 16-bit
// 138 -> 118 us, G = 4 E4M3 73 -> 67 us; 16-bit G = 4 is the same either way
// (108 us) and keeps the VALU path that the mixed-batch kernel shares.
template <int DT, bool KV8>
hipError_t launch_dt(const AttnParams& p, int group, int grid, hipStream_t s) {
  constexpr int R = KV8 ? 5 : 3;
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<DT, 1, R, KV8, false>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<DT, 2, R, KV8, false>), dim3(grid), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<DT, 4, R, KV8, KV8>), dim3(grid), dim3(256), 0, s, p); break;
    case 8:
      hipLaunchKernelGGL((decode_kernel<DT, 8, KV8 ? 3 : 2, KV8, true>), dim3(grid), dim3(256), 0, s,
                         p);
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
