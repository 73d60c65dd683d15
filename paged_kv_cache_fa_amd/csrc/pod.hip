// One launch for both passes of cascade attention on gfx950: the suffix
// decode (HBM-bound, VALU) and the shared-prefix append (MFMA) run side by
// side in the same CUs ([Guide] "FlashInfer: GPU Kernels for LLM Inference
// (2026 Guide)", section "Cascade attention for shared prefixes", and the
// mixed prefill + decode batches of POD-attention named in section
// "Features (from the repository README)").
//
// Workgroups 0 .. dec_blocks-1 are decode workers (4 independent waves, the
// suffix plan's work lists); the rest run the prefix plan's append tiles
// (bins by workgroup index mod 8, as in the append kernel) with 4 waves, so
// their tiles hold at most 128 / G query positions. Both roles are compiled
// for 2 waves per SIMD (at most 256 registers each) and a CU holds one
// decode and one append workgroup at once: the append waves' matrix work
// overlaps the decode waves' memory streaming. The decode role keeps a
// 2-page ring to fit the register budget. Split units merge as in the two
// kernels (the prefix pass defers to the cascade combine).
#include "append_dev.h"
#include "decode_dev.h"

namespace pkfa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int DT, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void pod_kernel(AttnParams dp, AttnParams ap, int dec_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * app::VLayout::kBufElems];
  __shared__ int s_flag;
  const int blk = (int)blockIdx.x;
  if (blk < dec_blocks) {
    // the decode role takes the decode kernel's path for this group size
    // (bit-identical results); its LDS pages alias the append role's buffer
    constexpr bool kMPV = G >= 4;
    static_assert(!kMPV || 4 * dec::kVPageBytes <= sizeof(smem), "decode LDS pages do not fit");
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    dec::decode_worker<DT, G, 2, false, kMPV>(dp, blk * kWaves + wave,
                                               reinterpret_cast<uint8_t*>(smem) + wave * dec::kVPageBytes);
  }
  else
    app::append_worker<DT, G, 2, kWaves>(ap, blk - dec_blocks, (int)gridDim.x - dec_blocks, smem, s_flag);
}

template <int DT>
hipError_t launch_dt(const AttnParams& dp, const AttnParams& ap, int group, int dec_blocks,
                     int grid, hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL((pod_kernel<DT, 1>), dim3(grid), dim3(kThreads), 0, s, dp, ap, dec_blocks); break;
    case 2: hipLaunchKernelGGL((pod_kernel<DT, 2>), dim3(grid), dim3(kThreads), 0, s, dp, ap, dec_blocks); break;
    case 4: hipLaunchKernelGGL((pod_kernel<DT, 4>), dim3(grid), dim3(kThreads), 0, s, dp, ap, dec_blocks); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pod(const AttnParams& dp, int workers, const AttnParams& ap, int max_tiles,
                      int dtype, int group, hipStream_t s) {
  // decode workgroups first (a multiple of 8, so the append part keeps its
  // XCD bins), then the append grid of the append kernel
  constexpr int kPerBlock = kWaves;
  const int dec_blocks = (workers + 8 * kPerBlock - 1) / (8 * kPerBlock) * 8;
  const int app_blocks = (max_tiles + kAppendBins - 1) / kAppendBins * kAppendBins;
  const int grid = dec_blocks + app_blocks;
  if (grid <= 0) return hipSuccess;
  return dtype == FA_BF16 ? launch_dt<FA_BF16>(dp, ap, group, dec_blocks, grid, s)
                          : launch_dt<FA_F16>(dp, ap, group, dec_blocks, grid, s);
}

}  // namespace pkfa
