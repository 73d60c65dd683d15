// One launch for a decode batch and an append batch on gfx950: the suffix
// decode and the shared-prefix pass of cascade attention ([Guide]
// "FlashInfer: GPU Kernels for LLM Inference (2026 Guide)", section "Cascade
// attention for shared prefixes"), or the decode and prefill requests of a
// mixed batch (POD-attention, named in section "Features (from the
// repository README)").
//
// Workgroups 0 .. dec_blocks-1 are decode workers (independent waves, the
// decode plan's work lists); the rest run the append plan's tiles (bins by
// workgroup index mod 8, as in the append kernel). Two shapes:
//  * shared: 4-wave workgroups compiled for 2 waves per SIMD (at
//    most 256 registers each), two LDS stages, so a CU holds one decode and
//    one append workgroup at once and the append waves' matrix work overlaps
//    the decode waves' memory streaming; append tiles hold at most 128 / G
//    query positions (G <= 4), and the decode role keeps a 2-page ring;
//  * wide: the append kernel's 8-wave workgroups and four-stage LDS ring
//    (tiles of up to 256 / G positions); one workgroup fills a CU's LDS, so
//    each CU runs one role at a time. A decode workgroup runs 8 worker waves,
//    so a decode plan of 4 worker waves per CU holds half the CUs (which
//    still stream near the HBM peak) while the append tiles run at full rate
//    on the other half and then move onto the decode's CUs as they finish.
// Split units merge as in the two kernels (a cascade's prefix pass defers to
// the cascade combine).
#include "append_dev.h"
#include "decode_dev.h"

namespace pkfa {
namespace {

template <int DT, int G, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void pod_kernel(AttnParams dp, AttnParams ap, int dec_blocks) {
  constexpr int kStages = WAVES == 8 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * app::VLayout::kBufElems];
  __shared__ int s_flag;
  const int blk = (int)blockIdx.x;
  if (blk < dec_blocks) {
    // the decode role takes the decode kernel's path for this group size
    // (bit-identical results); its LDS pages alias the append role's buffer
    constexpr bool kMPV = G >= 4;
    static_assert(!kMPV || WAVES * dec::kVPageBytes <= sizeof(smem), "decode LDS pages do not fit");
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    dec::decode_worker<DT, G, 2, false, kMPV>(dp, blk * WAVES + wave,
                                               reinterpret_cast<uint8_t*>(smem) + wave * dec::kVPageBytes);
  }
  else
    app::append_worker<DT, G, kStages, WAVES>(ap, blk - dec_blocks, (int)gridDim.x - dec_blocks,
                                              smem, s_flag);
}

template <int DT, int WAVES>
hipError_t launch_dt(const AttnParams& dp, const AttnParams& ap, int group, int dec_blocks,
                     int grid, hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL((pod_kernel<DT, 1, WAVES>), dim3(grid), dim3(64 * WAVES), 0, s, dp, ap, dec_blocks); break;
    case 2: hipLaunchKernelGGL((pod_kernel<DT, 2, WAVES>), dim3(grid), dim3(64 * WAVES), 0, s, dp, ap, dec_blocks); break;
    case 4: hipLaunchKernelGGL((pod_kernel<DT, 4, WAVES>), dim3(grid), dim3(64 * WAVES), 0, s, dp, ap, dec_blocks); break;
    case 8:
      // the shared form's 128 columns would hold 16 positions of 8 heads; only
      // the wide form is built for G = 8
      if constexpr (WAVES == 8) {
        hipLaunchKernelGGL((pod_kernel<DT, 8, WAVES>), dim3(grid), dim3(64 * WAVES), 0, s, dp, ap, dec_blocks);
        break;
      } else {
        return hipErrorNotSupported;
      }
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pod(const AttnParams& dp, int workers, const AttnParams& ap, int max_tiles,
                      int dtype, int group, bool wide, hipStream_t s) {
  // decode workgroups first (a multiple of 8, so the append part keeps its
  // XCD bins), then the append grid of the append kernel
  const int per_block = wide ? 8 : 4;
  const int dec_blocks = (workers + 8 * per_block - 1) / (8 * per_block) * 8;
  const int app_blocks = (max_tiles + kAppendBins - 1) / kAppendBins * kAppendBins;
  const int grid = dec_blocks + app_blocks;
  if (grid <= 0) return hipSuccess;
  if (wide)
    return dtype == FA_BF16 ? launch_dt<FA_BF16, 8>(dp, ap, group, dec_blocks, grid, s)
                            : launch_dt<FA_F16, 8>(dp, ap, group, dec_blocks, grid, s);
  return dtype == FA_BF16 ? launch_dt<FA_BF16, 4>(dp, ap, group, dec_blocks, grid, s)
                          : launch_dt<FA_F16, 4>(dp, ap, group, dec_blocks, grid, s);
}

}  // namespace pkfa
