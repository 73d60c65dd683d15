// Batched paged decode that allocates nothing: fa_plan + fa_decode in one call,
// with the device workspace (uploaded plan image, arrival counters, fp32
// partial states) in a file-scope device array and the host plan workspace in
// a static host array, one of each per GPU. The call waits on its stream
// until the plan upload is done (work queued earlier on the stream included),
// then queues the decode kernel. For callers that cannot allocate
// device memory (serving loops that forbid it, harnesses without an
// allocator); the other entry points take caller-owned workspaces instead.
//
// The array's name is a host-side stand-in in host code: its device address
// is looked up once per GPU with hipGetSymbolAddress (with that GPU current)
// and only that address is passed to kernels and memsets. Calls on one GPU
// share its arrays: the arrival counters are cleared whenever the layout they
// sit in changes and are returned to zero by the decode kernel itself, and
// calls that overlap on one GPU (other streams, other host threads) race.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "plan_internal.h"

namespace pkfa {
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;   // device workspace per GPU
constexpr size_t kStaticHostBytes = size_t(1) << 20;  // host plan workspace per GPU
constexpr int kMaxDevices = 16;
}  // namespace
}  // namespace pkfa

static __device__ __align__(256) uint8_t scratch[pkfa::kScratchBytes];

namespace pkfa {
namespace {

struct DeviceSlot {
  int ready;        // 1 once `ptr` was looked up on this GPU
  void* ptr;        // device address of `scratch` on this GPU
  fa_plan_t plan;   // the plan kept between calls (tracks the cleared counter layout)
};
DeviceSlot g_slots[kMaxDevices];
alignas(256) uint8_t g_host[kMaxDevices][kStaticHostBytes];

}  // namespace
}  // namespace pkfa

extern "C" fa_status fa_decode_noalloc(const fa_geometry* geom, const int32_t* kv_indptr_h,
                                       const int32_t* kv_lens_h, int32_t batch, const void* q,
                                       const void* k_pages, const void* v_pages,
                                       int64_t page_stride, int64_t token_stride,
                                       int64_t head_stride, const int32_t* kv_indices_d,
                                       const int32_t* kv_indptr_d,
                                       const int32_t* last_page_len_d, float sm_scale, void* out,
                                       float* lse, void* stream) {
  using namespace pkfa;
  if (!geom || geom->mode != FA_MODE_DECODE) {
    set_error("fa_decode_noalloc: needs a decode geometry");
    return FA_ERR_INVALID;
  }
  size_t host_bytes = 0, dev_bytes = 0;
  fa_status st = fa_workspace_size(geom, &host_bytes, &dev_bytes);
  if (st != FA_OK) return st;
  if (dev_bytes > kScratchBytes || host_bytes > kStaticHostBytes) {
    set_error("fa_decode_noalloc: the geometry needs %zu device / %zu host workspace bytes, "
              "more than the static %zu / %zu (use fa_plan + fa_decode with caller-owned "
              "workspaces)", dev_bytes, host_bytes, kScratchBytes, kStaticHostBytes);
    return FA_ERR_CAPACITY;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("fa_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("fa_decode_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    return FA_ERR_UNSUPPORTED;
  }
  DeviceSlot& slot = g_slots[dev];
  if (!slot.ready) {
    e = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !slot.ptr) {
      set_error("fa_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return FA_ERR_HIP;
    }
    slot.ready = 1;
  }
  // the static host array is pageable: the plan is copied with hipMemcpyAsync
  // and the call waits on the stream for that copy (no event is created), so
  // the next call may rewrite the array
  st = plan_upload(&slot.plan, geom, kv_indptr_h, kv_lens_h, batch, nullptr, 0, g_host[dev],
                   kStaticHostBytes, slot.ptr, kScratchBytes, stream, false, false);
  if (st != FA_OK) return st;
  return fa_decode(&slot.plan, q, k_pages, v_pages, page_stride, token_stride, head_stride,
                   kv_indices_d, kv_indptr_d, last_page_len_d, sm_scale, out, lse, stream);
}
