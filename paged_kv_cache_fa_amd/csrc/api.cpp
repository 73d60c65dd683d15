// C ABI: argument validation, plan upload and kernel launches.
//
// Plan/run split as described in [Guide] "FlashInfer: GPU Kernels for LLM
// Inference (2026 Guide)", section "Quickstart" (plan with static geometry
// before graph capture, run with per-launch tensors) and [DeepDive]
// "FlashInfer: The Attention Kernel Library That Proves the Bottleneck ...",
// sections "Snippet One" (caller-owned workspace buffer, plan arguments) and
// "Why This Design Works" (static launch shape, dynamic tile assignment; a
// re-plan does not invalidate the captured launch). Run calls enqueue kernels
// only; their grids depend on the resolved geometry alone.
#include <hip/hip_runtime_api.h>

#include <sched.h>

#include <algorithm>
#include <atomic>
#include <math.h>
#include <string.h>

#include "kernels.h"
#include "plan_internal.h"

namespace pkfa {
static_assert(kAppendBins == kXcdBins, "planner bins and kernel bins differ");
// fa_cascade on one stream: both passes in one kernel (true) or two launches
constexpr bool kCascadeOneLaunch = true;
}  // namespace pkfa

namespace pkfa {
const char* last_error();
}

using namespace pkfa;

namespace {

// Wait until the copy kernel of this plan's last upload out of pinned host
// memory has read the image: each of its workgroups stores the upload's
// sequence number into its word of the host workspace's flag area.
void wait_upload_flags(PlanImpl* pl) {
  if (!pl->flag_ws) return;
  const volatile uint32_t* f = reinterpret_cast<const volatile uint32_t*>(
      static_cast<const uint8_t*>(pl->flag_ws) + pl->lay.host_flags);
  for (int spin = 0;; ++spin) {
    int i = 0;
    while (i < pl->flag_n && f[i] == pl->flag_seq) ++i;
    if (i == pl->flag_n) break;
    if (spin > 256) sched_yield();
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  pl->flag_ws = nullptr;
}

fa_status hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

fa_status check_run_args(const PlanImpl* pl, int want_mode, const void* q, const void* k,
                          const void* v, int64_t page_stride, int64_t token_stride,
                          int64_t head_stride, const int32_t* kv_indices, const int32_t* kv_indptr,
                          const int32_t* last_page_len, const void* out, bool ragged = false) {
  if (!pl || pl->magic != kPlanMagic || !pl->planned) {
    set_error("plan object was not filled by fa_plan");
    return FA_ERR_INVALID;
  }
  if (!pl->uploaded) {
    set_error("plan was built without a device workspace");
    return FA_ERR_NOT_PLANNED;
  }
  if (pl->geom.mode != want_mode) {
    set_error(want_mode == FA_MODE_DECODE ? "plan was made for append, not decode"
                                          : "plan was made for decode, not append");
    return FA_ERR_INVALID;
  }
  if ((pl->ragged != 0) != ragged) {
    set_error(ragged ? "plan was made by fa_plan (paged KV), not fa_plan_ragged"
                     : "plan was made by fa_plan_ragged (ragged KV), not fa_plan");
    return FA_ERR_INVALID;
  }
  if (!q || !k || !v || (!ragged && (!kv_indices || !kv_indptr || !last_page_len)) || !out) {
    set_error("NULL tensor argument");
    return FA_ERR_INVALID;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) {
    set_error("q, K/V pages and out must be 16-byte aligned");
    return FA_ERR_INVALID;
  }
  const int D = pl->geom.head_dim;
  // 16 bytes per stride step: 8 elements of a 16-bit pool, 16 of an E4M3 pool
  const int64_t eb = pl->geom.kv_dtype == FA_E4M3 ? 1 : 2;
  const int64_t step = 16 / eb;
  if (page_stride <= 0 || token_stride < D || head_stride < D || page_stride % step ||
      token_stride % step || head_stride % step ||
      (int64_t)token_stride * eb * pl->geom.page_size > 0x7fffffffLL) {
    set_error("strides must be positive multiples of %d elements with token/head stride >= "
              "head_dim", (int)step);
    return FA_ERR_INVALID;
  }
  return FA_OK;
}

AttnParams make_params(const PlanImpl* pl, const void* q, const void* k, const void* v,
                       int64_t page_stride, int64_t token_stride, int64_t head_stride,
                       const int32_t* kv_indices, const int32_t* kv_indptr,
                       const int32_t* last_page_len, const int32_t* qo_indptr, float sm_scale,
                       void* out, float* lse) {
  const uint8_t* ws = static_cast<const uint8_t*>(pl->dev_ws);
  AttnParams p;
  p.header = reinterpret_cast<const int32_t*>(ws + pl->lay.header);
  p.tiles = reinterpret_cast<const int32_t*>(ws + pl->lay.tiles);
  p.worker_ptr = reinterpret_cast<const int32_t*>(ws + pl->lay.worker_ptr);
  p.merge = reinterpret_cast<const int32_t*>(ws + pl->lay.merge);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.page_stride = page_stride;
  p.token_stride = token_stride;
  p.head_stride = head_stride;
  p.kv_indices = kv_indices;
  p.kv_indptr = kv_indptr;
  p.last_page_len = last_page_len;
  p.qo_indptr = qo_indptr;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.part_o = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + pl->lay.dev_part_o);
  p.part_lse = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + pl->lay.dev_part_lse);
  p.counters = reinterpret_cast<int32_t*>(const_cast<uint8_t*>(ws) + pl->lay.dev_counters);
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)pl->geom.head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.v_scale = 1.0f;
  p.kv_offsets = nullptr;
  p.num_qo_heads = pl->geom.num_qo_heads;
  p.num_kv_heads = pl->geom.num_kv_heads;
  p.defer_merge = 0;
  return p;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_CAPACITY: return "plan capacity exceeded";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_CAPTURING: return "stream is capturing a graph";
    case FA_ERR_NOT_PLANNED: return "plan has no device upload";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return pkfa::last_error(); }

fa_status fa_workspace_size(const fa_geometry* geom, size_t* host_bytes, size_t* device_bytes) {
  fa_geometry g;
  const fa_status st = resolve_geometry(geom, &g);
  if (st != FA_OK) return st;
  const Layout lay = compute_layout(g);
  if (host_bytes) *host_bytes = lay.host_bytes;
  if (device_bytes) *device_bytes = lay.dev_bytes;
  return FA_OK;
}

}  // extern "C"

namespace pkfa {

// fa_plan and fa_plan_ragged (and the no-allocation decode): build on the
// host, upload into dev_ws. Without events no HIP event is created: the call
// instead waits on the stream until the upload has read host_ws.
fa_status plan_upload(fa_plan_t* plan, const fa_geometry* geom, const int32_t* kv_indptr_h,
                      const int32_t* kv_lens_h, int32_t batch, const int32_t* qo_indptr_h,
                      int32_t causal, void* host_ws, size_t host_ws_bytes, void* dev_ws,
                      size_t dev_ws_bytes, void* stream, bool ragged, bool events) {
  if (!plan) {
    set_error("plan is NULL");
    return FA_ERR_INVALID;
  }
  PlanImpl* pl = impl(plan);
  if (pl->magic != kPlanMagic) {
    memset(plan, 0, sizeof(*plan));
    pl->magic = kPlanMagic;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // a copy kernel still reading host_ws must finish before it is rewritten (a
  // copy out of another host workspace leaves this one alone)
  if (pl->flag_ws == host_ws) wait_upload_flags(pl);
  if (dev_ws) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone) {
      set_error("fa_plan copies to the device and cannot be captured; plan before capture");
      return FA_ERR_CAPTURING;
    }
    // the previous copy out of host_ws must finish before host_ws is rewritten
    if (events && pl->upload_event) {
      e = hipEventSynchronize(static_cast<hipEvent_t>(pl->upload_event));
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    }
  }
  pl->planned = 0;
  pl->uploaded = 0;
  fa_geometry g;
  fa_status st = resolve_geometry(geom, &g);
  if (st != FA_OK) return st;
  st = build_plan(pl, g, kv_indptr_h, kv_lens_h, batch, qo_indptr_h, causal, host_ws,
                  host_ws_bytes, ragged);
  if (st != FA_OK) return st;
  pl->planned = 1;
  pl->dev_ws = dev_ws;
  if (!dev_ws) return FA_OK;
  if (dev_ws_bytes < pl->lay.dev_bytes || (reinterpret_cast<uintptr_t>(dev_ws) & 255)) {
    pl->planned = 0;
    set_error("device workspace needs %zu bytes, 256-byte aligned", pl->lay.dev_bytes);
    return FA_ERR_WORKSPACE;
  }
  // Arrival counters return to zero at the end of every run call; clear them
  // when this plan first uses a device workspace, and again whenever a new
  // geometry moves or grows the counter region (fresh memory holds garbage).
  const size_t cbytes = pl->lay.dev_part_lse - pl->lay.dev_counters;
  hipError_t e = hipSuccess;
  if (pl->zeroed_ws != dev_ws || pl->zeroed_off != pl->lay.dev_counters ||
      pl->zeroed_bytes < cbytes) {
    e = hipMemsetAsync(static_cast<uint8_t*>(dev_ws) + pl->lay.dev_counters, 0, cbytes, s);
    if (e != hipSuccess) {
      pl->planned = 0;
      return hip_fail(e, "hipMemsetAsync (arrival counters)");
    }
    pl->zeroed_ws = dev_ws;
    pl->zeroed_off = pl->lay.dev_counters;
    pl->zeroed_bytes = cbytes;
  }
  const size_t bytes = pl->lay.tiles + (size_t)pl->num_tiles * kTileInts * 4;
  // Pinned host workspaces are read by a copy kernel on the stream; pageable
  // ones go through hipMemcpyAsync.
  if (pl->upload_host != host_ws) {
    pl->upload_host = host_ws;
    pl->upload_src = nullptr;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, host_ws) == hipSuccess && attr.type == hipMemoryTypeHost &&
        attr.devicePointer && (reinterpret_cast<uintptr_t>(attr.devicePointer) & 15) == 0)
      pl->upload_src = attr.devicePointer;
    (void)hipGetLastError();  // a pageable pointer leaves an error behind; drop it
  }
  // With events (fa_plan), a copy kernel out of pinned memory reports through
  // the flag area of host_ws; the next fa_plan on this plan waits for it.
  const bool flags = events && pl->upload_src;
  if (flags && (pl->flags_cleared_ws != host_ws || pl->flags_cleared_off != pl->lay.host_flags)) {
    // new flag words: clear whatever the memory held (no copy of this plan
    // is pending on them: fa_plan waited above for any copy out of host_ws)
    memset(static_cast<uint8_t*>(host_ws) + pl->lay.host_flags, 0, kUploadMaxGrid * 4);
    pl->flags_cleared_ws = host_ws;
    pl->flags_cleared_off = pl->lay.host_flags;
  }
  const uint32_t seq = pl->flag_seq + 1 == 0 ? 1 : pl->flag_seq + 1;
  if (pl->upload_src)
    e = launch_upload(static_cast<uint32_t*>(dev_ws), static_cast<const uint32_t*>(pl->upload_src),
                      (int64_t)(bytes / 4),
                      flags ? reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(pl->upload_src) +
                                                          pl->lay.host_flags)
                            : nullptr,
                      seq, s);
  else
    e = hipMemcpyAsync(dev_ws, host_ws, bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) {
    pl->planned = 0;
    return hip_fail(e, "plan upload");
  }
  if (flags) {
    pl->flag_ws = host_ws;
    pl->flag_seq = seq;
    pl->flag_n = upload_grid((int64_t)(bytes / 4));
  }
  if (!events) {
    // no event guards host_ws: wait here until the upload has read it
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      pl->planned = 0;
      return hip_fail(e, "hipStreamSynchronize (plan upload)");
    }
    pl->uploaded = 1;
    return FA_OK;
  }
  for (void** slot : {&pl->upload_event, &pl->fork_event, &pl->join_event, &pl->join2_event}) {
    if (*slot) continue;
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      pl->planned = 0;
      return hip_fail(e, "hipEventCreateWithFlags");
    }
    *slot = ev;
  }
  if (!flags) {
    e = hipEventRecord(static_cast<hipEvent_t>(pl->upload_event), s);
    if (e != hipSuccess) {
      pl->planned = 0;
      return hip_fail(e, "hipEventRecord");
    }
  }
  pl->uploaded = 1;
  return FA_OK;
}

}  // namespace pkfa

extern "C" {

fa_status fa_plan(fa_plan_t* plan, const fa_geometry* geom, const int32_t* kv_indptr_h,
                  const int32_t* kv_lens_h, int32_t batch, const int32_t* qo_indptr_h,
                  int32_t causal, void* host_ws, size_t host_ws_bytes, void* dev_ws,
                  size_t dev_ws_bytes, void* stream) {
  return plan_upload(plan, geom, kv_indptr_h, kv_lens_h, batch, qo_indptr_h, causal, host_ws,
                     host_ws_bytes, dev_ws, dev_ws_bytes, stream, false, true);
}

fa_status fa_plan_ragged(fa_plan_t* plan, const fa_geometry* geom, const int32_t* kv_offsets_h,
                         int32_t batch, const int32_t* qo_indptr_h, int32_t causal,
                         void* host_ws, size_t host_ws_bytes, void* dev_ws, size_t dev_ws_bytes,
                         void* stream) {
  fa_geometry g;
  fa_status st = resolve_geometry(geom, &g);
  if (st != FA_OK) return st;
  if (batch < 0 || batch > g.max_batch || (batch > 0 && !kv_offsets_h)) {
    set_error("batch %d outside [0, %d] or kv_offsets NULL", batch, g.max_batch);
    return FA_ERR_INVALID;
  }
  const Layout lay = compute_layout(g);
  if (!host_ws || host_ws_bytes < lay.host_bytes) {
    set_error("host workspace needs %zu bytes", lay.host_bytes);
    return FA_ERR_WORKSPACE;
  }
  // request lengths into the host-only tail of the workspace (never part of
  // an upload that may still be reading the image)
  int32_t* lens = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(host_ws) + lay.host_lens);
  for (int b = 0; b < batch; ++b) {
    const int64_t L = (int64_t)kv_offsets_h[b + 1] - kv_offsets_h[b];
    if (L < 0) {
      set_error("kv_offsets decrease at request %d", b);
      return FA_ERR_INVALID;
    }
    lens[b] = (int32_t)L;
  }
  return plan_upload(plan, geom, kv_offsets_h, lens, batch, qo_indptr_h, causal, host_ws,
                     host_ws_bytes, dev_ws, dev_ws_bytes, stream, true, true);
}

fa_status fa_block_sparse_pages(const int32_t* block_indptr_h, const int32_t* block_indices_h,
                                int32_t num_row_blocks, const int32_t* col_offsets_h,
                                int32_t num_col_blocks, int32_t page_size, int32_t* kv_indptr_h,
                                int32_t* kv_indices_h, int64_t kv_indices_cap,
                                int32_t* last_page_len_h, int32_t* kv_lens_h, int64_t* num_pages) {
  if (num_row_blocks < 0 || num_col_blocks < 0 || page_size <= 0 || !num_pages ||
      (num_row_blocks > 0 && (!block_indptr_h || !kv_indptr_h || !last_page_len_h ||
                              !kv_lens_h)) ||
      !col_offsets_h || col_offsets_h[0] != 0) {
    set_error("block sparse: bad sizes, NULL table or col_offsets[0] != 0");
    return FA_ERR_INVALID;
  }
  if (num_row_blocks > 0 && block_indptr_h[0] != 0) {
    set_error("block sparse: block_indptr[0] must be 0");
    return FA_ERR_INVALID;
  }
  for (int32_t j = 0; j < num_col_blocks; ++j)
    if (col_offsets_h[j + 1] < col_offsets_h[j]) {
      set_error("block sparse: col_offsets decrease at block %d", j);
      return FA_ERR_INVALID;
    }
  // pass 1: validate and count pages
  int64_t total = 0;
  for (int32_t i = 0; i < num_row_blocks; ++i) {
    const int32_t b0 = block_indptr_h[i], b1 = block_indptr_h[i + 1];
    if (b1 < b0 || (b1 > b0 && !block_indices_h)) {
      set_error("block sparse: block_indptr decreases at row block %d", i);
      return FA_ERR_INVALID;
    }
    for (int32_t n = b0; n < b1; ++n) {
      const int32_t j = block_indices_h[n];
      if (j < 0 || j >= num_col_blocks || (n > b0 && j <= block_indices_h[n - 1])) {
        set_error("block sparse: row block %d: column blocks must be increasing and in range", i);
        return FA_ERR_INVALID;
      }
      const int64_t len = (int64_t)col_offsets_h[j + 1] - col_offsets_h[j];
      if (n + 1 < b1 && len % page_size) {
        set_error("block sparse: row block %d: column block %d of %lld rows is not the row's "
                  "last block and not a whole number of pages", i, j, (long long)len);
        return FA_ERR_INVALID;
      }
      total += (len + page_size - 1) / page_size;
    }
  }
  *num_pages = total;
  if (!kv_indices_h || kv_indices_cap < total) {
    set_error("block sparse: kv_indices needs %lld entries", (long long)total);
    return FA_ERR_CAPACITY;
  }
  // pass 2: page ids are first rows of page_size-row chunks of the blocks
  int64_t k = 0;
  kv_indptr_h[0] = 0;
  for (int32_t i = 0; i < num_row_blocks; ++i) {
    int64_t rows = 0;
    int32_t last = 0;
    for (int32_t n = block_indptr_h[i]; n < block_indptr_h[i + 1]; ++n) {
      const int32_t j = block_indices_h[n];
      const int32_t r0 = col_offsets_h[j], r1 = col_offsets_h[j + 1];
      for (int32_t r = r0; r < r1; r += page_size) {
        kv_indices_h[k++] = r;
        last = std::min(page_size, r1 - r);
      }
      rows += r1 - r0;
    }
    if (rows > 0x7fffffff) {
      set_error("block sparse: row block %d sees more than 2^31 keys", i);
      return FA_ERR_INVALID;
    }
    kv_indptr_h[i + 1] = (int32_t)k;
    kv_lens_h[i] = (int32_t)rows;
    last_page_len_h[i] = last;
  }
  return FA_OK;
}

fa_status fa_plan_info(const fa_plan_t* plan, fa_plan_stats* stats) {
  const PlanImpl* pl = plan ? impl(plan) : nullptr;
  if (!pl || pl->magic != kPlanMagic || !pl->planned || !stats) {
    set_error("plan object was not filled by fa_plan");
    return FA_ERR_INVALID;
  }
  memset(stats, 0, sizeof(*stats));
  stats->num_tiles = pl->num_tiles;
  stats->num_merge = pl->num_merge;
  stats->num_slots = pl->num_slots;
  stats->chunk_pages = pl->chunk_pages;
  stats->batch = pl->batch;
  stats->num_rows = pl->num_rows;
  stats->causal = pl->causal;
  stats->uploaded = pl->uploaded;
  stats->num_workers = pl->num_workers;
  stats->resolved = pl->geom;
  return FA_OK;
}

fa_status fa_plan_tiles(const fa_plan_t* plan, const int32_t** tiles_h, int32_t* num_tiles,
                        const int32_t** merge_h, int32_t* num_merge,
                        const int32_t** worker_ptr_h, int32_t* num_workers) {
  const PlanImpl* pl = plan ? impl(plan) : nullptr;
  if (!pl || pl->magic != kPlanMagic || !pl->planned) {
    set_error("plan object was not filled by fa_plan");
    return FA_ERR_INVALID;
  }
  const uint8_t* ws = static_cast<const uint8_t*>(pl->host_ws);
  if (tiles_h) *tiles_h = reinterpret_cast<const int32_t*>(ws + pl->lay.tiles);
  if (num_tiles) *num_tiles = pl->num_tiles;
  if (merge_h) *merge_h = reinterpret_cast<const int32_t*>(ws + pl->lay.merge);
  if (num_merge) *num_merge = pl->num_merge;
  if (worker_ptr_h)
    *worker_ptr_h = reinterpret_cast<const int32_t*>(ws + pl->lay.worker_ptr);
  if (num_workers) *num_workers = pl->geom.mode == FA_MODE_DECODE ? pl->num_workers : kXcdBins;
  return FA_OK;
}

fa_status fa_plan_destroy(fa_plan_t* plan) {
  if (!plan) return FA_OK;
  PlanImpl* pl = impl(plan);
  if (pl->magic == kPlanMagic) {
    // a pending copy still reads the host workspace and will write its flags
    wait_upload_flags(pl);
    for (void* ev : {pl->upload_event, pl->fork_event, pl->join_event, pl->join2_event})
      if (ev) (void)hipEventDestroy(static_cast<hipEvent_t>(ev));
  }
  memset(plan, 0, sizeof(*plan));
  return FA_OK;
}

fa_status fa_decode_scaled(const fa_plan_t* plan, const void* q, const void* k_pages,
                           const void* v_pages, int64_t page_stride, int64_t token_stride,
                           int64_t head_stride, const int32_t* kv_indices_d,
                           const int32_t* kv_indptr_d, const int32_t* last_page_len_d,
                           float sm_scale, float k_scale, float v_scale, void* out, float* lse,
                           void* stream) {
  const PlanImpl* pl = plan ? impl(plan) : nullptr;
  fa_status st = check_run_args(pl, FA_MODE_DECODE, q, k_pages, v_pages, page_stride,
                                token_stride, head_stride, kv_indices_d, kv_indptr_d,
                                last_page_len_d, out);
  if (st != FA_OK) return st;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !isfinite(k_scale) || !isfinite(v_scale)) {
    set_error("k_scale and v_scale must be finite and positive");
    return FA_ERR_INVALID;
  }
  AttnParams p = make_params(pl, q, k_pages, v_pages, page_stride, token_stride, head_stride,
                             kv_indices_d, kv_indptr_d, last_page_len_d, nullptr, sm_scale, out,
                             lse);
  p.scale_log2 *= k_scale;
  p.v_scale = v_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = pl->geom.num_qo_heads / pl->geom.num_kv_heads;
  const hipError_t e = launch_decode(p, pl->geom.dtype, pl->geom.kv_dtype == FA_E4M3, G,
                                     pl->num_workers, s);
  return e == hipSuccess ? FA_OK : hip_fail(e, "decode kernel launch");
}

fa_status fa_decode(const fa_plan_t* plan, const void* q, const void* k_pages,
                    const void* v_pages, int64_t page_stride, int64_t token_stride,
                    int64_t head_stride, const int32_t* kv_indices_d, const int32_t* kv_indptr_d,
                    const int32_t* last_page_len_d, float sm_scale, void* out, float* lse,
                    void* stream) {
  return fa_decode_scaled(plan, q, k_pages, v_pages, page_stride, token_stride, head_stride,
                          kv_indices_d, kv_indptr_d, last_page_len_d, sm_scale, 1.0f, 1.0f, out,
                          lse, stream);
}

namespace {

// Ragged KV: request b's keys are rows kv_offsets[b] .. kv_offsets[b+1]-1 of
// k / v. The kernels address them as pages of 16 rows that start at row
// kv_offsets[b] + 16 p, i.e. a page id is a row index and the page stride is
// the token stride.
AttnParams ragged_params(const PlanImpl* pl, const void* q, const void* k, const void* v,
                         int64_t token_stride, int64_t head_stride, const int32_t* kv_offsets_d,
                         const int32_t* qo_indptr, float sm_scale, void* out, float* lse) {
  AttnParams p = make_params(pl, q, k, v, token_stride, token_stride, head_stride, nullptr,
                             nullptr, nullptr, qo_indptr, sm_scale, out, lse);
  p.kv_offsets = kv_offsets_d ? kv_offsets_d
                              : reinterpret_cast<const int32_t*>(
                                    static_cast<const uint8_t*>(pl->dev_ws) + pl->lay.offsets);
  return p;
}

}  // namespace

fa_status fa_decode_ragged(const fa_plan_t* plan, const void* q, const void* k, const void* v,
                           int64_t token_stride, int64_t head_stride, const int32_t* kv_offsets_d,
                           float sm_scale, float k_scale, float v_scale, void* out, float* lse,
                           void* stream) {
  const PlanImpl* pl = plan ? impl(plan) : nullptr;
  fa_status st = check_run_args(pl, FA_MODE_DECODE, q, k, v, token_stride, token_stride,
                                head_stride, nullptr, nullptr, nullptr, out, true);
  if (st != FA_OK) return st;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !isfinite(k_scale) || !isfinite(v_scale)) {
    set_error("k_scale and v_scale must be finite and positive");
    return FA_ERR_INVALID;
  }
  AttnParams p = ragged_params(pl, q, k, v, token_stride, head_stride, kv_offsets_d, nullptr,
                               sm_scale, out, lse);
  p.scale_log2 *= k_scale;
  p.v_scale = v_scale;
  const int G = pl->geom.num_qo_heads / pl->geom.num_kv_heads;
  const hipError_t e = launch_decode(p, pl->geom.dtype, pl->geom.kv_dtype == FA_E4M3, G,
                                     pl->num_workers, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e, "decode kernel launch");
}

fa_status fa_append_ragged(const fa_plan_t* plan, const void* q, const int32_t* qo_indptr_d,
                           const void* k, const void* v, int64_t token_stride,
                           int64_t head_stride, const int32_t* kv_offsets_d, float sm_scale,
                           void* out, float* lse, void* stream) {
  const PlanImpl* pl = plan ? impl(plan) : nullptr;
  fa_status st = check_run_args(pl, FA_MODE_APPEND, q, k, v, token_stride, token_stride,
                                head_stride, nullptr, nullptr, nullptr, out, true);
  if (st != FA_OK) return st;
  if (!qo_indptr_d) {
    set_error("qo_indptr is NULL");
    return FA_ERR_INVALID;
  }
  const AttnParams p = ragged_params(pl, q, k, v, token_stride, head_stride, kv_offsets_d,
                                     qo_indptr_d, sm_scale, out, lse);
  const int G = pl->geom.num_qo_heads / pl->geom.num_kv_heads;
  const hipError_t e = launch_append(p, pl->geom.dtype, G, pl->geom.max_tiles,
                                     static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) {
    set_error("append kernel not built for this group size");
    return FA_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? FA_OK : hip_fail(e, "append kernel launch");
}

fa_status fa_append(const fa_plan_t* plan, const void* q, const int32_t* qo_indptr_d,
                    const void* k_pages, const void* v_pages, int64_t page_stride,
                    int64_t token_stride, int64_t head_stride, const int32_t* kv_indices_d,
                    const int32_t* kv_indptr_d, const int32_t* last_page_len_d, float sm_scale,
                    void* out, float* lse, void* stream) {
  const PlanImpl* pl = plan ? impl(plan) : nullptr;
  fa_status st = check_run_args(pl, FA_MODE_APPEND, q, k_pages, v_pages, page_stride,
                                token_stride, head_stride, kv_indices_d, kv_indptr_d,
                                last_page_len_d, out);
  if (st != FA_OK) return st;
  if (!qo_indptr_d) {
    set_error("qo_indptr is NULL");
    return FA_ERR_INVALID;
  }
  const AttnParams p = make_params(pl, q, k_pages, v_pages, page_stride, token_stride,
                                   head_stride, kv_indices_d, kv_indptr_d, last_page_len_d,
                                   qo_indptr_d, sm_scale, out, lse);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = pl->geom.num_qo_heads / pl->geom.num_kv_heads;
  const hipError_t e = launch_append(p, pl->geom.dtype, G, pl->geom.max_tiles, s);
  if (e == hipErrorNotSupported) {
    set_error("append kernel not built for this group size");
    return FA_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? FA_OK : hip_fail(e, "append kernel launch");
}

fa_status fa_cascade(const fa_plan_t* prefix_plan, const fa_plan_t* suffix_plan, const void* q,
                     const void* k_pages, const void* v_pages, int64_t page_stride,
                     int64_t token_stride, int64_t head_stride, const int32_t* prefix_qo_indptr_d,
                     const int32_t* prefix_indices_d, const int32_t* prefix_indptr_d,
                     const int32_t* prefix_last_page_len_d, const int32_t* kv_indices_d,
                     const int32_t* kv_indptr_d, const int32_t* last_page_len_d, float sm_scale,
                     void* prefix_out, float* prefix_lse, void* suffix_out, float* suffix_lse,
                     void* out, float* lse, void* stream, void* prefix_stream,
                     void* suffix_stream) {
  const PlanImpl* pp = prefix_plan ? impl(prefix_plan) : nullptr;
  const PlanImpl* sp = suffix_plan ? impl(suffix_plan) : nullptr;
  fa_status st = check_run_args(pp, FA_MODE_APPEND, q, k_pages, v_pages, page_stride, token_stride,
                                head_stride, prefix_indices_d, prefix_indptr_d,
                                prefix_last_page_len_d, prefix_out);
  if (st != FA_OK) return st;
  st = check_run_args(sp, FA_MODE_DECODE, q, k_pages, v_pages, page_stride, token_stride,
                      head_stride, kv_indices_d, kv_indptr_d, last_page_len_d, suffix_out);
  if (st != FA_OK) return st;
  const fa_geometry& gp = pp->geom;
  const fa_geometry& gs = sp->geom;
  if (pp->causal || pp->batch != 1 || pp->num_rows != sp->batch || gp.dtype != gs.dtype ||
      gs.kv_dtype != gs.dtype ||
      gp.num_qo_heads != gs.num_qo_heads || gp.num_kv_heads != gs.num_kv_heads) {
    set_error("cascade: the prefix plan must be a non-causal append of one request whose rows "
              "are the suffix plan's requests, with the same heads and dtype and 16-bit K/V "
              "pages");
    return FA_ERR_INVALID;
  }
  if (!prefix_qo_indptr_d || !prefix_lse || !suffix_lse || !out || !aligned16(out) ||
      !aligned16(prefix_out) || !aligned16(suffix_out)) {
    set_error("cascade: NULL or misaligned state / output buffer");
    return FA_ERR_INVALID;
  }
  // every prefix q tile sees the same keys, so either none or all of its
  // (q tile, kv head) units split, with merge entries in that order
  const int64_t units = (int64_t)(sp->batch + gp.qo_tile - 1) / gp.qo_tile * gp.num_kv_heads;
  if (pp->num_merge != 0 && pp->num_merge != units) {
    set_error("cascade: unexpected prefix split layout");
    return FA_ERR_INVALID;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t s_pre = prefix_stream ? static_cast<hipStream_t>(prefix_stream) : s;
  hipStream_t s_suf = suffix_stream ? static_cast<hipStream_t>(suffix_stream) : s;
  const bool fork_pre = s_pre != s, fork_suf = s_suf != s;
  hipError_t e = hipSuccess;
  if (fork_pre || fork_suf) {
    if (!sp->fork_event || !sp->join_event || !sp->join2_event) {
      set_error("cascade: the suffix plan was not uploaded to a device workspace");
      return FA_ERR_NOT_PLANNED;
    }
    e = hipEventRecord(static_cast<hipEvent_t>(sp->fork_event), s);
    if (e == hipSuccess && fork_pre)
      e = hipStreamWaitEvent(s_pre, static_cast<hipEvent_t>(sp->fork_event), 0);
    if (e == hipSuccess && fork_suf)
      e = hipStreamWaitEvent(s_suf, static_cast<hipEvent_t>(sp->fork_event), 0);
    if (e != hipSuccess) return hip_fail(e, "cascade fork");
  }
  // suffix decode (HBM-bound) and the shared-prefix pass (MFMA-bound)
  const int G = gs.num_qo_heads / gs.num_kv_heads;
  const AttnParams ps = make_params(sp, q, k_pages, v_pages, page_stride, token_stride, head_stride,
                                    kv_indices_d, kv_indptr_d, last_page_len_d, nullptr, sm_scale,
                                    suffix_out, suffix_lse);
  AttnParams pa = make_params(pp, q, k_pages, v_pages, page_stride, token_stride, head_stride,
                              prefix_indices_d, prefix_indptr_d, prefix_last_page_len_d,
                              prefix_qo_indptr_d, sm_scale, prefix_out, prefix_lse);
  pa.defer_merge = 1;  // the prefix chunks are merged together with the suffix below
  const bool wide = gp.qo_tile > kPodCols / G;
  if (!fork_pre && !fork_suf && kCascadeOneLaunch && gp.qo_tile <= kPodWideCols / G &&
      (G <= 4 || wide)) {
    // both passes in one launch: q tiles of up to 128 / G positions share each
    // CU with a decode workgroup (G <= 4), wider ones take whole CUs beside
    // the decode's
    e = launch_pod(ps, sp->num_workers, pa, gp.max_tiles, gs.dtype, G, wide, s);
    if (e != hipSuccess) return hip_fail(e, "cascade kernel launch");
  } else {
    e = launch_decode(ps, gs.dtype, false, G, sp->num_workers, s_suf);
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    e = launch_append(pa, gp.dtype, G, gp.max_tiles, s_pre);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  }
  if (fork_pre) {
    e = hipEventRecord(static_cast<hipEvent_t>(sp->join_event), s_pre);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(sp->join_event), 0);
    if (e != hipSuccess) return hip_fail(e, "cascade join");
  }
  if (fork_suf) {
    e = hipEventRecord(static_cast<hipEvent_t>(sp->join2_event), s_suf);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(sp->join2_event), 0);
    if (e != hipSuccess) return hip_fail(e, "cascade join");
  }
  // grid from the suffix geometry's max_batch; the kernel reads the batch of
  // the current suffix plan from its uploaded header
  e = launch_cascade_merge(pa.header, pa.merge, pa.part_o, pa.part_lse, prefix_out, prefix_lse,
                           suffix_out, suffix_lse, out, lse, ps.header, gs.max_batch,
                           gs.num_qo_heads, G, gs.num_kv_heads, gp.qo_tile, gs.dtype, s);
  return e == hipSuccess ? FA_OK : hip_fail(e, "cascade merge kernel launch");
}

fa_status fa_pod(const fa_plan_t* prefill_plan, const void* q_p, const int32_t* qo_indptr_p_d,
                 const int32_t* kv_indices_p_d, const int32_t* kv_indptr_p_d,
                 const int32_t* last_page_len_p_d, void* out_p, float* lse_p,
                 const fa_plan_t* decode_plan, const void* q_d, const int32_t* kv_indices_d,
                 const int32_t* kv_indptr_d, const int32_t* last_page_len_d, void* out_d,
                 float* lse_d, const void* k_pages, const void* v_pages, int64_t page_stride,
                 int64_t token_stride, int64_t head_stride, float sm_scale, void* stream) {
  const PlanImpl* pp = prefill_plan ? impl(prefill_plan) : nullptr;
  const PlanImpl* dp = decode_plan ? impl(decode_plan) : nullptr;
  fa_status st = check_run_args(pp, FA_MODE_APPEND, q_p, k_pages, v_pages, page_stride,
                                token_stride, head_stride, kv_indices_p_d, kv_indptr_p_d,
                                last_page_len_p_d, out_p);
  if (st != FA_OK) return st;
  st = check_run_args(dp, FA_MODE_DECODE, q_d, k_pages, v_pages, page_stride, token_stride,
                      head_stride, kv_indices_d, kv_indptr_d, last_page_len_d, out_d);
  if (st != FA_OK) return st;
  const fa_geometry& ga = pp->geom;
  const fa_geometry& gd = dp->geom;
  const int G = gd.num_qo_heads / gd.num_kv_heads;
  // prefill tiles wider than the shared form's take the append kernel's
  // workgroup shape (one role per CU at a time); G = 8 has only that shape
  const bool wide = ga.qo_tile > kPodCols / G;
  if (!qo_indptr_p_d || ga.dtype != gd.dtype || ga.num_qo_heads != gd.num_qo_heads ||
      ga.num_kv_heads != gd.num_kv_heads || gd.kv_dtype != gd.dtype || (G > 4 && !wide) ||
      ga.qo_tile > kPodWideCols / G) {
    set_error("pod: the plans need the same dtype and heads, 16-bit K/V pages, a prefill "
              "qo_tile of at most 256 / G (more than 128 / G for num_qo_heads / num_kv_heads "
              "= 8) and qo_indptr");
    return FA_ERR_INVALID;
  }
  const AttnParams pa = make_params(pp, q_p, k_pages, v_pages, page_stride, token_stride,
                                    head_stride, kv_indices_p_d, kv_indptr_p_d, last_page_len_p_d,
                                    qo_indptr_p_d, sm_scale, out_p, lse_p);
  const AttnParams pd = make_params(dp, q_d, k_pages, v_pages, page_stride, token_stride,
                                    head_stride, kv_indices_d, kv_indptr_d, last_page_len_d,
                                    nullptr, sm_scale, out_d, lse_d);
  const hipError_t e = launch_pod(pd, dp->num_workers, pa, ga.max_tiles, gd.dtype, G, wide,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e, "pod kernel launch");
}

fa_status fa_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                         void* v_out, float* s_out, int64_t n, int32_t heads, int32_t head_dim,
                         int32_t dtype, void* stream) {
  if (n < 0 || heads <= 0 || head_dim <= 0 || (head_dim & 7) ||
      (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_F32)) {
    set_error("merge_state: bad sizes or dtype");
    return FA_ERR_INVALID;
  }
  if (n == 0) return FA_OK;
  if (!v_a || !s_a || !v_b || !s_b || !v_out || !aligned16(v_a) || !aligned16(v_b) ||
      !aligned16(v_out)) {
    set_error("merge_state: NULL or misaligned buffer");
    return FA_ERR_INVALID;
  }
  hipError_t e = launch_merge_state(v_a, s_a, v_b, s_b, v_out, s_out, n, heads, head_dim, dtype,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e, "merge_state kernel launch");
}

fa_status fa_merge_states(const void* v, const float* s, int64_t n, int32_t k, int32_t heads,
                          int32_t head_dim, int32_t dtype, void* v_out, float* s_out,
                          void* stream) {
  if (n < 0 || k < 0 || heads <= 0 || head_dim <= 0 || (head_dim & 7) ||
      (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_F32)) {
    set_error("merge_states: bad sizes or dtype");
    return FA_ERR_INVALID;
  }
  if (n == 0) return FA_OK;
  if ((k > 0 && (!v || !s || !aligned16(v))) || !v_out || !aligned16(v_out)) {
    set_error("merge_states: NULL or misaligned buffer");
    return FA_ERR_INVALID;
  }
  hipError_t e = launch_merge_states(v, s, n, k, heads, head_dim, dtype, v_out, s_out,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e, "merge_states kernel launch");
}

}  // extern "C"
