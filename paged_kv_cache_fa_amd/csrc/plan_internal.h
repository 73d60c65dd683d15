// Internal plan object and workspace layout. Host-only C++ (no HIP headers),
// so the planner builds and is tested with a plain host compiler too.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/fa.h"

namespace pkfa {

constexpr uint32_t kPlanMagic = 0x70666131u;  // "pfa1"
constexpr int kTileInts = 8;                   // {b, h, row0, row1, key0, key1, slot0, nchunk}
constexpr int kMergeInts = 4;                  // {row0, kv_head, base slot, n_chunks}
constexpr int kHeaderInts = 16;  // {num_tiles, num_merge, batch, num_rows, causal, chunk_pages, num_workers, ragged, ...}
constexpr int kSupportedHeadDim = 128;
constexpr int kSupportedPageSize = 16;
constexpr int kMaxPiecePages = 128;  // decode pieces: the kernel holds 128 page ids per wave
constexpr int kXcdBins = 8;          // append tile bins, one per XCD (workgroup i runs on XCD i % 8)
constexpr int kAppendCols = 256;     // query columns of an append tile: G heads x 256 / G positions
constexpr int kPiecesPerWorker = 1;  // decode: work lists per worker wave
constexpr int kUploadMaxGrid = 64;   // workgroups of the plan copy kernel (one flag word each)
// decode: set-up and epilogue of one piece, in pages of streaming time
constexpr int kPieceCostPages16 = 4;
constexpr int kPieceCostPagesE4M3 = 8;

// Byte offsets of the regions inside the host and device workspaces.
// Upload image (same offsets in host and device workspace):
//   header | merge [max_merge][4] | tile offsets (decode: [workers+1] per
//   worker wave; append: [9] per XCD bin) | ragged KV row offsets
//   [max_batch+1] | tiles [max_tiles][8]
// Device only: arrival counters [max_partials] (zero between calls), partial
// lse [max_partials][G] (log2 units), partial out [max_partials][G][head_dim].
// Host only: scratch for sorting and dealing tiles (decode: pieces, dealing
// order, bin heap, bin of each dealt piece, bin offsets; append: per-group
// cost / order / bin / sequence), per-request / per-unit counts, and the
// request lengths of a ragged plan, and the completion words of the copy
// kernel that reads the image out of pinned host memory ([kUploadMaxGrid]).
struct Layout {
  size_t header, merge, worker_ptr, offsets, tiles, upload_end;
  size_t dev_counters, dev_part_lse, dev_part_o, dev_bytes;
  size_t host_unsorted, host_order, host_cost, host_bin, host_seg, host_units, host_lens,
      host_flags, host_bytes;
  int32_t workers;
};

struct PlanImpl {
  uint32_t magic;
  int32_t planned;    // 1 after a successful fa_plan
  int32_t uploaded;   // 1 if the plan was copied into a device workspace
  int32_t num_tiles, num_merge, num_slots, chunk_pages, batch, num_rows, causal, num_workers;
  int32_t ragged;     // 1: planned by fa_plan_ragged (contiguous KV rows, no page table)
  fa_geometry geom;   // resolved
  Layout lay;
  void* host_ws;
  void* dev_ws;
  void* upload_event;  // hipEvent_t recorded after the copy out of host_ws
  void* zeroed_ws;     // device workspace whose counters were cleared,
  size_t zeroed_off;   // at this offset,
  size_t zeroed_bytes; // this many bytes
  void* fork_event;    // hipEvent_t fork / join events for the cascade call's streams
  void* join_event;
  void* join2_event;
  void* upload_host;   // host workspace whose device mapping was looked up
  void* upload_src;    // its device-visible address (pinned memory), or null
  // Completion words of the last copy kernel out of pinned host memory: each
  // of its `flag_n` workgroups stores `flag_seq` into its word of the host
  // workspace's flag area once its reads are done. flag_ws is null when no
  // such copy is pending.
  void* flag_ws;
  uint32_t flag_seq;
  int32_t flag_n;
  void* flags_cleared_ws;  // host workspace whose flag area holds no stale
  size_t flags_cleared_off;  // word at this offset
};
static_assert(sizeof(PlanImpl) <= sizeof(fa_plan_t), "plan object too large");

inline PlanImpl* impl(fa_plan_t* p) { return reinterpret_cast<PlanImpl*>(p); }
inline const PlanImpl* impl(const fa_plan_t* p) { return reinterpret_cast<const PlanImpl*>(p); }

// Fill default knobs and check the geometry. Returns FA_OK or an error code.
fa_status resolve_geometry(const fa_geometry* in, fa_geometry* out);
Layout compute_layout(const fa_geometry& g);

// Build the plan into the host workspace (upload image + scratch). Host only.
// With ragged, kv_indptr holds the requests' first KV rows (batch+1 offsets,
// copied into the image) instead of page offsets.
fa_status build_plan(PlanImpl* p, const fa_geometry& g, const int32_t* kv_indptr,
                     const int32_t* kv_lens, int32_t batch, const int32_t* qo_indptr,
                     int32_t causal, void* host_ws, size_t host_ws_bytes, bool ragged);

void set_error(const char* fmt, ...);

// fa_plan's body (api.cpp): plan into host_ws and upload into dev_ws on
// `stream` (a hipStream_t). With events false no HIP event is created: the
// call waits on the stream until the upload has read host_ws.
fa_status plan_upload(fa_plan_t* plan, const fa_geometry* geom, const int32_t* kv_indptr_h,
                      const int32_t* kv_lens_h, int32_t batch, const int32_t* qo_indptr_h,
                      int32_t causal, void* host_ws, size_t host_ws_bytes, void* dev_ws,
                      size_t dev_ws_bytes, void* stream, bool ragged, bool events);

}  // namespace pkfa
