// Kernel parameter blocks and launchers (host side of the kernels).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pkfa {

// One work tile = {request, kv_head, row_begin, row_end, key_begin, key_end,
// slot0, n_chunks} (int32 x 8), read from the device workspace.
struct AttnParams {
  const int32_t* header;      // {num_tiles, num_merge, ...}
  const int32_t* tiles;
  const int32_t* worker_ptr;  // decode: [workers+1] tile range of each worker wave
  const int32_t* merge;
  const uint16_t* q;          // [rows, Hq, 128]
  const uint16_t* k;          // page pools (16-bit elements, or E4M3 bytes)
  const uint16_t* v;
  int64_t page_stride, token_stride, head_stride;  // elements of the pool type
  const int32_t* kv_indices;
  const int32_t* kv_indptr;
  const int32_t* last_page_len;
  const int32_t* qo_indptr;   // append only
  const int32_t* kv_offsets;  // ragged KV: request b's keys are rows kv_offsets[b] ..
                              // kv_offsets[b+1]-1, a page id is a row index; null: paged
  uint16_t* out;              // [rows, Hq, 128]
  float* lse;                 // [rows, Hq] natural log, may be null
  float* part_o;              // [slots, G, 128] fp32 partial outputs (normalised)
  float* part_lse;            // [slots, G] partial lse in log2 units
  int32_t* counters;          // [slots] arrivals per split unit, indexed by its first slot
  float scale_log2;           // sm_scale * k_scale * log2(e)
  float v_scale;              // per-tensor V scale, applied to the final output
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t defer_merge;        // append: split tiles only publish their partial states
};

constexpr int kAppendBins = 8;  // append tile bins = XCDs (workgroup i runs bin i % 8)

// kv_e4m3: the K/V pools hold E4M3 codes (strides in bytes) instead of dtype.
hipError_t launch_decode(const AttnParams& p, int dtype, bool kv_e4m3, int group, int workers,
                         hipStream_t s);
hipError_t launch_append(const AttnParams& p, int dtype, int group, int max_tiles, hipStream_t s);
// Decode workers (dp, `workers` waves) and append tiles (ap, its max_tiles
// grid) in one launch; group 1, 2 or 4. Shared form (wide = false): 4-wave
// workgroups, a decode and an append workgroup per CU, append tiles of at
// most kPodCols / group query positions. Wide form: the append kernel's
// 8-wave workgroups and LDS ring (tiles of up to kPodWideCols / group
// positions), one workgroup and so one role per CU at a time.
constexpr int kPodCols = 128;
constexpr int kPodWideCols = 256;
hipError_t launch_pod(const AttnParams& dp, int workers, const AttnParams& ap, int max_tiles,
                      int dtype, int group, bool wide, hipStream_t s);
// Copy n_words 32-bit words from device-visible pinned host memory into device
// memory with a small kernel (both 16-byte aligned).
// Copy n_words from src (device-visible host memory) to dst; when flags is not
// null, workgroup i stores seq into flags[i] once its reads are done.
int upload_grid(int64_t n_words);
hipError_t launch_upload(uint32_t* dst, const uint32_t* src, int64_t n_words, uint32_t* flags,
                         uint32_t seq, hipStream_t s);
hipError_t launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                              void* vo, float* so, int64_t n, int heads, int head_dim, int dtype,
                              hipStream_t s);
// Cascade combine: out[r, h] = merge of the shared-prefix state of (r, h)
// (the prefix plan's deferred chunk partials, or prefix_out / prefix_lse when
// that plan did not split) with the suffix state, for the suffix plan's
// current batch (header word 2, at most max_n rows: the grid's size).
hipError_t launch_cascade_merge(const int32_t* prefix_header, const int32_t* prefix_merge,
                                const float* part_o, const float* part_lse, const void* prefix_out,
                                const float* prefix_lse, const void* suffix_out,
                                const float* suffix_lse, void* out, float* lse,
                                const int32_t* suffix_header, int64_t max_n, int heads, int group,
                                int num_kv_heads, int qo_tile, int dtype, hipStream_t s);
hipError_t launch_merge_states(const void* v, const float* s, int64_t n, int k, int heads,
                               int head_dim, int dtype, void* vo, float* so, hipStream_t st);

}  // namespace pkfa
