/*
 * fa.h -- C ABI of the paged-KV attention library for AMD Instinct MI355X (gfx950).
 *
 * What the library computes is described on these pages (cited by title and
 * section):
 *
 *  [Guide]    "FlashInfer: GPU Kernels for LLM Inference (2026 Guide)":
 *             "What FlashInfer is" (block-sparse KV format; load-balanced
 *             scheduling that stays compatible with graphs), "Cascade attention
 *             for shared prefixes" (merge_state / merge_states), "Quickstart"
 *             (plan step with static geometry before graph capture, run step
 *             with per-launch tensors; NHD layout by default).
 *  [DeepDive] "FlashInfer: The Attention Kernel Library That Proves the
 *             Bottleneck in LLM Inference Was Never the Model. It Was the
 *             Memory Access Pattern.": "Snippet One: Paged KV-Cache Attention
 *             and MLA" (page pool, CSR page table, last_page_len, caller-owned
 *             workspace buffer, plan arguments), "It In Action" step 1 (a
 *             per-step plan builds the tile-to-request map), "Why This Design
 *             Works" (static launch geometry, dynamic assignment).
 *
 * Conventions shared by every entry point:
 *  - Every call returns fa_status; nothing throws and nothing aborts.
 *  - The library never allocates or frees device memory. Every device buffer
 *    (queries, pages, page tables, outputs, workspace) is owned by the caller
 *    and must stay alive until the work enqueued on `stream` has finished.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream. Run
 *    calls (fa_decode, fa_append, fa_merge_state, fa_merge_states) only
 *    enqueue kernels: no synchronisation, no allocation, no host-to-device
 *    copy, and their launch shapes depend only on the fa_geometry a plan was
 *    made with. They may therefore be captured in a hipGraph, and a captured
 *    graph stays valid when fa_plan is called again with the same geometry and
 *    workspace pointers (the plan rewrites the device workspace the graph
 *    reads). fa_plan itself copies to the device and refuses to run on a
 *    capturing stream.
 *  - Scores use natural-log log-sum-exp (`lse = log(sum_j exp(s_j))`) and
 *    `s_j = sm_scale * <q, k_j>`; `sm_scale <= 0` selects 1/sqrt(head_dim).
 *  - Query head h reads kv head h / (num_qo_heads / num_kv_heads).
 *  - Supported: head_dim 128, page_size 16, num_qo_heads / num_kv_heads in
 *    {1, 2, 4, 8}, fp16 or bf16 q / K / V / out with fp32 accumulation, and
 *    for decode also FP8 (E4M3) K/V pages under fp16 or bf16 q / out. Other
 *    shapes return FA_ERR_UNSUPPORTED.
 */
#ifndef PAGED_KV_FA_H_
#define PAGED_KV_FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fa_status;
#define FA_OK 0
#define FA_ERR_INVALID (-1)     /* bad argument, inconsistent page table, misaligned pointer */
#define FA_ERR_UNSUPPORTED (-2) /* head_dim / page_size / group size / dtype not built */
#define FA_ERR_WORKSPACE (-3)   /* a workspace is missing or smaller than fa_workspace_size */
#define FA_ERR_CAPACITY (-4)    /* more tiles / partial states / merge rows than the geometry allows */
#define FA_ERR_HIP (-5)         /* a HIP runtime call failed (fa_last_error names it) */
#define FA_ERR_CAPTURING (-6)   /* fa_plan called on a stream that is capturing a graph */
#define FA_ERR_NOT_PLANNED (-7) /* run call with a plan that has no device upload */

/* FA_E4M3: OCP 8-bit floating point E4M3 (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, subnormals, no infinities, NaN = S.1111.111, max 448), one
 * byte per element; a K/V page-pool type only (fa_geometry.kv_dtype). */
typedef enum { FA_F16 = 0, FA_BF16 = 1, FA_F32 = 2, FA_E4M3 = 3 } fa_dtype;
typedef enum { FA_MODE_DECODE = 0, FA_MODE_APPEND = 1 } fa_mode;

/* Static geometry: fixed for the life of a captured graph. Zero knobs take
 * defaults; the resolved values are reported by fa_plan_info. */
typedef struct {
  int32_t mode;            /* fa_mode: decode (one query row per request) or append */
  int32_t dtype;           /* fa_dtype of q, K/V pages and out (FA_F16 or FA_BF16) */
  int32_t max_batch;       /* upper bound on the number of requests */
  int32_t max_qo_tokens;   /* append: upper bound on packed query rows; ignored for decode */
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;        /* 128 */
  int32_t page_size;       /* 16 */
  /* plan knobs (0 = default) */
  int32_t num_cu;          /* compute units to spread tiles over (default 256) */
  int32_t tiles_per_cu;    /* decode: worker waves per compute unit (default 4); append: tiles per CU (default 2) */
  int32_t min_chunk_pages; /* smallest split-KV chunk / decode piece size in pages (default 1) */
  int32_t qo_tile;         /* append: query rows per tile, 1..256/G (default 256/G,
                              G = num_qo_heads / num_kv_heads); decode: 1 */
  int32_t max_tiles;       /* capacities; the defaults cover every plan whose total pages
                              (plus 4 or 8 per request) stay within 128 pages per bin (decode:
                              bins = num_cu * tiles_per_cu * pieces_per_worker / num_kv_heads),
                              and append plans up to max_qo_tokens rows; larger plans return
                              FA_ERR_CAPACITY */
  int32_t max_partials;
  int32_t max_merge;
  int32_t pieces_per_worker; /* decode: work lists per worker wave (default 1) */
  int32_t kv_dtype;        /* K/V page-pool type: 0 or `dtype` = the same as q; FA_E4M3 = FP8
                              pages with per-tensor scales (decode only, see fa_decode_scaled).
                              Resolved to `dtype` when the same. */
  int32_t reserved[7];
} fa_geometry;

/* Caller-allocated plan object. Zero it before first use; release the HIP
 * event it may hold with fa_plan_destroy. Not shared between streams that run
 * concurrently. */
typedef struct {
  uint64_t opaque[64];
} fa_plan_t;

typedef struct {
  int32_t num_tiles;       /* work tiles in the current plan */
  int32_t num_merge;       /* query rows whose state is split over several tiles */
  int32_t num_slots;       /* fp32 partial states in use */
  int32_t chunk_pages;     /* split-KV chunk length (append) / piece size (decode) in pages */
  int32_t batch;
  int32_t num_rows;        /* query rows (batch for decode) */
  int32_t causal;
  int32_t uploaded;        /* 1 if the plan was copied to a device workspace */
  int32_t num_workers;     /* decode: worker waves (num_cu * tiles_per_cu); append: 0 */
  fa_geometry resolved;    /* geometry with every default filled in */
} fa_plan_stats;

/* Host and device workspace sizes in bytes for a geometry ([DeepDive]
 * "Snippet One": the caller allocates the decode wrapper's workspace buffer
 * once and the plan and run calls work inside it; here the two sizes are
 * exact for the geometry instead of a fixed 128 MB). Either output may be
 * NULL. Errors: FA_ERR_INVALID / FA_ERR_UNSUPPORTED for a bad geometry. */
fa_status fa_workspace_size(const fa_geometry* geom, size_t* host_bytes, size_t* device_bytes);

/* Build the split-KV work plan on the host ([Guide] "What FlashInfer is",
 * idea 3; [DeepDive] "It In Action" step 1) and copy it into `dev_ws` on
 * `stream`.
 *
 *  kv_indptr_h  host int32 [batch+1]: CSR offsets of each request's pages in
 *               kv_indices (must start at 0 and be non-decreasing).
 *  kv_lens_h    host int32 [batch]: valid tokens per request; must satisfy
 *               (n_b-1)*page_size < kv_len <= n_b*page_size for n_b pages, or
 *               0 with no pages.
 *  qo_indptr_h  host int32 [batch+1] for append (packed query rows of each
 *               request), NULL for decode.
 *  causal       append: row i of a request with qo_len new rows sees keys
 *               0 .. kv_len - qo_len + i (its new tokens are already in the
 *               pages); ignored for decode.
 *  host_ws      caller host memory of fa_workspace_size's host_bytes (pinned
 *               memory recommended). Pinned: a copy kernel on `stream` reads
 *               the image out of it and then stores a sequence number into
 *               completion words at its end; pageable: hipMemcpyAsync and a
 *               HIP event. Either way fa_plan waits for its own previous copy
 *               out of host_ws before writing it again; other plans must not
 *               use the same host_ws.
 *  dev_ws       caller device memory of device_bytes, 256-byte aligned, or
 *               NULL to plan on the host only (no HIP call is made; the plan
 *               can then be inspected but not run).
 * Errors: FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_CAPACITY,
 * FA_ERR_CAPTURING, FA_ERR_HIP. On error the previous plan is unusable. */
fa_status fa_plan(fa_plan_t* plan, const fa_geometry* geom, const int32_t* kv_indptr_h,
                  const int32_t* kv_lens_h, int32_t batch, const int32_t* qo_indptr_h,
                  int32_t causal, void* host_ws, size_t host_ws_bytes, void* dev_ws,
                  size_t dev_ws_bytes, void* stream);

/* Plan over a ragged (contiguous) KV cache instead of a paged one ([Guide]
 * "What FlashInfer is", idea 1: one block-sparse format describes a ragged
 * tensor as well as a page table; [DeepDive] "Snippet One": single-request
 * decode over a contiguous KV cache). Request b's keys are rows
 * kv_offsets_h[b] .. kv_offsets_h[b+1]-1 of K / V tensors [total_rows,
 * num_kv_heads, head_dim]; a single request over a contiguous K / V is the
 * batch-1 case (kv_offsets {0, kv_len}).
 *  kv_offsets_h  host int32 [batch+1], starting at 0 and non-decreasing.
 * The offsets are also copied into the device workspace, where run calls read
 * them when given no device copy. The work plan is the one fa_plan makes for
 * the same lengths (page_size rows standing for a page). Other arguments and
 * errors as fa_plan. Run the plan with fa_decode_ragged / fa_append_ragged
 * only; the paged run calls refuse it (and these refuse fa_plan's plans). */
fa_status fa_plan_ragged(fa_plan_t* plan, const fa_geometry* geom, const int32_t* kv_offsets_h,
                         int32_t batch, const int32_t* qo_indptr_h, int32_t causal,
                         void* host_ws, size_t host_ws_bytes, void* dev_ws, size_t dev_ws_bytes,
                         void* stream);

/* Page table of a block-sparse pattern ([Windows] "Core Features", Attention
 * Kernels: block-sparse and variable block-sparse patterns; [Guide] "What
 * FlashInfer is", idea 1: one block-sparse format covers them with the page
 * table). Query rows are cut into row blocks and keys into column blocks:
 * column block j is rows col_offsets_h[j] .. col_offsets_h[j+1]-1 of K / V
 * [rows, num_kv_heads, head_dim] (equal sizes: BSR; any sizes: variable
 * block-sparse). Row block i attends to the keys of column blocks
 * block_indices_h[block_indptr_h[i] .. block_indptr_h[i+1]-1] (increasing;
 * every block but a row block's last one a whole number of pages). Host only,
 * no HIP call.
 * Output: a paged table over the same K / V whose page ids are row indices
 * (chunks of page_size rows of the selected blocks): kv_indptr_h int32
 * [num_row_blocks+1], kv_indices_h int32 [*num_pages] (row of each page),
 * last_page_len_h and kv_lens_h int32 [num_row_blocks]. Plan it with fa_plan
 * (decode when every row block is one query row, else append with qo_indptr =
 * the row blocks' row offsets, non-causal) and run fa_decode / fa_append with
 * page_stride = token_stride.
 * *num_pages always receives the page count; kv_indices_h may be NULL (or
 * kv_indices_cap too small) to ask for it: FA_ERR_CAPACITY. Errors:
 * FA_ERR_INVALID for a malformed pattern. */
fa_status fa_block_sparse_pages(const int32_t* block_indptr_h, const int32_t* block_indices_h,
                                int32_t num_row_blocks, const int32_t* col_offsets_h,
                                int32_t num_col_blocks, int32_t page_size, int32_t* kv_indptr_h,
                                int32_t* kv_indices_h, int64_t kv_indices_cap,
                                int32_t* last_page_len_h, int32_t* kv_lens_h, int64_t* num_pages);

/* Summary of the current plan. */
fa_status fa_plan_info(const fa_plan_t* plan, fa_plan_stats* stats);

/* Host copies of the current plan ([Guide] "What FlashInfer is", idea 3: the
 * load-balanced tile assignment that the plan phase computes; exposed so a
 * caller can inspect the balance), valid until the next fa_plan on this plan.
 * tiles int32 [num_tiles][8]:
 *   decode  {request, kv_head, kv_indptr[request], first_slot, key_begin, key_end, slot,
 *           n_pieces};
 *   append  {request, kv_head, row_begin, row_end, key_begin, key_end, slot0, n_chunks}.
 * Decode: worker wave w runs tiles worker_ptr[w] .. worker_ptr[w+1]-1 in
 * order (worker_ptr int32 [num_workers+1]; *num_workers receives num_cu *
 * tiles_per_cu). Append: tiles are listed in 8 bins, one per XCD: bin x is
 * tiles worker_ptr[x] .. worker_ptr[x+1]-1 (worker_ptr int32 [9];
 * *num_workers receives 8), and workgroup i runs bin i mod 8.
 * A slot of -1 means the tile writes the final output. merge int32
 * [num_merge][4] = {first row, kv_head, first_slot, n_states} per split unit.
 * Any output pointer may be NULL. */
fa_status fa_plan_tiles(const fa_plan_t* plan, const int32_t** tiles_h, int32_t* num_tiles,
                        const int32_t** merge_h, int32_t* num_merge,
                        const int32_t** worker_ptr_h, int32_t* num_workers);

/* Release the HIP events a plan keeps (cascade fork/join, pageable host
 * workspaces). If the plan's last copy out of a pinned host workspace is
 * still pending, waits until the copy kernel has read the image and written
 * its completion words, so the host workspace can be freed afterwards (the
 * device workspace, as always, only once the work queued on it is done). */
fa_status fa_plan_destroy(fa_plan_t* plan);

/* Batched decode over the paged KV cache ([DeepDive] "Snippet One", batch
 * decode wrapper plan/run; [Guide] "Quickstart").
 *
 *  q            device [batch, num_qo_heads, head_dim], geometry dtype, contiguous.
 *  k_pages, v_pages  device page pools; element (page, slot, kv_head, d) of K is
 *               k_pages[page*page_stride + slot*token_stride + kv_head*head_stride + d]
 *               (strides in elements, d contiguous). The combined pool
 *               [num_pages, 2, page_size, num_kv_heads, head_dim] is
 *               k_pages = pool, v_pages = pool + page_size*num_kv_heads*head_dim,
 *               page_stride = 2*page_size*num_kv_heads*head_dim,
 *               token_stride = num_kv_heads*head_dim, head_stride = head_dim.
 *               Pointers 16-byte aligned, strides multiples of 8.
 *  kv_indices_d, kv_indptr_d, last_page_len_d  device int32 CSR page table
 *               (same content as given to fa_plan; last_page_len in [1, page_size]).
 *  out          device [batch, num_qo_heads, head_dim], geometry dtype.
 *  lse          device fp32 [batch, num_qo_heads] or NULL.
 * A request with no keys gets out = 0 and lse = -inf. Requests whose keys were
 * split by the plan are combined with the log-sum-exp merge inside the same
 * kernel (the last piece to finish merges). One kernel launch on `stream`.
 * Errors: FA_ERR_INVALID, FA_ERR_NOT_PLANNED, FA_ERR_HIP. */
fa_status fa_decode(const fa_plan_t* plan, const void* q, const void* k_pages,
                    const void* v_pages, int64_t page_stride, int64_t token_stride,
                    int64_t head_stride, const int32_t* kv_indices_d, const int32_t* kv_indptr_d,
                    const int32_t* last_page_len_d, float sm_scale, void* out, float* lse,
                    void* stream);

/* For callers that cannot allocate (serving loops or harnesses that forbid
 * device allocation): fa_plan + fa_decode in one call, with no caller-owned
 * workspace and no allocation of any kind. The plan image, the arrival
 * counters and the fp32 partial states live in a file-scope device array of
 * 16 MiB per GPU and the host plan workspace in a static host array of 1 MiB
 * per GPU, both held until the process ends.
 *  geom, kv_indptr_h, kv_lens_h, batch  as in fa_plan (decode geometry only).
 *  q, pages, strides, page tables, sm_scale, out, lse  as in fa_decode.
 * The call plans on the host, copies the plan into the GPU's array on
 * `stream` and waits on `stream` until that copy is done (work queued earlier
 * on the stream included), then queues the decode kernel. It cannot be
 * captured into a graph. Calls on one GPU share its arrays: calls that overlap
 * (other streams or host threads on the same GPU) race. The results are those
 * of fa_plan + fa_decode with the same geometry, bit for bit. Errors: those
 * of fa_plan and fa_decode; FA_ERR_CAPACITY (nothing queued) when the
 * geometry's workspaces (fa_workspace_size) exceed the static arrays. */
fa_status fa_decode_noalloc(const fa_geometry* geom, const int32_t* kv_indptr_h,
                            const int32_t* kv_lens_h, int32_t batch, const void* q,
                            const void* k_pages, const void* v_pages, int64_t page_stride,
                            int64_t token_stride, int64_t head_stride,
                            const int32_t* kv_indices_d, const int32_t* kv_indptr_d,
                            const int32_t* last_page_len_d, float sm_scale, void* out, float* lse,
                            void* stream);

/* Decode over a paged KV cache whose stored values carry one scale per tensor
 * ([Tool] "FlashInfer", "What it does": FP8 compute for attention; [Guide]
 * "Features (from the repository README)": FP8 with per-tensor scaling).
 * The stored element e of K stands for k_scale * e, of V for v_scale * e:
 * s_j = sm_scale * k_scale * <q, k_j> and out = v_scale * sum_j p_j v_j, with
 * lse over those s_j. The pages' element type is the plan's kv_dtype: with
 * FA_E4M3 every page element is one byte, so page_stride, token_stride and
 * head_stride count bytes and must be multiples of 16; with 16-bit pages the
 * call is fa_decode with the two scales. K/V codes are widened exactly and
 * the products accumulate in fp32, as in fa_decode.
 *  k_scale, v_scale  finite and > 0.
 * Other arguments as fa_decode. Errors: FA_ERR_INVALID (also for a bad
 * scale), FA_ERR_NOT_PLANNED, FA_ERR_HIP. fa_decode on an FA_E4M3 plan is
 * this call with both scales 1. */
fa_status fa_decode_scaled(const fa_plan_t* plan, const void* q, const void* k_pages,
                           const void* v_pages, int64_t page_stride, int64_t token_stride,
                           int64_t head_stride, const int32_t* kv_indices_d,
                           const int32_t* kv_indptr_d, const int32_t* last_page_len_d,
                           float sm_scale, float k_scale, float v_scale, void* out, float* lse,
                           void* stream);

/* Decode over a ragged KV cache planned by fa_plan_ragged.
 *  k, v          device [total_rows, num_kv_heads, head_dim] (element (row, h, d) at
 *                row*token_stride + h*head_stride + d; 16-byte aligned; strides as in
 *                fa_decode, in bytes for an FA_E4M3 plan).
 *  kv_offsets_d  device int32 [batch+1], the same content as given to fa_plan_ragged,
 *                or NULL to use the copy in the plan's workspace.
 *  k_scale, v_scale  as in fa_decode_scaled (1 for unscaled 16-bit K / V).
 * Other arguments, results and errors as fa_decode_scaled. */
fa_status fa_decode_ragged(const fa_plan_t* plan, const void* q, const void* k, const void* v,
                           int64_t token_stride, int64_t head_stride, const int32_t* kv_offsets_d,
                           float sm_scale, float k_scale, float v_scale, void* out, float* lse,
                           void* stream);

/* Append / prefill over a ragged KV cache planned by fa_plan_ragged with
 * qo_indptr (the new rows' K / V are the last qo_len rows of each request).
 * k, v, strides and kv_offsets_d as in fa_decode_ragged; other arguments,
 * results and errors as fa_append. */
fa_status fa_append_ragged(const fa_plan_t* plan, const void* q, const int32_t* qo_indptr_d,
                           const void* k, const void* v, int64_t token_stride,
                           int64_t head_stride, const int32_t* kv_offsets_d, float sm_scale,
                           void* out, float* lse, void* stream);

/* Append / prefill over the paged KV cache, causal or not as planned ([Guide]
 * "Features (from the repository README)": prefill and append kernels). The
 * new tokens' K/V must already be in the pages.
 *
 *  q            device [num_rows, num_qo_heads, head_dim] packed rows
 *               (request b owns rows qo_indptr[b] .. qo_indptr[b+1]-1).
 *  qo_indptr_d  device int32 [batch+1], same content as given to fa_plan.
 *  out / lse    device [num_rows, num_qo_heads, head_dim] / fp32 [num_rows, num_qo_heads].
 * Other arguments as fa_decode. Errors as fa_decode. */
fa_status fa_append(const fa_plan_t* plan, const void* q, const int32_t* qo_indptr_d,
                    const void* k_pages, const void* v_pages, int64_t page_stride,
                    int64_t token_stride, int64_t head_stride, const int32_t* kv_indices_d,
                    const int32_t* kv_indptr_d, const int32_t* last_page_len_d, float sm_scale,
                    void* out, float* lse, void* stream);

/* A mixed batch in one launch ([Windows] "Core Features", Attention Kernels:
 * POD-attention, prefill and decode fused for mixed batching): the append /
 * prefill requests of prefill_plan and the decode requests of decode_plan, over
 * the same page pools, in one kernel. The prefill plan's q tile picks its
 * shape: tiles of at most 128 / G query positions run beside the decode
 * workgroups in the same compute units; wider
 * tiles, up to the append kernel's 256 / G (the default qo_tile of an append
 * geometry), run the append kernel's workgroups, and each compute unit runs
 * decode or append work at a time. The results are those of fa_append (q_p,
 * qo_indptr_p_d, kv_*_p_d, out_p, lse_p) and fa_decode (q_d, kv_*_d, out_d,
 * lse_d), bit for bit. Both plans need the same dtype and heads and 16-bit
 * K/V pages; with num_qo_heads / num_kv_heads = 8 only the wider tiles are
 * built (qo_tile 17..32). Pools and strides as in fa_decode. Errors as
 * fa_decode. */
fa_status fa_pod(const fa_plan_t* prefill_plan, const void* q_p, const int32_t* qo_indptr_p_d,
                 const int32_t* kv_indices_p_d, const int32_t* kv_indptr_p_d,
                 const int32_t* last_page_len_p_d, void* out_p, float* lse_p,
                 const fa_plan_t* decode_plan, const void* q_d, const int32_t* kv_indices_d,
                 const int32_t* kv_indptr_d, const int32_t* last_page_len_d, void* out_d,
                 float* lse_d, const void* k_pages, const void* v_pages, int64_t page_stride,
                 int64_t token_stride, int64_t head_stride, float sm_scale, void* stream);

/* Cascade attention over one shared prefix ([Guide] "Cascade attention for
 * shared prefixes"; [DeepDive] "Why This Design Works": the shared prefix is
 * stored once and read once): for every request b,
 *   out[b] = merge_state(attention(q[b], prefix), attention(q[b], suffix of b)).
 *  prefix_plan  an append plan of ONE request whose rows are the batch's
 *               queries (qo_indptr {0, batch}), non-causal, over the prefix pages.
 *  suffix_plan  a decode plan over the per-request suffix pages.
 *  prefix_qo_indptr_d  device int32 {0, batch}.
 *  prefix_indices_d / prefix_indptr_d / prefix_last_page_len_d  the prefix's
 *               page table (one request); kv_* the suffix page tables.
 *  prefix_out, suffix_out  device [batch, num_qo_heads, head_dim] scratch in
 *               the q dtype; prefix_lse, suffix_lse device fp32 [batch, num_qo_heads].
 *               (prefix_out / prefix_lse are only written when the prefix plan
 *               does not split its keys; split prefix chunks stay as fp32
 *               partial states in the prefix plan's workspace.)
 *  out / lse    device [batch, num_qo_heads, head_dim] / fp32 (lse may be NULL).
 * With both extra streams NULL (or equal to `stream`), one kernel on `stream`
 * runs both passes side by side (fa_pod's two shapes, picked by the prefix
 * plan's q tile: up to 128 / G positions, G <= 4, the prefix workgroups
 * share each compute unit with a decode workgroup; up to 256 / G, the append
 * geometry's default, the decode takes half the compute units and the prefix
 * tiles the other half at full rate, then all of them). Otherwise the
 * suffix decode runs on `suffix_stream` and the prefix pass on
 * `prefix_stream` (each NULL or equal to `stream` = run on `stream`); streams
 * other than `stream` are forked from it and joined back with events of the
 * suffix plan (capturable). Then one combine kernel on `stream` merges, per
 * (request, head), the prefix chunks and the suffix state by log-sum-exp.
 * In the wide shape a decode plan of 4 worker waves per compute unit holds
 * half of them, so a prefix plan of one round of tiles for the other half
 * (num_cu 128, tiles_per_cu 1 on 256 compute units) fits it best.
 * (Measured on MI355X at batch 256 / 16k prefix, G = 4, with 1 GiB of pool
 * copies rotated, per call in one run: 179-184 us with that prefix plan,
 * 196-200 us with two rounds of 256 / G tiles, 204 us with 128 / G tiles
 * sharing the compute units; the passes on separate streams, sharing or
 * splitting the compute units, were slower than in order.) Other
 * arguments as fa_decode. Errors: FA_ERR_INVALID, FA_ERR_NOT_PLANNED,
 * FA_ERR_HIP. */
fa_status fa_cascade(const fa_plan_t* prefix_plan, const fa_plan_t* suffix_plan, const void* q,
                     const void* k_pages, const void* v_pages, int64_t page_stride,
                     int64_t token_stride, int64_t head_stride, const int32_t* prefix_qo_indptr_d,
                     const int32_t* prefix_indices_d, const int32_t* prefix_indptr_d,
                     const int32_t* prefix_last_page_len_d, const int32_t* kv_indices_d,
                     const int32_t* kv_indptr_d, const int32_t* last_page_len_d, float sm_scale,
                     void* prefix_out, float* prefix_lse, void* suffix_out, float* suffix_lse,
                     void* out, float* lse, void* stream, void* prefix_stream,
                     void* suffix_stream);

/* Merge two attention states computed over disjoint key sets ([Guide]
 * "Cascade attention for shared prefixes"):
 *   s = log(exp(s_a) + exp(s_b)),  v = exp(s_a - s) v_a + exp(s_b - s) v_b.
 *  v_a, v_b, v_out  device [n, heads, head_dim] in `dtype` (FA_F16, FA_BF16, FA_F32).
 *  s_a, s_b, s_out  device fp32 [n, heads]; -inf marks an empty state.
 * v_out / s_out may alias v_a / s_a. head_dim must be a multiple of 8 and the
 * pointers 16-byte aligned. Errors: FA_ERR_INVALID, FA_ERR_HIP. */
fa_status fa_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                         void* v_out, float* s_out, int64_t n, int32_t heads, int32_t head_dim,
                         int32_t dtype, void* stream);

/* Merge k states per row ([Guide] "Cascade attention for shared prefixes"):
 *  v  device [n, k, heads, head_dim] in `dtype`; s device fp32 [n, k, heads];
 *  v_out device [n, heads, head_dim] in `dtype`; s_out fp32 [n, heads] or NULL.
 * All states -inf gives v = 0, s = -inf. Errors: FA_ERR_INVALID, FA_ERR_HIP. */
fa_status fa_merge_states(const void* v, const float* s, int64_t n, int32_t k, int32_t heads,
                          int32_t head_dim, int32_t dtype, void* v_out, float* s_out,
                          void* stream);

/* Measurement utility, not a step of the attention path: reads `bytes` of
 * device memory at `src` once with 16-byte non-temporal loads from
 * `workgroups` workgroups of 256 threads (each a contiguous share), the plain
 * streaming read that the
 * decode's HBM bandwidth is compared with. The loads are folded by XOR;
 * `flag` (device, 4 bytes) is written only in the unlikely case that the fold
 * equals a fixed key, so the probe adds no write traffic. `bytes` must be a
 * positive multiple of 16 and `src` 16-byte aligned (the caller owns both
 * buffers). Launch is asynchronous on `stream`. Errors: FA_ERR_INVALID,
 * FA_ERR_HIP. */
fa_status fa_probe_stream_read(const void* src, int64_t bytes, uint32_t* flag, int32_t workgroups,
                               void* stream);

/* Static description of a status code. Error reporting of this interface
 * itself: the pages define no error codes (their Python calls raise), so
 * every entry point returns one of the FA_ codes above and these two calls
 * turn it into text. */
const char* fa_status_string(fa_status status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_FA_H_ */
