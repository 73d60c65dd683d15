// Split-KV work planner: host-only, integer-only.
//
// [Guide] "FlashInfer: GPU Kernels for LLM Inference (2026 Guide)", section
// "What FlashInfer is" (idea 3: plan the split of uneven requests so the load
// is even while the launch stays static for graphs) and [DeepDive] "FlashInfer:
// The Attention Kernel Library That Proves the Bottleneck ...", sections "It In
// Action" step 1 (a per-step plan computes only tile assignments) and "Why This
// Design Works" (static launch, dynamic assignment). The pages give no
// algorithm; this planner fixes one per mode. A *unit* is one kv head of one
// q tile (a request in decode, up to qo_tile query rows in append).
//
// Decode (HBM-bound, one wave per worker): requests are cut into pieces of
// about the mean load of a wave (at most 128 pages: a wave keeps the ids of
// one piece in two registers) and the pieces are dealt largest first to
// static work lists, one per worker wave, the kv heads of a piece to
// neighbouring waves. A unit cut into C > 1 pieces gets C fp32 partial
// states, combined by log-sum-exp by the last piece to finish.
//
// Append (MFMA-bound, one workgroup per tile): every q tile is cut into
// chunks of P = max(min_chunk_pages, ceil(units / target)) pages, so tiles
// cost about the same. The (request, kv head) groups are dealt, largest
// first, to 8 bins of least cost, one per XCD, so the q tiles that read the
// same keys run on one XCD and share its L2; within a bin a group's tiles are
// listed in descending cost, and workgroup i runs tiles of bin i mod 8.
//
// Launch shapes depend only on capacities derived from the geometry, never on
// the lengths, which keeps a captured graph valid across plans.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "plan_internal.h"

namespace pkfa {

namespace {
thread_local char g_err[512] = "";

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

const char* last_error() { return g_err; }

fa_status resolve_geometry(const fa_geometry* in, fa_geometry* out) {
  if (!in || !out) {
    set_error("geometry is NULL");
    return FA_ERR_INVALID;
  }
  fa_geometry g = *in;
  if (g.mode != FA_MODE_DECODE && g.mode != FA_MODE_APPEND) {
    set_error("unknown mode %d", g.mode);
    return FA_ERR_INVALID;
  }
  if (g.max_batch <= 0 || g.num_qo_heads <= 0 || g.num_kv_heads <= 0 ||
      g.num_qo_heads % g.num_kv_heads != 0) {
    set_error("need max_batch > 0 and num_qo_heads a positive multiple of num_kv_heads");
    return FA_ERR_INVALID;
  }
  if (g.mode == FA_MODE_APPEND && g.max_qo_tokens <= 0) {
    set_error("append geometry needs max_qo_tokens > 0");
    return FA_ERR_INVALID;
  }
  if (g.num_cu < 0 || g.tiles_per_cu < 0 || g.min_chunk_pages < 0 || g.qo_tile < 0 ||
      g.max_tiles < 0 || g.max_partials < 0 || g.max_merge < 0 || g.pieces_per_worker < 0) {
    set_error("negative plan knob");
    return FA_ERR_INVALID;
  }
  const int G = g.num_qo_heads / g.num_kv_heads;
  if (g.head_dim != kSupportedHeadDim || g.page_size != kSupportedPageSize ||
      !(G == 1 || G == 2 || G == 4 || G == 8) || (g.dtype != FA_F16 && g.dtype != FA_BF16)) {
    set_error("unsupported: head_dim %d page_size %d group %d dtype %d (built: 128, 16, "
              "{1,2,4,8}, fp16/bf16)", g.head_dim, g.page_size, G, g.dtype);
    return FA_ERR_UNSUPPORTED;
  }
  const bool app = g.mode == FA_MODE_APPEND;
  if (g.kv_dtype == 0) g.kv_dtype = g.dtype;
  if (g.kv_dtype != g.dtype && !(g.kv_dtype == FA_E4M3 && !app)) {
    set_error("unsupported: kv_dtype %d with dtype %d in %s (built: the q dtype, or E4M3 for "
              "decode)", g.kv_dtype, g.dtype, app ? "append" : "decode");
    return FA_ERR_UNSUPPORTED;
  }
  if (!app) g.max_qo_tokens = 0;
  if (!g.num_cu) g.num_cu = 256;
  if (!g.tiles_per_cu) g.tiles_per_cu = app ? 2 : 4;
  if (!g.min_chunk_pages) g.min_chunk_pages = 1;
  g.pieces_per_worker = app ? 0 : (g.pieces_per_worker ? g.pieces_per_worker : kPiecesPerWorker);
  // an append tile holds kAppendCols query columns: the G heads x kAppendCols / G positions
  g.qo_tile = app ? (g.qo_tile ? g.qo_tile : kAppendCols / G) : 1;
  if (app && g.qo_tile > kAppendCols / G) {
    set_error("qo_tile %d exceeds the %d query positions of an append tile for group %d",
              g.qo_tile, kAppendCols / G, G);
    return FA_ERR_UNSUPPORTED;
  }
  const int64_t target = (int64_t)g.num_cu * g.tiles_per_cu;
  int64_t mt, mp, mm;
  if (app) {
    const int64_t nqt = (int64_t)g.max_batch + cdiv(g.max_qo_tokens, g.qo_tile);
    mt = g.max_tiles ? g.max_tiles : target + (int64_t)g.num_kv_heads * nqt;
    mp = g.max_partials ? g.max_partials : 2 * (int64_t)g.qo_tile * target;
    mm = g.max_merge ? g.max_merge : target;
  } else {
    const int64_t units = (int64_t)g.max_batch * g.num_kv_heads;
    mt = g.max_tiles ? g.max_tiles : (int64_t)g.pieces_per_worker * target + units;
    mp = g.max_partials ? g.max_partials : (int64_t)g.pieces_per_worker * target + units;
    mm = g.max_merge ? g.max_merge : units;
  }
  if (target * std::max(1, g.pieces_per_worker) > (1 << 22)) {
    set_error("num_cu * tiles_per_cu (* pieces_per_worker) too large");
    return FA_ERR_INVALID;
  }
  if (mt > (1 << 26) || mp > (1 << 26) || mm > (1 << 26)) {
    set_error("capacities too large");
    return FA_ERR_INVALID;
  }
  g.max_tiles = (int32_t)mt;
  g.max_partials = (int32_t)mp;
  g.max_merge = (int32_t)mm;
  *out = g;
  return FA_OK;
}

Layout compute_layout(const fa_geometry& g) {
  Layout L;
  const int G = g.num_qo_heads / g.num_kv_heads;
  L.workers = g.mode == FA_MODE_DECODE ? g.num_cu * g.tiles_per_cu : 0;
  L.header = 0;
  L.merge = kHeaderInts * 4;
  L.worker_ptr = L.merge + (size_t)g.max_merge * kMergeInts * 4;
  L.offsets = L.worker_ptr + (size_t)(std::max<int32_t>(L.workers, kXcdBins) + 1) * 4;
  L.tiles = align_up(L.offsets + ((size_t)g.max_batch + 1) * 4, 64);
  L.upload_end = L.tiles + (size_t)g.max_tiles * kTileInts * 4;
  L.dev_counters = align_up(L.upload_end, 256);
  L.dev_part_lse = align_up(L.dev_counters + (size_t)g.max_partials * 4, 256);
  L.dev_part_o = align_up(L.dev_part_lse + (size_t)g.max_partials * G * 4, 256);
  L.dev_bytes = align_up(L.dev_part_o + (size_t)g.max_partials * G * g.head_dim * 4, 256);
  L.host_unsorted = align_up(L.upload_end, 64);
  L.host_order = L.host_unsorted + (size_t)g.max_tiles * kTileInts * 4;
  // tile order (append) / first piece of each decode segment (at most workers + 1)
  // decode bins: at most workers * pieces_per_worker
  const int64_t bins = (int64_t)L.workers * std::max(1, g.pieces_per_worker) + 2;
  const size_t nlist = (size_t)std::max<int64_t>(g.max_tiles, bins);
  L.host_cost = align_up(L.host_order + nlist * 4, 8);
  L.host_bin = L.host_cost + nlist * 8;
  L.host_seg = align_up(L.host_bin + nlist * 4, 8);
  L.host_units = align_up(L.host_seg + (size_t)bins * 4, 8);
  // per (request, kv head): 2 int32 (decode) or int64 cost + 3 int32 (append)
  L.host_lens = L.host_units + (size_t)g.max_batch * g.num_kv_heads * 24;
  L.host_flags = align_up(L.host_lens + ((size_t)g.max_batch + 1) * 4, 256);
  L.host_bytes = L.host_flags + (size_t)kUploadMaxGrid * 4;
  return L;
}

namespace {

fa_status capacity_error(const char* what, int64_t n, int32_t cap) {
  set_error("%lld %s exceed the capacity %d", (long long)n, what, cap);
  return FA_ERR_CAPACITY;
}

// Decode: NS = S * pieces_per_worker / Hkv bins; bin s and kv head h form the
// work list of wave s * Hkv + h (lists beyond S wrap round), so the Hkv waves
// of a bin read the same pages at the same time. Each request is cut into
// pieces of Q pages (the last one shorter; a request with no pages is one
// empty piece), with Q the bins' mean cost, and a piece costs its pages plus
// c0 pages' worth of set-up and epilogue. Pieces are dealt largest first
// (stable), each to the bin of least cost (lowest index on ties), and keep
// the dealing order inside their bin. Tiles are stored wave-major:
// worker_ptr[w] .. worker_ptr[w+1]-1 are wave w's.
fa_status plan_decode(const fa_geometry& g, const Layout& lay, uint8_t* ws, const int32_t* kv_indptr,
                      const int32_t* kv_lens, int32_t batch, int64_t* ntiles_out,
                      int64_t* nmerge_out, int64_t* slots_out, int64_t* piece_pages_out) {
  const int ps = g.page_size, Hkv = g.num_kv_heads;
  const int64_t S = lay.workers;
  int32_t* merge = reinterpret_cast<int32_t*>(ws + lay.merge);
  int32_t* wptr = reinterpret_cast<int32_t*>(ws + lay.worker_ptr);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + lay.tiles);
  int32_t* items = reinterpret_cast<int32_t*>(ws + lay.host_unsorted);  // [np][4] b, p0, p1, i
  int32_t* order = reinterpret_cast<int32_t*>(ws + lay.host_order);     // dealing order
  int64_t* heap = reinterpret_cast<int64_t*>(ws + lay.host_cost);       // [NS] cost << 23 | bin
  int32_t* bin_of = reinterpret_cast<int32_t*>(ws + lay.host_bin);      // bin of the n-th dealt
  int32_t* first = reinterpret_cast<int32_t*>(ws + lay.host_seg);       // [NS+1]
  int32_t* npc = reinterpret_cast<int32_t*>(ws + lay.host_units);       // [batch] pieces
  int32_t* base = npc + batch;                                           // [batch] first slot
  const int64_t NS = std::max<int64_t>(1, S * g.pieces_per_worker / Hkv);
  const int64_t c0 = g.kv_dtype == FA_E4M3 ? kPieceCostPagesE4M3 : kPieceCostPages16;
  int64_t N = 0;
  for (int b = 0; b < batch; ++b) N += cdiv(kv_lens[b], ps);
  const int64_t Q = std::min<int64_t>(
      kMaxPiecePages,
      std::max<int64_t>({1, (int64_t)g.min_chunk_pages, cdiv(N + c0 * batch, NS)}));
  // pieces in request order
  int64_t np = 0;
  for (int b = 0; b < batch; ++b) np += std::max<int64_t>(1, cdiv(cdiv(kv_lens[b], ps), Q));
  if (np * Hkv > g.max_tiles) return capacity_error("tiles", np * Hkv, g.max_tiles);
  int64_t cnt[kMaxPiecePages + 2] = {};
  for (int b = 0, k = 0; b < batch; ++b) {
    const int64_t n = cdiv(kv_lens[b], ps);
    npc[b] = (int32_t)std::max<int64_t>(1, cdiv(n, Q));
    for (int32_t i = 0; i < npc[b]; ++i, ++k) {
      int32_t* r = items + (int64_t)k * 4;
      r[0] = b;
      r[1] = (int32_t)(i * Q);
      r[2] = (int32_t)std::min<int64_t>((i + 1) * Q, n);
      r[3] = i;
      ++cnt[r[2] - r[1]];
    }
  }
  // dealing order: descending pages, stable (counting sort)
  int64_t start[kMaxPiecePages + 2];
  for (int64_t pg = Q, acc = 0; pg >= 0; --pg) {
    start[pg] = acc;
    acc += cnt[pg];
  }
  for (int64_t k = 0; k < np; ++k) {
    const int32_t* r = items + k * 4;
    order[start[r[2] - r[1]]++] = (int32_t)k;
  }
  // deal: a binary min-heap of (cost, bin) keys; ascending keys form a heap
  constexpr int kBinBits = 23;
  for (int64_t x = 0; x < NS; ++x) heap[x] = x;
  for (int64_t n = 0; n < np; ++n) {
    const int32_t* r = items + (int64_t)order[n] * 4;
    const int64_t top = heap[0];
    bin_of[n] = (int32_t)(top & ((1 << kBinBits) - 1));
    const int64_t key = top + ((int64_t)(r[2] - r[1] + c0) << kBinBits);
    // sift the raised key down from the root
    int64_t i = 0;
    for (;;) {
      const int64_t c = 2 * i + 1;
      if (c >= NS) break;
      const int64_t m = (c + 1 < NS && heap[c + 1] < heap[c]) ? c + 1 : c;
      if (heap[m] >= key) break;
      heap[i] = heap[m];
      i = m;
    }
    heap[i] = key;
  }
  // bins' pieces in dealing order
  for (int64_t x = 0; x <= NS; ++x) first[x] = 0;
  for (int64_t n = 0; n < np; ++n) ++first[bin_of[n] + 1];
  for (int64_t x = 0; x < NS; ++x) first[x + 1] += first[x];
  int32_t* binned = items + np * 4;  // [np] item per bin position
  for (int64_t n = 0; n < np; ++n) binned[first[bin_of[n]]++] = order[n];
  for (int64_t x = NS; x > 0; --x) first[x] = first[x - 1];
  first[0] = 0;
  // slots: unit (b, h) of a request cut into C > 1 pieces owns base[b] + h*C .. + C-1
  int64_t nmerge = 0, slots = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t C = npc[b];
    base[b] = -1;
    if (C <= 1) continue;
    base[b] = (int32_t)slots;
    for (int h = 0; h < Hkv; ++h, ++nmerge) {
      if (nmerge >= g.max_merge) continue;
      int32_t* m = merge + nmerge * kMergeInts;
      m[0] = b;
      m[1] = h;
      m[2] = (int32_t)(slots + (int64_t)h * C);
      m[3] = C;
    }
    slots += (int64_t)C * Hkv;
  }
  const int64_t ntiles = np * Hkv;
  if (slots > g.max_partials) return capacity_error("partial states", slots, g.max_partials);
  if (nmerge > g.max_merge) return capacity_error("merge entries", nmerge, g.max_merge);
  // wave-major tiles: list j = bin * Hkv + head runs on wave j % S
  int64_t k = 0;
  for (int64_t w = 0; w < S; ++w) {
    wptr[w] = (int32_t)k;
    for (int64_t j = w; j < NS * Hkv; j += S) {
      const int64_t sgm = j / Hkv;
      const int h = (int)(j % Hkv);
      for (int64_t q = first[sgm]; q < first[sgm + 1]; ++q, ++k) {
        const int32_t* r = items + (int64_t)binned[q] * 4;
        const int b = r[0];
        const int32_t C = npc[b];
        const int32_t ub = base[b] >= 0 ? base[b] + h * C : -1;
        int32_t* t = tiles + k * kTileInts;
        t[0] = b;
        t[1] = h;
        t[2] = kv_indptr[b];
        t[3] = ub;
        t[4] = r[1] * ps;
        t[5] = (int32_t)std::min<int64_t>((int64_t)r[2] * ps, kv_lens[b]);
        t[6] = ub >= 0 ? ub + r[3] : -1;
        t[7] = C;
      }
    }
  }
  wptr[S] = (int32_t)k;
  *ntiles_out = ntiles;
  *nmerge_out = nmerge;
  *slots_out = slots;
  *piece_pages_out = Q;
  return FA_OK;
}

// Append: uniform chunks of P pages; groups dealt to XCD bins, LPT inside.
fa_status plan_append(const fa_geometry& g, const Layout& lay, uint8_t* ws, const int32_t* kv_lens,
                      int32_t batch, const int32_t* qo_indptr, int32_t causal, int64_t* ntiles_out,
                      int64_t* nmerge_out, int64_t* slots_out, int64_t* P_out) {
  const int ps = g.page_size, Hkv = g.num_kv_heads, qt = g.qo_tile;
  int32_t* merge = reinterpret_cast<int32_t*>(ws + lay.merge);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + lay.tiles);
  int32_t* unsorted = reinterpret_cast<int32_t*>(ws + lay.host_unsorted);
  int32_t* order = reinterpret_cast<int32_t*>(ws + lay.host_order);
  int64_t* cost = reinterpret_cast<int64_t*>(ws + lay.host_cost);
  // Visit q tiles in (request, tile) order; fn(b, row0, row1, visible_keys).
  auto for_each_qtile = [&](auto&& fn) {
    for (int b = 0; b < batch; ++b) {
      const int64_t L = kv_lens[b];
      const int64_t r0 = qo_indptr[b], r1 = qo_indptr[b + 1], ql = r1 - r0;
      for (int64_t t0 = 0; t0 < ql; t0 += qt) {
        const int64_t t1 = std::min(ql, t0 + qt);
        const int64_t vis = causal ? std::min(L, L - ql + t1) : L;
        fn(b, r0 + t0, r0 + t1, vis);
      }
    }
  };
  int64_t units = 0;
  for_each_qtile([&](int, int64_t, int64_t, int64_t vis) { units += cdiv(vis, ps); });
  units *= Hkv;
  const int64_t target = (int64_t)g.num_cu * g.tiles_per_cu;
  const int64_t P = std::max<int64_t>(g.min_chunk_pages, cdiv(units, target));
  int64_t ntiles = 0, nmerge = 0, slots = 0;
  for_each_qtile([&](int b, int64_t q0, int64_t q1, int64_t vis) {
    const int64_t C = std::max<int64_t>(1, cdiv(cdiv(vis, ps), P));
    const int64_t rows = q1 - q0;
    for (int h = 0; h < Hkv; ++h) {
      int64_t base = -1;
      if (C > 1) {
        base = slots;
        slots += C * rows;
        if (nmerge < g.max_merge) {
          int32_t* m = merge + nmerge * kMergeInts;
          m[0] = (int32_t)q0;
          m[1] = h;
          m[2] = (int32_t)base;
          m[3] = (int32_t)C;
        }
        ++nmerge;
      }
      for (int64_t c = 0; c < C; ++c) {
        if (ntiles < g.max_tiles) {
          const int64_t k0 = c * P * ps, k1 = std::min((c + 1) * P * ps, vis);
          int32_t* t = unsorted + ntiles * kTileInts;
          t[0] = b;
          t[1] = h;
          t[2] = (int32_t)q0;
          t[3] = (int32_t)q1;
          t[4] = (int32_t)k0;
          t[5] = (int32_t)k1;
          t[6] = C > 1 ? (int32_t)(base + c * rows) : -1;
          t[7] = (int32_t)C;
          cost[ntiles] = (k1 - k0) * rows;
        }
        ++ntiles;
      }
    }
  });
  if (ntiles > g.max_tiles) return capacity_error("tiles", ntiles, g.max_tiles);
  if (slots > g.max_partials) return capacity_error("partial states", slots, g.max_partials);
  if (nmerge > g.max_merge) return capacity_error("merge entries", nmerge, g.max_merge);
  // XCD bins: deal the (request, kv head) groups, largest first, to the bin
  // with the least cost; order tiles by (bin, group dealing order, cost desc).
  const int64_t ngroups = (int64_t)batch * Hkv;
  int64_t* gcost = reinterpret_cast<int64_t*>(ws + lay.host_units);
  int32_t* gorder = reinterpret_cast<int32_t*>(gcost + ngroups);
  int32_t* gbin = gorder + ngroups;
  int32_t* gseq = gbin + ngroups;
  for (int64_t i = 0; i < ngroups; ++i) {
    gcost[i] = 0;
    gorder[i] = (int32_t)i;
  }
  auto group_of = [&](int64_t t) {
    return (int64_t)unsorted[t * kTileInts] * Hkv + unsorted[t * kTileInts + 1];
  };
  for (int64_t t = 0; t < ntiles; ++t) gcost[group_of(t)] += cost[t];
  std::stable_sort(gorder, gorder + ngroups, [&](int32_t a, int32_t b) { return gcost[a] > gcost[b]; });
  int64_t bcost[kXcdBins] = {};
  for (int64_t n = 0; n < ngroups; ++n) {
    int x = 0;
    for (int j = 1; j < kXcdBins; ++j)
      if (bcost[j] < bcost[x]) x = j;
    gbin[gorder[n]] = x;
    gseq[gorder[n]] = (int32_t)n;
    bcost[x] += gcost[gorder[n]];
  }
  for (int64_t i = 0; i < ntiles; ++i) order[i] = (int32_t)i;
  std::stable_sort(order, order + ntiles, [&](int32_t a, int32_t b) {
    const int64_t ga = group_of(a), gb = group_of(b);
    if (gbin[ga] != gbin[gb]) return gbin[ga] < gbin[gb];
    if (gseq[ga] != gseq[gb]) return gseq[ga] < gseq[gb];
    return cost[a] > cost[b];
  });
  int32_t* wptr = reinterpret_cast<int32_t*>(ws + lay.worker_ptr);
  for (int x = 0; x <= kXcdBins; ++x) wptr[x] = 0;
  for (int64_t i = 0; i < ntiles; ++i) {
    memcpy(tiles + i * kTileInts, unsorted + (int64_t)order[i] * kTileInts, kTileInts * 4);
    ++wptr[gbin[group_of(order[i])] + 1];
  }
  for (int x = 0; x < kXcdBins; ++x) wptr[x + 1] += wptr[x];
  *ntiles_out = ntiles;
  *nmerge_out = nmerge;
  *slots_out = slots;
  *P_out = P;
  return FA_OK;
}

}  // namespace

fa_status build_plan(PlanImpl* p, const fa_geometry& g, const int32_t* kv_indptr,
                     const int32_t* kv_lens, int32_t batch, const int32_t* qo_indptr,
                     int32_t causal, void* host_ws, size_t host_ws_bytes, bool ragged) {
  const bool app = g.mode == FA_MODE_APPEND;
  const int ps = g.page_size;
  if (batch < 0 || batch > g.max_batch) {
    set_error("batch %d outside [0, %d]", batch, g.max_batch);
    return FA_ERR_INVALID;
  }
  if (batch > 0 && (!kv_indptr || !kv_lens)) {
    set_error("kv_indptr / kv_lens is NULL");
    return FA_ERR_INVALID;
  }
  if (app != (qo_indptr != nullptr)) {
    set_error(app ? "append plan needs qo_indptr" : "decode plan takes no qo_indptr");
    return FA_ERR_INVALID;
  }
  if (kv_indptr && kv_indptr[0] != 0) {
    set_error("kv_indptr[0] must be 0");
    return FA_ERR_INVALID;
  }
  for (int b = 0; b < batch; ++b) {
    const int64_t n = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
    const int64_t L = kv_lens[b];
    if (n < 0) {
      set_error("kv_indptr decreases at request %d", b);
      return FA_ERR_INVALID;
    }
    if (ragged ? n != L : (n == 0 ? L != 0 : !((n - 1) * ps < L && L <= n * ps))) {
      set_error("request %d: kv_len %lld inconsistent with %lld pages", b, (long long)L,
                (long long)n);
      return FA_ERR_INVALID;
    }
  }
  if (app) {
    if (qo_indptr[0] != 0) {
      set_error("qo_indptr[0] must be 0");
      return FA_ERR_INVALID;
    }
    for (int b = 0; b < batch; ++b) {
      const int64_t ql = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
      if (ql < 0) {
        set_error("qo_indptr decreases at request %d", b);
        return FA_ERR_INVALID;
      }
      if (causal && ql > kv_lens[b]) {
        set_error("request %d: causal qo_len %lld exceeds kv_len %d", b, (long long)ql, kv_lens[b]);
        return FA_ERR_INVALID;
      }
    }
    if (qo_indptr[batch] > g.max_qo_tokens) {
      set_error("%d query rows exceed max_qo_tokens %d", qo_indptr[batch], g.max_qo_tokens);
      return FA_ERR_INVALID;
    }
  }
  const Layout lay = compute_layout(g);
  if (!host_ws || host_ws_bytes < lay.host_bytes) {
    set_error("host workspace needs %zu bytes", lay.host_bytes);
    return FA_ERR_WORKSPACE;
  }
  uint8_t* ws = static_cast<uint8_t*>(host_ws);
  int32_t* header = reinterpret_cast<int32_t*>(ws + lay.header);
  int64_t ntiles = 0, nmerge = 0, slots = 0, P = 0;
  fa_status st = app ? plan_append(g, lay, ws, kv_lens, batch, qo_indptr, causal, &ntiles, &nmerge,
                                   &slots, &P)
                     : plan_decode(g, lay, ws, kv_indptr, kv_lens, batch, &ntiles, &nmerge, &slots,
                                   &P);
  if (st != FA_OK) return st;
  memset(header, 0, kHeaderInts * 4);
  header[0] = (int32_t)ntiles;
  header[1] = (int32_t)nmerge;
  header[2] = batch;
  header[3] = app ? qo_indptr[batch] : batch;
  header[4] = app ? causal : 0;
  header[5] = (int32_t)P;
  header[6] = lay.workers;
  header[7] = ragged ? 1 : 0;
  if (ragged) {
    int32_t* offs = reinterpret_cast<int32_t*>(ws + lay.offsets);
    for (int b = 0; b <= batch; ++b) offs[b] = kv_indptr ? kv_indptr[b] : 0;
  }

  p->num_tiles = (int32_t)ntiles;
  p->num_merge = (int32_t)nmerge;
  p->num_slots = (int32_t)slots;
  p->chunk_pages = (int32_t)P;
  p->batch = batch;
  p->num_rows = header[3];
  p->causal = header[4];
  p->num_workers = lay.workers;
  p->ragged = ragged ? 1 : 0;
  p->geom = g;
  p->lay = lay;
  p->host_ws = host_ws;
  return FA_OK;
}

}  // namespace pkfa
