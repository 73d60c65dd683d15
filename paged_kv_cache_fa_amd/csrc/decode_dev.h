// Paged-KV decode kernel for gfx950.
//
// What it computes: for each request b and query head h, scaled-dot-product
// attention of q[b, h] over the request's keys gathered through its page
// table ([DeepDive] "FlashInfer: The Attention Kernel Library That Proves the
// Bottleneck ...", section "Snippet One: Paged KV-Cache Attention and MLA":
// page pool, CSR page list, last_page_len), split into key chunks by the
// planner ([Guide] "FlashInfer: GPU Kernels for LLM Inference (2026 Guide)",
// section "What FlashInfer is", idea 3). Chunks of one request are combined by
// the log-sum-exp merge ([Guide] section "Cascade attention for shared
// prefixes").
//
// MI355X design (decode is HBM-bound):
//  * one wave64 per worker, 4 independent waves per 256-thread workgroup, no
//    barriers; the planner cuts requests into pieces and deals them, largest
//    first, to static per-wave work lists of the same cost (pages plus a
//    per-piece overhead), the kv heads of a piece to neighbouring waves, so
//    they read whole token rows of the same pages at about the same time;
//  * all G = Hq/Hkv query heads of the kv head are packed in the wave (GQA),
//    so each K/V byte is read from HBM once for all of them;
//  * lane = 8 x row-group + segment: row group r (0..7) owns tokens r and r+8
//    of every 16-token page, segment s (0..7) owns dims [8s, 8s+8) and
//    [64+8s, 64+8s+8); each K/V row (256 B) is two fully coalesced 128-byte
//    halves, 16 bytes per lane (buffer_load_dwordx4);
//  * loads go through a per-page buffer resource whose size stops at the
//    last valid token, so slots past last_page_len read as zero without any
//    memory access and without branches; K/V loads carry the non-temporal
//    cache policy (the pages are read once);
//  * a ring of NBUF pages in registers: page j+NBUF-1 is requested while page
//    j is consumed;
//  * scores: packed 2-element dot products (v_dot2_f32_bf16 / _f16) and an
//    8-lane DPP sum; P*V: the two tokens a lane holds are paired per element
//    (v_perm) and multiplied with the packed probabilities by the same dot2,
//    accumulating in fp32;
//  * E4M3 pages (one byte per element, one scale per tensor): a 128-byte K/V
//    row is one 16-byte load per lane (segment s owns dims [16s, 16s+16));
//    codes are widened exactly to the q type in registers (v_cvt_scalef32_pk
//    with scale 1) and take the same dot2 path; the K scale joins the score
//    scale and the V scale the final normalisation;
//  * for G >= 4 both products run on the matrix cores instead (MPV, see
//    consume_page_mpv): at 4 or 8 heads per kv head the VALU dot products
//    would take most of the vector issue rate at HBM speed (G = 8: 138 us
//    on the batch-64 lengths against 103 us this way; G = 4: 108 -> 102 us;
//    E4M3 pages at G = 4: 73 -> 60 us), while for G <= 2 the VALU path is as
//    fast or faster;
//  * each row group keeps its own online-softmax state (reference max in log2
//    units, sum, 16 fp32 accumulators per head); the reference is only moved
//    (and the accumulators rescaled) when a wave-wide vote finds a score more
//    than 2^8 above it, so most pages skip the rescale;
//  * a (request, kv head) cut into several pieces: each piece writes an fp32
//    partial state, then the last wave to arrive (an agent-scope counter per
//    split unit, counted one piece later so the wait for the stores is free)
//    merges all pieces and writes the final output, so one launch does the
//    whole decode. Counters and queue heads are reset by the kernel itself,
//    so it can be replayed from a graph.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pkfa {
namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kRescaleSlack = 8.0f;  // log2 units: probabilities stay <= 2^8
constexpr int kCoherent = 16;          // cache policy sc1: device-coherent access
// Cache policy nt (non-temporal) for K/V page loads: every byte is read once,
// so the lines are streamed rather than kept (batch-64 GQA decode over
// 9.7k pages: 123 -> 110 us per launch).
constexpr int kStream = 2;

// One page of the lane's two tokens (r and r+8). 16-bit pools: k[0], k[1]
// = token r dims [8s, 8s+8) and [64+8s, 64+8s+8), k[2], k[3] the same for
// token r+8. E4M3 pools (KV8): k[0] = token r dims [16s, 16s+16), k[1] =
// token r+8 (one 16-byte load per 128-byte row).
template <bool KV8>
struct PageRegs {
  static constexpr int N = KV8 ? 2 : 4;
  u32x4 k[N];
  u32x4 v[N];
};

// Dims of the lane's 16 accumulators: float4 group i (i = 0..3) of segment s
// starts at dim acc_dim(s, i).
template <bool KV8>
__device__ __forceinline__ int acc_dim(int s, int i) {
  return KV8 ? 16 * s + 4 * i : (i < 2 ? 8 * s + 4 * i : 64 + 8 * s + 4 * (i - 2));
}

// q operands of a piece. VALU path: lo[g], hi[g] = dims acc_dim(s, 0..1)
// and acc_dim(s, 2..3) of head g. MPV: b[i] = the B operand of the i-th
// 16x16x32 MFMA of the scores: head n = lane % 16 (zero for n >= G), dims
// 32i + 8 (lane / 16) .. +8 (E4M3 pools: dims 32 (lane / 16) + 8i .. +8, so
// that a lane's four K operands come from 32 consecutive code bytes).
template <int G, bool MPV>
struct QOps {
  u32x4 lo[G], hi[G];
};
template <int G>
struct QOps<G, true> {
  u32x4 b[4];
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == FA_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

// The fp32 partial outputs [slots][G][128] as one buffer (byte offsets < 2^31:
// the planner's capacities keep slots * G * 512 below that).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const AttnParams& p) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p.part_o, 0, 0x7fffffff, 0x00020000);
}

template <bool KV8>
__device__ __forceinline__ void load_page(PageRegs<KV8>& pr, const AttnParams& p, int pid, int hk,
                                          uint32_t bytes, const uint32_t (&off)[4]) {
  constexpr int N = PageRegs<KV8>::N;
  const int64_t base = ((int64_t)pid * p.page_stride + (int64_t)hk * p.head_stride) * (KV8 ? 1 : 2);
  const __amdgpu_buffer_rsrc_t rk =
      page_rsrc(reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(p.k) + base), bytes);
  const __amdgpu_buffer_rsrc_t rv =
      page_rsrc(reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(p.v) + base), bytes);
#pragma unroll
  for (int i = 0; i < N; ++i) pr.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off[i], 0, kStream);
#pragma unroll
  for (int i = 0; i < N; ++i) pr.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off[i], 0, kStream);
}

template <int DT, int G, bool KV8>
__device__ __forceinline__ void consume_page(const PageRegs<KV8>& pr, const QOps<G, false>& q,
                                             float (&m)[G], float (&l)[G], float (&acc)[G][16],
                                             float scale, bool va, bool vb) {
  using E = Elt<DT>;
  float sa[G], sb[G];
  // key pairs of tokens r (ka) and r+8 (kb) in the q layout: pair i < 4 meets
  // q.lo[g][i], pair 4 + i meets q.hi[g][i]
  uint32_t ka[8], kb[8];
  if constexpr (KV8) {
    // E4M3 codes widened to the q type; dword i holds dims 16s+4i .. 16s+4i+3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ka[2 * i] = E::template from_e4m3<false>(pr.k[0][i]);
      ka[2 * i + 1] = E::template from_e4m3<true>(pr.k[0][i]);
      kb[2 * i] = E::template from_e4m3<false>(pr.k[1][i]);
      kb[2 * i + 1] = E::template from_e4m3<true>(pr.k[1][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ka[i] = pr.k[0][i];
      ka[4 + i] = pr.k[1][i];
      kb[i] = pr.k[2][i];
      kb[4 + i] = pr.k[3][i];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x = E::dot2(q.lo[g][i], ka[i], x);
      y = E::dot2(q.lo[g][i], kb[i], y);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x = E::dot2(q.hi[g][i], ka[4 + i], x);
      y = E::dot2(q.hi[g][i], kb[4 + i], y);
    }
    const float xs = octet_sum(x) * scale;
    const float ys = octet_sum(y) * scale;
    sa[g] = va ? xs : kNegInf;
    sb[g] = vb ? ys : kNegInf;
  }
  bool need = false;
#pragma unroll
  for (int g = 0; g < G; ++g) need |= fmaxf(sa[g], sb[g]) > m[g] + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(m[g], fmaxf(sa[g], sb[g]));
      const float alpha = fast_exp2(m[g] - (mn == kNegInf ? 0.f : mn));
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[g][e] *= alpha;
      m[g] = mn;
    }
  }
  // element e of tokens r and r+8 side by side: (A_e, B_e)
  uint32_t pv[16];
  if constexpr (KV8) {
    // interleave the codes of the two tokens byte by byte (A0 B0 A1 B1 and
    // A2 B2 A3 B3), then widen each code pair
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p01 = __builtin_amdgcn_perm(pr.v[1][i], pr.v[0][i], 0x05010400u);
      const uint32_t p23 = __builtin_amdgcn_perm(pr.v[1][i], pr.v[0][i], 0x07030602u);
      pv[4 * i] = E::template from_e4m3<false>(p01);
      pv[4 * i + 1] = E::template from_e4m3<true>(p01);
      pv[4 * i + 2] = E::template from_e4m3<false>(p23);
      pv[4 * i + 3] = E::template from_e4m3<true>(p23);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[2 * i] = __builtin_amdgcn_perm(pr.v[2][i], pr.v[0][i], 0x05040100u);
      pv[2 * i + 1] = __builtin_amdgcn_perm(pr.v[2][i], pr.v[0][i], 0x07060302u);
      pv[8 + 2 * i] = __builtin_amdgcn_perm(pr.v[3][i], pr.v[1][i], 0x05040100u);
      pv[8 + 2 * i + 1] = __builtin_amdgcn_perm(pr.v[3][i], pr.v[1][i], 0x07060302u);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float ms = m[g] == kNegInf ? 0.f : m[g];
    const float pa = fast_exp2(sa[g] - ms);
    const float pb = fast_exp2(sb[g] - ms);
    l[g] += pa + pb;
    const uint32_t pp = E::pack(pa, pb);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = E::dot2(pp, pv[e], acc[g][e]);
  }
}

// ---- all matrix-core path (MPV) -----------------------------------------
// Lane l = 16 gq + c: column c is a head (zero q past G), lane group gq.
// K and V are loaded in the row-group layout of the VALU path (each load
// instruction reads the 128-byte halves of 8 token rows; the MFMA operand
// layouts read 64 bytes of 16 rows per instruction, which measured 16%
// slower at batch 64) and pass through a per-wave LDS page. Per page:
// S^T = K Q^T (4 x 16x16x32, K read back as A operands with ds_read_b128)
// leaves the scores of tokens 4gq .. 4gq+3 for head c in the lane, which is
// also the B-operand layout of P^T for O^T += V^T P^T (8 x 16x16x16, dims
// 16n .. 16n+15; V^T read by ds_read_b64_tr_b16). The online-softmax state
// is per head column (max across the 4 lane groups by two lane swaps) and
// O^T stays in 32 accumulators: the lane holds dims 16n + 4gq .. +3 of head c.
template <int G, bool MPV>
struct WaveState {
  float m[G], l[G], acc[G][16];
};
template <int G>
struct WaveState<G, true> {
  float m, l;
  f32x4 o[8];
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x16(v4s a, u32x2 b, f32x4 c) {
  if constexpr (DT == FA_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(v4s, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Per-wave V page in LDS: 16 token rows of 256 B (16-bit elements) at a
// stride of 288 B; the 16-byte chunk k (dims 8k .. 8k+7) of row r sits in
// slot k ^ (4 (r & 3) + r / 4). Of the layouts measured with
// SQ_LDS_BANK_CONFLICT (row strides 256, 272, 288, 320 B with six chunk
// swizzles), this one is free of bank conflicts for both the 16-byte row
// writes and the transposed 8-byte reads.
constexpr int kVRowBytes = 288;
constexpr int kVPageBytes = 16 * kVRowBytes;
__device__ __forceinline__ uint32_t vslot(int r, int k) {
  return (uint32_t)(r * kVRowBytes + ((k ^ (((r & 3) << 2) | (r >> 2))) << 4));
}

template <int DT, int G, bool KV8>
__device__ __forceinline__ void consume_page_mpv(const PageRegs<KV8>& pr, const QOps<G, true>& q,
                                                 uint8_t* vl, int lane, WaveState<G, true>& st,
                                                 float scale, int nvalid) {
  using E = Elt<DT>;
  const int t = lane & 15, gq = lane >> 4;
  // K and V were loaded in the row-group layout (lane = 8 r + s holds tokens
  // r and r+8, 16 bytes of each per load: every load instruction reads whole
  // 128-byte halves of 8 token rows); they reach the MFMA layouts through
  // the wave's LDS page (E4M3 codes widened to the q type on the way in).
  const int r = lane >> 3, sg = lane & 7;
  auto to_lds = [&](const u32x4 (&w)[PageRegs<KV8>::N]) {
    if constexpr (KV8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 x;
          x[0] = E::template from_e4m3<false>(w[i][2 * h]);
          x[1] = E::template from_e4m3<true>(w[i][2 * h]);
          x[2] = E::template from_e4m3<false>(w[i][2 * h + 1]);
          x[3] = E::template from_e4m3<true>(w[i][2 * h + 1]);
          *reinterpret_cast<u32x4*>(vl + vslot(r + 8 * i, 2 * sg + h)) = x;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(vl + vslot(r + 8 * (i >> 1), 8 * (i & 1) + sg)) = w[i];
    }
  };
  // scores S^T[token 4gq + j][head t]: A operand i = dims 32i + 8gq of token t.
  // E4M3: dims 32gq + 8i. The K codes go to LDS as they are (rows of 128
  // bytes, 16-byte chunk c of row r at c ^ ((r / 2) mod 8), so the 16 rows
  // a lane group reads fall in distinct banks); a lane reads its 32 code
  // bytes in two 16-byte reads and widens them itself: half the LDS traffic
  // of widening before the store.
  u32x4 ka[4];
  if constexpr (KV8) {
    auto kslot = [](int row, int c) { return (uint32_t)(row * 128 + ((c ^ ((row >> 1) & 7)) << 4)); };
    *reinterpret_cast<u32x4*>(vl + kslot(r, sg)) = pr.k[0];
    *reinterpret_cast<u32x4*>(vl + kslot(r + 8, sg)) = pr.k[1];
    const u32x4 c0 = *reinterpret_cast<const u32x4*>(vl + kslot(t, 2 * gq));
    const u32x4 c1 = *reinterpret_cast<const u32x4*>(vl + kslot(t, 2 * gq + 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4& c = i < 2 ? c0 : c1;
      const int w = 2 * (i & 1);
      ka[i] = u32x4{E::template from_e4m3<false>(c[w]), E::template from_e4m3<true>(c[w]),
                    E::template from_e4m3<false>(c[w + 1]), E::template from_e4m3<true>(c[w + 1])};
    }
  } else {
    to_lds(pr.k);
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[i] = *reinterpret_cast<const u32x4*>(vl + vslot(t, 4 * i + gq));
  }
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) c = mfma16x16x32<DT>(ka[i], q.b[i], c);
  // the V page replaces K in LDS (LDS operations of a wave run in order)
  to_lds(pr.v);
  // online softmax per head column
  float sv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sv[j] = 4 * gq + j < nvalid ? c[j] * scale : kNegInf;
  float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mx = pair32_max(pair16_max(mx));
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kRescaleSlack)) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - (mn == kNegInf ? 0.f : mn));
    st.l *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] *= alpha;
    st.m = mn;
  }
  const float ms = st.m == kNegInf ? 0.f : st.m;
  float pj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pj[j] = fast_exp2(sv[j] - ms);
  st.l += (pj[0] + pj[1]) + (pj[2] + pj[3]);
  const u32x2 pb = {E::pack(pj[0], pj[1]), E::pack(pj[2], pj[3])};
  // O^T += V^T P^T: lane reads dim 16n + t of tokens 4gq .. 4gq+3
  const int e = t >> 2, qq = t & 3;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const uint32_t a = vslot(4 * gq + e, 2 * n + (qq >> 1)) + 8u * (uint32_t)(qq & 1);
    const v4s va =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vl + a));
    st.o[n] = mfma16x16x16<DT>(va, pb, st.o[n]);
  }
}

// Sum the lane groups' partial row sums (the max is already common).
template <int G>
__device__ __forceinline__ void finish_state(WaveState<G, true>& st) {
  st.l = pair32_sum(pair16_sum(st.l));
}

template <int DT, int G, bool KV8>
__device__ __forceinline__ void write_final_mpv(const AttnParams& p, int row, int hk, int lane,
                                                const WaveState<G, true>& st) {
  const int c = lane & 15, gq = lane >> 4;
  if (c >= G) return;
  const int Hq = p.num_qo_heads;
  const int h = hk * G + c;
  const bool live = st.l > 0.f;
  const float inv = live ? p.v_scale / st.l : 0.f;
  uint16_t* op = p.out + ((int64_t)row * Hq + h) * 128 + 4 * gq;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const u32x2 w = {Elt<DT>::pack(st.o[n][0] * inv, st.o[n][1] * inv),
                     Elt<DT>::pack(st.o[n][2] * inv, st.o[n][3] * inv)};
    *reinterpret_cast<u32x2*>(op + 16 * n) = w;
  }
  if (gq == 0 && p.lse) p.lse[(int64_t)row * Hq + h] = live ? (st.m + fast_log2(st.l)) * kLn2 : kNegInf;
}

template <int G>
__device__ __forceinline__ void write_partial_mpv(const AttnParams& p, int64_t slot, int lane,
                                                  const WaveState<G, true>& st) {
  const int c = lane & 15, gq = lane >> 4;
  if (c >= G) return;
  const int64_t sh = slot * G + c;
  const bool live = st.l > 0.f;
  const float inv = live ? 1.f / st.l : 0.f;
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(p);
  const uint32_t o = (uint32_t)sh * 512u + 16u * (uint32_t)gq;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    u32x4 u;
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = __float_as_uint(st.o[n][k] * inv);
    __builtin_amdgcn_raw_buffer_store_b128(u, rs, o + 64u * n, 0, kCoherent);
  }
  if (gq == 0)
    __hip_atomic_store(p.part_lse + sh, live ? st.m + fast_log2(st.l) : kNegInf, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Online merge of the fp32 partial states in slots base .. base+C-1: the 16 /
// G copies of each head column (lanes c, c + G, ...) take every (16/G)-th
// piece, then the copies are merged across lanes. Leaves a finished state
// (l summed) in the lanes of column c < G.
template <int G>
__device__ __forceinline__ void gather_partials_mpv(const AttnParams& p, int64_t base, int C,
                                                    int lane, WaveState<G, true>& st) {
  constexpr int NC = 16 / G;  // copies of a head column
  const int c = lane & 15, gq = lane >> 4;
  const int hc = c % G, copy = c / G;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(p);
  for (int k = copy; k < C; k += NC) {
    const int64_t sh = (base + k) * G + hc;
    const float s2 = __hip_atomic_load(p.part_lse + sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t o = (uint32_t)sh * 512u + 16u * (uint32_t)gq;
    f32x4 v[8];
#pragma unroll
    for (int n = 0; n < 8; ++n)
      v[n] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o + 64u * n, 0,
                                                                             kCoherent));
    const float mn = fmaxf(st.m, s2);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float f = fast_exp2(st.m - ms);
    const float w = fast_exp2(s2 - ms);
    st.l = st.l * f + w;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = st.o[n] * f + w * v[n];
    st.m = mn;
  }
  // merge the copies: lanes c ^ (G << b) inside each row of 16
#pragma unroll
  for (int b = G; b < 16; b <<= 1) {
    const float m2 = __shfl_xor(st.m, b, 64);
    const float mn = fmaxf(st.m, m2);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float f = fast_exp2(st.m - ms);
    st.l = st.l * f;
    st.l += __shfl_xor(st.l, b, 64);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x = st.o[n][k] * f;
        st.o[n][k] = x + __shfl_xor(x, b, 64);
      }
    }
    st.m = mn;
  }
}

// Merge the 8 row-group states of the wave (lanes that differ in bits 3..5).
template <int G>
__device__ __forceinline__ void merge_row_groups(float (&m)[G], float (&l)[G],
                                                 float (&acc)[G][16]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = m[g];
    M = fmaxf(M, xor8(M));
    M = pair32_max(pair16_max(M));
    const float f = fast_exp2(m[g] - (M == kNegInf ? 0.f : M));
    float L = l[g] * f;
    L += xor8(L);
    L = pair32_sum(pair16_sum(L));
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float a = acc[g][e] * f;
      a += xor8(a);
      acc[g][e] = pair32_sum(pair16_sum(a));
    }
    m[g] = M;
    l[g] = L;
  }
}

// Online merge of the fp32 partial states in slots base .. base+C-1 (slot
// layout [slot][G][128], piece c taken by row group c % 8). The partials were
// published by other waves with device-coherent stores; they are read back
// with device-coherent loads (sc1).
template <int G, bool KV8>
__device__ __forceinline__ void gather_partials(const AttnParams& p, int64_t base, int C, int r,
                                                int s, float (&m)[G], float (&l)[G],
                                                float (&acc)[G][16]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = 0.f;
  }
  // one resource over the whole partial array: row groups read different slots
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(p);
  auto load_state = [&](int c, int g, float& s2, float (&v)[16]) {
    const int64_t sh = (base + c) * G + g;
    s2 = __hip_atomic_load(p.part_lse + sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t o = (uint32_t)sh * 512u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 raw =
          __builtin_amdgcn_raw_buffer_load_b128(rs, o + 4 * acc_dim<KV8>(s, i), 0, kCoherent);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[4 * i + k] = __uint_as_float(raw[k]);
    }
  };
  auto add_state = [&](int g, float s2, const float (&v)[16]) {
    const float mn = fmaxf(m[g], s2);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float f = fast_exp2(m[g] - ms);
    const float w = fast_exp2(s2 - ms);
    l[g] = l[g] * f + w;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = acc[g][e] * f + w * v[e];
    m[g] = mn;
  };
  // up to four chunks per row group per round (c, c+8, c+16, c+24), all
  // requested before any is used: a unit of up to 32 pieces is one round trip
  for (int c = r; c < C; c += 32) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s2[4], v[4][16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s2[u] = kNegInf;
        if (c + 8 * u < C) load_state(c + 8 * u, g, s2[u], v[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c + 8 * u < C) add_state(g, s2[u], v[u]);
    }
  }
}

template <int DT, int G, bool KV8>
__device__ __forceinline__ void write_final(const AttnParams& p, int row, int hk, int r, int s,
                                            const float (&m)[G], const float (&l)[G],
                                            const float (&acc)[G][16]) {
  const int Hq = p.num_qo_heads;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (r != g) continue;  // row group g writes head g of the group
    const int h = hk * G + g;
    const bool live = l[g] > 0.f;
    // the V scale (1 for unscaled pools) joins the normalisation
    const float inv = live ? p.v_scale / l[g] : 0.f;
    uint16_t* op = p.out + ((int64_t)row * Hq + h) * 128;
    u32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = Elt<DT>::pack(acc[g][2 * i] * inv, acc[g][2 * i + 1] * inv);
      hi[i] = Elt<DT>::pack(acc[g][8 + 2 * i] * inv, acc[g][8 + 2 * i + 1] * inv);
    }
    *reinterpret_cast<u32x4*>(op + acc_dim<KV8>(s, 0)) = lo;
    *reinterpret_cast<u32x4*>(op + acc_dim<KV8>(s, 2)) = hi;
    if (s == 0 && p.lse)
      p.lse[(int64_t)row * Hq + h] = live ? (m[g] + fast_log2(l[g])) * kLn2 : kNegInf;
  }
}

// Publish a chunk's normalised state with device-coherent stores (sc1), so a
// wave on any XCD can read it after the arrival counter says it is complete.
template <int G, bool KV8>
__device__ __forceinline__ void write_partial(const AttnParams& p, int64_t slot, int r, int s,
                                              const float (&m)[G], const float (&l)[G],
                                              const float (&acc)[G][16]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (r != g) continue;
    const int64_t sh = slot * G + g;
    const bool live = l[g] > 0.f;
    const float inv = live ? 1.f / l[g] : 0.f;
    const __amdgpu_buffer_rsrc_t rs = part_rsrc(p);
    const uint32_t o = (uint32_t)sh * 512u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 u;
#pragma unroll
      for (int k = 0; k < 4; ++k) u[k] = __float_as_uint(acc[g][4 * i + k] * inv);
      __builtin_amdgcn_raw_buffer_store_b128(u, rs, o + 4 * acc_dim<KV8>(s, i), 0, kCoherent);
    }
    if (s == 0)
      __hip_atomic_store(p.part_lse + sh, live ? m[g] + fast_log2(l[g]) : kNegInf, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Identity of a piece, wave-uniform.
struct PieceId {
  int row, hk, base, slot, npieces;
};

// A piece being set up: tile fields (wave-uniform after v_readlane), its page
// ids (lane i holds pages i and i+64; at most 128 pages, a planner guarantee)
// and the device page-table check (kv_indptr[b], kv_indptr[b+1],
// last_page_len[b] in lanes 0..2).
struct PieceCtx {
  PieceId id;
  int pbeg, key0, key1_plan, first_page, npg_plan;
  int ids0, ids1, chk;
};

// Request the tile of piece t (one VGPR, lanes 0..7).
__device__ __forceinline__ int load_tile(const AttnParams& p, int t, int lane) {
  return p.tiles[t * 8 + (lane & 7)];
}

// Take the tile fields and request the page ids and the page-table check.
__device__ __forceinline__ void open_piece(const AttnParams& p, int tv, int lane, PieceCtx& c) {
  const int b = __builtin_amdgcn_readlane(tv, 0);
  c.id.row = b;
  c.id.hk = __builtin_amdgcn_readlane(tv, 1);
  c.pbeg = __builtin_amdgcn_readlane(tv, 2);
  c.id.base = __builtin_amdgcn_readlane(tv, 3);
  c.key0 = __builtin_amdgcn_readlane(tv, 4);
  c.key1_plan = __builtin_amdgcn_readlane(tv, 5);
  c.id.slot = __builtin_amdgcn_readlane(tv, 6);
  c.id.npieces = __builtin_amdgcn_readlane(tv, 7);
  c.first_page = c.key0 >> 4;
  c.npg_plan = c.key1_plan > c.key0 ? ((c.key1_plan + 15) >> 4) - c.first_page : 0;
  if (p.kv_offsets) {
    // ragged KV: page j of the piece starts at row pbeg + 16 (first_page + j)
    // (the tile carries kv_offsets[b]); the check reads the row offsets
    const int row0 = c.pbeg + 16 * c.first_page;
    c.ids0 = lane < c.npg_plan ? row0 + 16 * lane : 0;
    c.ids1 = lane + 64 < c.npg_plan ? row0 + 16 * (lane + 64) : 0;
    c.chk = lane == 0 ? p.kv_offsets[b] : lane == 1 ? p.kv_offsets[b + 1] : 0;
  } else {
    const int32_t* ids_base = p.kv_indices + c.pbeg + c.first_page;
    c.ids0 = lane < c.npg_plan ? ids_base[lane] : 0;
    c.ids1 = lane + 64 < c.npg_plan ? ids_base[lane + 64] : 0;
    c.chk = lane == 0 ? p.kv_indptr[b] : lane == 1 ? p.kv_indptr[b + 1] : p.last_page_len[b];
  }
}

// Wave-uniform bounds of a piece, taken from its context once its loads have
// arrived.
struct PieceRun {
  int hk, row, key1, first_page, npg;
};

// Bytes per token row of the pool, and the lane's load offsets in a page.
template <bool KV8>
__device__ __forceinline__ uint32_t page_offsets(const AttnParams& p, int lane, uint32_t (&off)[4]) {
  const uint32_t r = lane >> 3, s = lane & 7;
  const uint32_t ts2 = (uint32_t)p.token_stride * (KV8 ? 1u : 2u);
  if constexpr (KV8) {
    off[0] = r * ts2 + s * 16u;
    off[1] = (r + 8) * ts2 + s * 16u;
    off[2] = off[3] = 0u;  // unused
  } else {
    off[0] = r * ts2 + s * 16u;
    off[1] = r * ts2 + 128u + s * 16u;
    off[2] = (r + 8) * ts2 + s * 16u;
    off[3] = (r + 8) * ts2 + 128u + s * 16u;
  }
  return ts2;
}

__device__ __forceinline__ int page_id_of(const PieceCtx& c, int j) {
  return j < 64 ? __builtin_amdgcn_readlane(c.ids0, j & 63) : __builtin_amdgcn_readlane(c.ids1, j & 63);
}

// Bytes of page j of a piece that hold valid tokens (a buffer load past them
// returns 0); kept scalar so the buffer resource needs no per-lane loop.
__device__ __forceinline__ uint32_t page_bytes_of(const PieceRun& run, int j, uint32_t ts2) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(min(16, run.key1 - (run.first_page + j) * 16) *
                                                  (int)ts2);
}

// Start a piece: check it against the device page table, request its q rows
// and its first NBUF-1 pages into the ring. The caller runs this before the
// previous piece's epilogue, which then overlaps the first loads' latency.
template <int G, int NBUF, bool KV8, bool MPV>
__device__ __forceinline__ void begin_piece(const AttnParams& p, const PieceCtx& c, int lane,
                                            PieceRun& run, PageRegs<KV8> (&buf)[NBUF],
                                            QOps<G, MPV>& q) {
  // The context's fields are wave-uniform; readfirstlane says so to the
  // compiler (it loses track across the loop that hands pieces over), so the
  // page buffer resources stay scalar.
  run.hk = __builtin_amdgcn_readfirstlane(c.id.hk);
  run.row = __builtin_amdgcn_readfirstlane(c.id.row);
  // The device page table must agree with the plan (offset, and the key
  // range inside the request's valid tokens); a piece that disagrees reads
  // nothing.
  const int span = __builtin_amdgcn_readlane(c.chk, 1) - __builtin_amdgcn_readlane(c.chk, 0);
  const int kv_len = p.kv_offsets ? span  // ragged: rows
                                  : (span > 0 ? (span - 1) * 16 + __builtin_amdgcn_readlane(c.chk, 2) : 0);
  const int key0 = __builtin_amdgcn_readfirstlane(c.key0);
  const int key1_plan = __builtin_amdgcn_readfirstlane(c.key1_plan);
  const bool agrees = __builtin_amdgcn_readlane(c.chk, 0) == __builtin_amdgcn_readfirstlane(c.pbeg) &&
                      key1_plan <= kv_len;
  run.first_page = __builtin_amdgcn_readfirstlane(c.first_page);
  run.key1 = agrees ? key1_plan : key0;
  run.npg = agrees ? __builtin_amdgcn_readfirstlane(c.npg_plan) : 0;
  const int s = lane & 7;
  const uint16_t* qp = p.q + ((int64_t)run.row * p.num_qo_heads + run.hk * G) * 128;
  if constexpr (MPV) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      q.b[i] = n < G ? *reinterpret_cast<const u32x4*>(qp + n * 128 + (KV8 ? 32 * g + 8 * i
                                                                           : 32 * i + 8 * g))
                     : u32x4{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      q.lo[g] = *reinterpret_cast<const u32x4*>(qp + g * 128 + acc_dim<KV8>(s, 0));
      q.hi[g] = *reinterpret_cast<const u32x4*>(qp + g * 128 + acc_dim<KV8>(s, 2));
    }
  }
  uint32_t off[4];
  const uint32_t ts2 = page_offsets<KV8>(p, lane, off);
  if (run.npg >= 2 * NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u)
      load_page(buf[u], p, page_id_of(c, u), run.hk, 16u * ts2, off);
  } else {
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u)
      if (u < run.npg)
        load_page(buf[u], p, page_id_of(c, u), run.hk, page_bytes_of(run, u, ts2), off);
  }
}

// Stream one piece begun by begin_piece: keys [key0, key1) of kv head hk of
// request row, for its G q heads; leaves the state per row group in (m, l,
// acc). hook(k) runs at the start of steady ring pass k counted from the end
// (k = 2, 1, 0 for the last three passes; all three run after the loop if
// the piece has fewer), where the caller overlaps the set-up of its next
// piece with the loads.
template <int DT, int G, int NBUF, bool KV8, bool MPV, typename Hook>
__device__ __forceinline__ void stream_piece(const AttnParams& p, const PieceCtx& c,
                                             const PieceRun& run, int lane,
                                             PageRegs<KV8> (&buf)[NBUF], const QOps<G, MPV>& q,
                                             void* lds, WaveState<G, MPV>& st, Hook&& hook) {
  const int r = lane >> 3;
  const int hk = run.hk, npg = run.npg, key1 = run.key1;
  uint32_t off[4];
  const uint32_t ts2 = page_offsets<KV8>(p, lane, off);
  if constexpr (MPV) {
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      st.m[g] = kNegInf;
      st.l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[g][e] = 0.f;
    }
  }
  auto consume = [&](const PageRegs<KV8>& pr, int nvalid) {
    if constexpr (MPV)
      consume_page_mpv<DT, G, KV8>(pr, q, static_cast<uint8_t*>(lds), lane, st, p.scale_log2,
                                   nvalid);
    else
      consume_page<DT, G, KV8>(pr, q, st.m, st.l, st.acc, p.scale_log2, r < nvalid, r + 8 < nvalid);
  };
  int j = 0;
  int hooks_left = 3;
  if (npg >= 2 * NBUF) {
    // Steady state: every page touched here is full and has a successor, so
    // all loads are unconditional and the next page id is fetched one page
    // ahead; the compiler then keeps NBUF-1 pages in flight.
    const uint32_t full = 16u * ts2;
    int nid = page_id_of(c, NBUF - 1);
    auto ring_pass = [&](int j0) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int jn = j0 + u + NBUF - 1;
        const int pid = nid;
        nid = page_id_of(c, jn + 1);
        load_page(buf[(u + NBUF - 1) % NBUF], p, pid, hk, full, off);
        consume(buf[u], 16);
      }
    };
    // passes: the peeled first one, then while j + 2 NBUF - 1 < npg
    const int passes = 1 + (npg - NBUF) / NBUF - ((npg - NBUF) % NBUF == 0 ? 1 : 0);
    // The first pass is peeled so that the q loads are waited for there; in
    // the loop only K/V page loads are then outstanding at the loop header
    // and the compiler's wait counts keep NBUF-1 pages in flight.
    if (passes - 1 < 3) hook(--hooks_left);
    ring_pass(0);
    int k = 1;
    for (j = NBUF; j + 2 * NBUF - 1 < npg; j += NBUF, ++k) {
      if (passes - 1 - k < hooks_left) hook(--hooks_left);
      ring_pass(j);
    }
  }
  // Tail: at most 2*NBUF-1 pages, the last one possibly partial.
  for (; j < npg; j += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int jj = j + u;
      if (jj >= npg) break;
      const int jn = jj + NBUF - 1;
      if (jn < npg)
        load_page(buf[(u + NBUF - 1) % NBUF], p, page_id_of(c, jn), hk, page_bytes_of(run, jn, ts2),
                  off);
      const int tb = (run.first_page + jj) * 16;
      consume(buf[u], key1 - tb);
    }
  }
  while (hooks_left > 0) hook(--hooks_left);
}

// Worker wave w runs the pieces worker_ptr[w] .. worker_ptr[w+1]-1 in order
// (the planner gives every wave the same number of pages). The next piece's
// tile and page ids are requested while the current piece's last pages
// stream, so a new piece starts without a dependent round trip. A split
// unit's pieces publish fp32 partial states; a wave reports a piece's
// arrival only after its next piece (the partial's stores have long
// completed by then, so the wait is free), and the last arriving piece
// merges the unit and clears its counter, so the kernel can be replayed from
// a graph.
template <int DT, int G, int NBUF, bool KV8, bool MPV>
__device__ __forceinline__ void decode_worker(const AttnParams& p, int w, void* lds) {
  const int lane = threadIdx.x & 63;
  const int r = lane >> 3, s = lane & 7;
  if (w >= p.header[6]) return;  // the grid rounds the worker count up to whole workgroups
  const int t_end = __builtin_amdgcn_readfirstlane(p.worker_ptr[w + 1]);
  int t = __builtin_amdgcn_readfirstlane(p.worker_ptr[w]);
  auto fetch_add = [&](int32_t* ptr) -> int {  // lane 0 only; result read by readlane
    int v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(ptr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
  };
  WaveState<G, MPV> st;
  // arrival of a split piece whose partial was published earlier; the last
  // arrival of the unit merges all its pieces and writes the output
  auto finish_arrival = [&](const PieceId& pd, int arr) {
    if (__builtin_amdgcn_readlane(arr, 0) != pd.npieces - 1) return;
    if (lane == 0) p.counters[pd.base] = 0;
    if constexpr (MPV) {
      gather_partials_mpv<G>(p, pd.base, pd.npieces, lane, st);
      write_final_mpv<DT, G, KV8>(p, pd.row, pd.hk, lane, st);
    } else {
      gather_partials<G, KV8>(p, pd.base, pd.npieces, r, s, st.m, st.l, st.acc);
      merge_row_groups<G>(st.m, st.l, st.acc);
      write_final<DT, G, KV8>(p, pd.row, pd.hk, r, s, st.m, st.l, st.acc);
    }
  };
  auto arrive = [&](const PieceId& pd) -> int {
    // the partial's coherent stores must be complete before the count
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return fetch_add(p.counters + pd.base);
  };

  PieceId pd = {0, 0, -1, -1, 0};  // pending arrival (slot < 0: none)
  PieceCtx cur, nxt;
  PieceRun run, nrun;
  PageRegs<KV8> buf[NBUF];
  QOps<G, MPV> q;
  if (t < t_end) {
    open_piece(p, load_tile(p, t, lane), lane, cur);
    begin_piece<G, NBUF, KV8, MPV>(p, cur, lane, run, buf, q);
  }
  while (t < t_end) {
    // overlapped set-up of the next piece: request its tile (pass 2 from the
    // end) and its page ids (pass 1); it begins (q and first pages requested)
    // before this piece's epilogue
    const int tn = t + 1;
    int tvn = 0;
    auto hook = [&](int k) {
      if (k == 2 && tn < t_end) tvn = load_tile(p, tn, lane);
      if (k == 1 && tn < t_end) open_piece(p, tvn, lane, nxt);
    };
    stream_piece<DT, G, NBUF, KV8, MPV>(p, cur, run, lane, buf, q, lds, st, hook);
    const int arr = pd.slot >= 0 ? arrive(pd) : 0;
    if (tn < t_end) begin_piece<G, NBUF, KV8, MPV>(p, nxt, lane, nrun, buf, q);
    if constexpr (MPV) {
      finish_state<G>(st);
      if (cur.id.slot < 0)
        write_final_mpv<DT, G, KV8>(p, cur.id.row, cur.id.hk, lane, st);
      else
        write_partial_mpv<G>(p, cur.id.slot, lane, st);
    } else {
      merge_row_groups<G>(st.m, st.l, st.acc);
      if (cur.id.slot < 0)
        write_final<DT, G, KV8>(p, cur.id.row, cur.id.hk, r, s, st.m, st.l, st.acc);
      else
        write_partial<G, KV8>(p, cur.id.slot, r, s, st.m, st.l, st.acc);
    }
    if (pd.slot >= 0) finish_arrival(pd, arr);
    pd = cur.id;
    t = tn;
    cur = nxt;
    run = nrun;
  }
  if (pd.slot >= 0) finish_arrival(pd, arrive(pd));
}

}  // namespace dec
}  // namespace pkfa
