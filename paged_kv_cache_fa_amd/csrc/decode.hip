// Paged-KV decode kernel for gfx950.
//
// What it computes: for each request b and query head h, scaled-dot-product
// attention of q[b, h] over the request's keys gathered through its page
// table ([DeepDive] "FlashInfer: The Attention Kernel Library That Proves the
// Bottleneck ...", section "Snippet One: Paged KV-Cache Attention and MLA":
// page pool, CSR page list, last_page_len), split into key chunks by the
// planner ([Guide] "FlashInfer: GPU Kernels for LLM Inference (2026 Guide)",
// section "What FlashInfer is", idea 3). A chunk's state (out, lse) is either
// final or an fp32 partial merged later by log-sum-exp ([Guide] section
// "Cascade attention for shared prefixes").
//
// MI355X design (decode is HBM-bound, so no MFMA):
//  * one wave64 per tile {request, kv head, key chunk}; 4 independent waves
//    per 256-thread workgroup, no barriers;
//  * all G = Hq/Hkv query heads of the kv head are packed in the wave (GQA),
//    so each K/V byte is read from HBM once for all of them;
//  * lane = 8 x row-group + segment: row group r (0..7) owns tokens r and r+8
//    of every 16-token page, segment s (0..7) owns dims [8s, 8s+8) and
//    [64+8s, 64+8s+8); each K/V row (256 B) is two fully coalesced 128-byte
//    halves, 16 bytes per lane (buffer_load_dwordx4);
//  * loads go through a per-page buffer resource whose size stops at the
//    last valid token, so slots past last_page_len read as zero without any
//    memory access and without branches;
//  * scores: packed 2-element dot products (v_dot2_f32_bf16 / _f16) and an
//    8-lane DPP sum; every row group keeps its own online-softmax state
//    (running max in log2 units, sum, 16 fp32 accumulators per head), merged
//    across the 8 row groups once at the end;
//  * the next page is loaded while the current one is consumed, and page ids
//    are fetched 64 at a time one batch ahead.
#include "device_common.h"
#include "kernels.h"

namespace pkfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PageRegs {
  u32x4 k[4];  // token r lo/hi, token r+8 lo/hi
  u32x4 v[4];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void load_page(PageRegs& pr, const AttnParams& p, int pid, int hk,
                                          uint32_t bytes, const uint32_t (&off)[4]) {
  const int64_t base = (int64_t)pid * p.page_stride + (int64_t)hk * p.head_stride;
  const __amdgpu_buffer_rsrc_t rk = page_rsrc(p.k + base, bytes);
  const __amdgpu_buffer_rsrc_t rv = page_rsrc(p.v + base, bytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) pr.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off[i], 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) pr.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off[i], 0, 0);
}

template <int DT, int G>
__device__ __forceinline__ void consume_page(const PageRegs& pr, const u32x4 (&qlo)[G],
                                             const u32x4 (&qhi)[G], float (&m)[G], float (&l)[G],
                                             float (&acc)[G][16], float scale, bool va, bool vb) {
  using E = Elt<DT>;
  float sa[G], sb[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x = E::dot2(qlo[g][i], pr.k[0][i], x);
      y = E::dot2(qlo[g][i], pr.k[2][i], y);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x = E::dot2(qhi[g][i], pr.k[1][i], x);
      y = E::dot2(qhi[g][i], pr.k[3][i], y);
    }
    sa[g] = va ? octet_sum(x) * scale : kNegInf;
    sb[g] = vb ? octet_sum(y) * scale : kNegInf;
  }
  float va_f[16], vb_f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    va_f[2 * i] = E::lo(pr.v[0][i]);
    va_f[2 * i + 1] = E::hi(pr.v[0][i]);
    va_f[8 + 2 * i] = E::lo(pr.v[1][i]);
    va_f[8 + 2 * i + 1] = E::hi(pr.v[1][i]);
    vb_f[2 * i] = E::lo(pr.v[2][i]);
    vb_f[2 * i + 1] = E::hi(pr.v[2][i]);
    vb_f[8 + 2 * i] = E::lo(pr.v[3][i]);
    vb_f[8 + 2 * i + 1] = E::hi(pr.v[3][i]);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mn = fmaxf(m[g], fmaxf(sa[g], sb[g]));
    const float ms = mn == kNegInf ? 0.f : mn;
    const float alpha = fast_exp2(m[g] - ms);
    const float pa = fast_exp2(sa[g] - ms);
    const float pb = fast_exp2(sb[g] - ms);
    l[g] = l[g] * alpha + pa + pb;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = acc[g][e] * alpha + pa * va_f[e] + pb * vb_f[e];
    m[g] = mn;
  }
}

template <int DT, int G>
__global__ __launch_bounds__(256) void decode_kernel(AttnParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tile_id = blockIdx.x * 4 + wave;
  if (tile_id >= p.header[0]) return;
  const int32_t* t = p.tiles + tile_id * 8;
  const int b = t[0], hk = t[1], row = t[2], slot0 = t[6];
  const int key0 = t[4];
  const int pbeg = p.kv_indptr[b];
  const int npages_req = p.kv_indptr[b + 1] - pbeg;
  const int kv_len = npages_req > 0 ? (npages_req - 1) * 16 + p.last_page_len[b] : 0;
  const int key1 = min(t[5], kv_len);
  const int Hq = p.num_qo_heads;

  const int r = lane >> 3;
  const int s = lane & 7;
  // byte offsets inside a page (relative to the kv head's row of slot 0)
  const uint32_t ts2 = (uint32_t)p.token_stride * 2u;
  const uint32_t off[4] = {r * ts2 + s * 16u, r * ts2 + 128u + s * 16u, (r + 8) * ts2 + s * 16u,
                           (r + 8) * ts2 + 128u + s * 16u};

  u32x4 qlo[G], qhi[G];
  const uint16_t* qp = p.q + ((int64_t)row * Hq + hk * G) * 128;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qlo[g] = *reinterpret_cast<const u32x4*>(qp + g * 128 + s * 8);
    qhi[g] = *reinterpret_cast<const u32x4*>(qp + g * 128 + 64 + s * 8);
  }
  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = 0.f;
  }

  const int first_page = key0 >> 4;
  const int npg = key1 > key0 ? ((key1 + 15) >> 4) - first_page : 0;
  const int32_t* ids_base = p.kv_indices + pbeg + first_page;
  int ids = lane < npg ? ids_base[lane] : 0;
  int ids_next = lane + 64 < npg ? ids_base[64 + lane] : 0;
  auto page_id = [&](int j) -> int {
    if (j > 0 && (j & 63) == 0) {
      ids = ids_next;
      ids_next = j + 64 + lane < npg ? ids_base[j + 64 + lane] : 0;
    }
    return __builtin_amdgcn_readlane(ids, j & 63);
  };
  // bytes of the page that hold valid tokens (a buffer load past them returns 0)
  auto page_bytes = [&](int j) -> uint32_t {
    const int valid = min(16, key1 - (first_page + j) * 16);
    return (uint32_t)valid * ts2;
  };
  const float scale = p.scale_log2;

  PageRegs A, B;
  if (npg > 0) load_page(A, p, page_id(0), hk, page_bytes(0), off);
  for (int j = 0; j < npg; j += 2) {
    if (j + 1 < npg) load_page(B, p, page_id(j + 1), hk, page_bytes(j + 1), off);
    {
      const int tb = (first_page + j) * 16;
      consume_page<DT, G>(A, qlo, qhi, m, l, acc, scale, tb + r < key1, tb + r + 8 < key1);
    }
    if (j + 1 >= npg) break;
    if (j + 2 < npg) load_page(A, p, page_id(j + 2), hk, page_bytes(j + 2), off);
    {
      const int tb = (first_page + j + 1) * 16;
      consume_page<DT, G>(B, qlo, qhi, m, l, acc, scale, tb + r < key1, tb + r + 8 < key1);
    }
  }

  // merge the 8 row-group states (lanes that differ in bits 3..5)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = m[g];
    M = fmaxf(M, xor_shfl(M, 8));
    M = fmaxf(M, xor_shfl(M, 16));
    M = fmaxf(M, xor_shfl(M, 32));
    const float Ms = M == kNegInf ? 0.f : M;
    const float f = fast_exp2(m[g] - Ms);
    float L = l[g] * f;
    L += xor_shfl(L, 8);
    L += xor_shfl(L, 16);
    L += xor_shfl(L, 32);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float a = acc[g][e] * f;
      a += xor_shfl(a, 8);
      a += xor_shfl(a, 16);
      a += xor_shfl(a, 32);
      acc[g][e] = a;
    }
    m[g] = M;
    l[g] = L;
  }

  // row group g writes head g of the group
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (r != g) continue;
    const int h = hk * G + g;
    const bool live = l[g] > 0.f;
    const float inv = live ? 1.f / l[g] : 0.f;
    const float lse2 = live ? m[g] + fast_log2(l[g]) : kNegInf;  // log2 units
    if (slot0 < 0) {
      uint16_t* op = p.out + ((int64_t)row * Hq + h) * 128;
      u32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = Elt<DT>::pack(acc[g][2 * i] * inv, acc[g][2 * i + 1] * inv);
        hi[i] = Elt<DT>::pack(acc[g][8 + 2 * i] * inv, acc[g][8 + 2 * i + 1] * inv);
      }
      *reinterpret_cast<u32x4*>(op + s * 8) = lo;
      *reinterpret_cast<u32x4*>(op + 64 + s * 8) = hi;
      if (s == 0 && p.lse) p.lse[(int64_t)row * Hq + h] = lse2 * kLn2;
    } else {
      float* op = p.part_o + ((int64_t)slot0 * Hq + h) * 128;
      float4* o4 = reinterpret_cast<float4*>(op + s * 8);
      o4[0] = make_float4(acc[g][0] * inv, acc[g][1] * inv, acc[g][2] * inv, acc[g][3] * inv);
      o4[1] = make_float4(acc[g][4] * inv, acc[g][5] * inv, acc[g][6] * inv, acc[g][7] * inv);
      float4* o4h = reinterpret_cast<float4*>(op + 64 + s * 8);
      o4h[0] = make_float4(acc[g][8] * inv, acc[g][9] * inv, acc[g][10] * inv, acc[g][11] * inv);
      o4h[1] = make_float4(acc[g][12] * inv, acc[g][13] * inv, acc[g][14] * inv, acc[g][15] * inv);
      if (s == 0) p.part_lse[(int64_t)slot0 * Hq + h] = lse2;
    }
  }
}

template <int DT>
hipError_t launch_dt(const AttnParams& p, int group, int grid, hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<DT, 1>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<DT, 2>), dim3(grid), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<DT, 4>), dim3(grid), dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<DT, 8>), dim3(grid), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnParams& p, int dtype, int group, int max_tiles, hipStream_t s) {
  const int grid = (max_tiles + 3) / 4;
  if (grid <= 0) return hipSuccess;
  return dtype == FA_BF16 ? launch_dt<FA_BF16>(p, group, grid, s)
                          : launch_dt<FA_F16>(p, group, grid, s);
}

}  // namespace pkfa
