// Paged-KV append / prefill kernel for gfx950 (MFMA).
//
// What it computes ([Guide] "FlashInfer: GPU Kernels for LLM Inference (2026
// Guide)", section "Features (from the repository README)": prefill and
// append over paged and ragged caches; [DeepDive] "FlashInfer: The Attention
// Kernel Library That Proves the Bottleneck ...", section "Snippet One"):
// request b has qo_len new query rows whose K/V are already in its pages;
// with the causal mask, row i (position kv_len - qo_len + i) attends to keys
// 0 .. kv_len - qo_len + i. Without it, every row sees all kv_len keys (the
// shared-prefix pass of cascade attention, [Guide] section "Cascade attention
// for shared prefixes").
//
// MI355X design (the work is a dense contraction, so it runs on MFMA):
//  * one workgroup per tile {request, kv head, 32 query rows, key chunk},
//    one wave per query head of the kv head's group (GQA): the G waves share
//    every K/V block staged in LDS;
//  * K/V blocks of 64 keys are fetched with 16-byte global loads one block
//    ahead into registers and stored to a double-buffered LDS; V is written
//    transposed (4 keys x 8 dims per thread, regrouped with v_perm) so the
//    PV operand reads 4 consecutive keys per dim;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: each lane then owns one query column and
//    16 of its 32 keys per tile, so the online-softmax max / sum need one
//    cross-lane exchange (lanes l and l^32) and the rescale of the output
//    accumulators is lane-local;
//  * O^T += V^T P^T reuses the score registers (rounded to the input type) as
//    the B operand; the contraction index (keys) is permuted identically in
//    both operands, so the result is unaffected;
//  * a chunked (split) query tile writes fp32 partial states; the last
//    workgroup of the split (agent-scope counter, reset by that workgroup)
//    merges them by log-sum-exp.
#include "device_common.h"
#include "kernels.h"

namespace pkfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int kBlockKeys = 64;
constexpr int kKStride = 136;  // 16-bit elements per K row in LDS (128 dims + 8 pad)
constexpr int kVStride = 68;   // 16-bit elements per V^T row in LDS (64 keys + 4 pad)
constexpr int kKElems = kBlockKeys * kKStride;
constexpr int kVElems = 128 * kVStride;
constexpr int kBufElems = kKElems + kVElems;
constexpr int kCoherent = 16;  // cache policy sc1: device-coherent access

template <int DT>
struct Mfma;
template <>
struct Mfma<FA_BF16> {
  __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<FA_F16> {
  __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const AttnParams& p) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p.part_o, 0, 0x7fffffff, 0x00020000);
}

// One thread's share of a K/V block: tasks of 4 consecutive keys x 8 dims.
template <int TPT>
struct Stage {
  u32x4 k[TPT][4];
  u32x4 v[TPT][4];
};

template <int G>
struct Geo {
  static constexpr int kThreads = 64 * G;
  static constexpr int kTasks = (kBlockKeys / 4) * (128 / 8);  // 256
  static constexpr int kTPT = kTasks >= kThreads ? kTasks / kThreads : 1;
};

template <int DT, int G>
__global__ __launch_bounds__(64 * G) void append_kernel(AttnParams p) {
  using GE = Geo<G>;
  constexpr int TPT = GE::kTPT;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kBufElems];
  __shared__ int s_flag;

  const int tile_id = blockIdx.x;
  if (tile_id >= p.header[0]) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // query head within the group
  const int lane = tid & 63;
  const int jq = lane & 31, h = lane >> 5;

  // tile fields, made wave-uniform
  const int32_t* t = p.tiles + tile_id * 8;
  const int tv = t[lane & 7];
  const int b = __builtin_amdgcn_readlane(tv, 0), hk = __builtin_amdgcn_readlane(tv, 1);
  const int q0 = __builtin_amdgcn_readlane(tv, 2), q1 = __builtin_amdgcn_readlane(tv, 3);
  const int key0 = __builtin_amdgcn_readlane(tv, 4);
  const int slot0 = __builtin_amdgcn_readlane(tv, 6), nchunk = __builtin_amdgcn_readlane(tv, 7);
  const int pv = lane == 0   ? p.kv_indptr[b]
                 : lane == 1 ? p.kv_indptr[b + 1]
                 : lane == 2 ? p.last_page_len[b]
                 : lane == 3 ? p.qo_indptr[b]
                             : p.qo_indptr[b + 1];
  const int pbeg = __builtin_amdgcn_readlane(pv, 0);
  const int npages_req = __builtin_amdgcn_readlane(pv, 1) - pbeg;
  const int kv_len = npages_req > 0 ? (npages_req - 1) * 16 + __builtin_amdgcn_readlane(pv, 2) : 0;
  const int qo_beg = __builtin_amdgcn_readlane(pv, 3);
  const int qo_len = __builtin_amdgcn_readlane(pv, 4) - qo_beg;
  const int key1 = min(__builtin_amdgcn_readlane(tv, 5), kv_len);
  const int rows = q1 - q0;
  const int Hq = p.num_qo_heads;
  const int head = hk * G + wave;

  // this lane's query column: row q0 + jq, absolute position qpos
  const bool qvalid = jq < rows;
  const int qpos = p.causal ? kv_len - qo_len + (q0 + jq - qo_beg) : 0x7fffffff;
  const int qpos_min = p.causal ? kv_len - qo_len + (q0 - qo_beg) : 0x7fffffff;

  // Q^T operand: 8 blocks of 16 dims, this lane supplies dims 16 kb + 8 h .. +8
  u32x4 qf[8];
  {
    const uint16_t* qp = p.q + ((int64_t)(q0 + jq) * Hq + head) * 128 + 8 * h;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      qf[kb] = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * kb) : u32x4{0, 0, 0, 0};
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = kNegInf, l = 0.f;
  const float scale = p.scale_log2;

  const int nblocks = key1 > key0 ? (key1 - key0 + kBlockKeys - 1) / kBlockKeys : 0;
  const int first_page = key0 >> 4;

  // --- K/V staging ---------------------------------------------------------
  // task tk: key group kg = tk >> 4 (keys 4kg..4kg+3), dim group dg = tk & 15
  auto page_of = [&](int blk, int tk) -> int {
    const int pg = first_page + blk * (kBlockKeys / 16) + ((tk >> 4) >> 2);
    return pg < npages_req ? p.kv_indices[pbeg + pg] : 0;
  };
  auto fetch = [&](Stage<TPT>& st, int blk, const int (&pid)[TPT]) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tk = tid + i * GE::kThreads;
      const bool active = tk < GE::kTasks;
      const int kg = (tk >> 4) & 15, dg = tk & 15;
      const int kbase = key0 + blk * kBlockKeys + 4 * kg;
      const int64_t pbase = (int64_t)pid[i] * p.page_stride + (int64_t)hk * p.head_stride + 8 * dg;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = kbase + kk;
        const int64_t off = pbase + (int64_t)(key & 15) * p.token_stride;
        if (active && key < key1) {
          st.k[i][kk] = *reinterpret_cast<const u32x4*>(p.k + off);
          st.v[i][kk] = *reinterpret_cast<const u32x4*>(p.v + off);
        } else {
          st.k[i][kk] = u32x4{0, 0, 0, 0};
          st.v[i][kk] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto store = [&](const Stage<TPT>& st, int buf) {
    uint16_t* sk = smem + buf * kBufElems;
    uint16_t* sv = sk + kKElems;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tk = tid + i * GE::kThreads;
      if (tk >= GE::kTasks) continue;
      const int kg = (tk >> 4) & 15, dg = tk & 15;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        *reinterpret_cast<u32x4*>(sk + (4 * kg + kk) * kKStride + 8 * dg) = st.k[i][kk];
      // transpose 4 keys x 8 dims -> 8 dims x 4 keys
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = st.v[i][0][w], a1 = st.v[i][1][w], a2 = st.v[i][2][w], a3 = st.v[i][3][w];
        const u32x2 lo = {__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                          __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
        const u32x2 hi = {__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                          __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
        const int d = 8 * dg + 2 * w;
        *reinterpret_cast<u32x2*>(sv + d * kVStride + 4 * kg) = lo;
        *reinterpret_cast<u32x2*>(sv + (d + 1) * kVStride + 4 * kg) = hi;
      }
    }
  };

  Stage<TPT> st;
  int pid_cur[TPT], pid_next[TPT];
  if (nblocks > 0) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) pid_cur[i] = page_of(0, tid + i * GE::kThreads);
    fetch(st, 0, pid_cur);
    store(st, 0);
  }
  __syncthreads();

  for (int blk = 0; blk < nblocks; ++blk) {
    const int buf = blk & 1;
    const bool more = blk + 1 < nblocks;
    if (more) {
#pragma unroll
      for (int i = 0; i < TPT; ++i) pid_next[i] = page_of(blk + 1, tid + i * GE::kThreads);
      fetch(st, blk + 1, pid_next);
    }
    const uint16_t* sk = smem + buf * kBufElems;
    const uint16_t* sv = sk + kKElems;
    const int kb0 = key0 + blk * kBlockKeys;

    // S^T = K Q^T for two tiles of 32 keys
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
      const uint16_t* krow = sk + (32 * kt + jq) * kKStride + 8 * h;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        s[kt] = Mfma<DT>::run(*reinterpret_cast<const u32x4*>(krow + 16 * kb), qf[kb], s[kt]);
    }
    // scale, mask, block max: register r of tile kt holds key 32 kt + 8 (r/4) + 4 h + r%4
    const bool need_mask = kb0 + kBlockKeys > key1 || kb0 + kBlockKeys - 1 > qpos_min;
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kt][r] * scale;
        if (need_mask) {
          const int key = kb0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= key1 || key > qpos) x = kNegInf;
        }
        s[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float mn = fmaxf(m, mx);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(s[kt][r] - ms);
        s[kt][r] = e;
        rs += e;
      }
    rs += xor_shfl(rs, 32);
    l = l * alpha + rs;
    m = mn;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // O^T += V^T P^T over 4 key blocks of 16 (keys permuted alike in both operands)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        u32x4 pb;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pb[e] = Elt<DT>::pack(s[kt][8 * kh + 2 * e], s[kt][8 * kh + 2 * e + 1]);
        const int kofs = 32 * kt + 16 * kh + 4 * h;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint16_t* vrow = sv + (32 * db + jq) * kVStride + kofs;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          o[db] = Mfma<DT>::run(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, o[db]);
        }
      }

    if (more) {
      store(st, buf ^ 1);
#pragma unroll
      for (int i = 0; i < TPT; ++i) pid_cur[i] = pid_next[i];
    }
    __syncthreads();
  }

  // --- epilogue --------------------------------------------------------------
  // register r of o[db] holds dim 32 db + 8 (r/4) + 4 h + r%4 of query jq
  const bool live = l > 0.f;
  const float inv = live ? 1.f / l : 0.f;
  const float lse2 = live ? m + fast_log2(l) : kNegInf;
  if (slot0 < 0) {
    if (qvalid) {
      uint16_t* op = p.out + ((int64_t)(q0 + jq) * Hq + head) * 128;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const u32x2 w = {Elt<DT>::pack(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv),
                           Elt<DT>::pack(o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + 32 * db + 8 * rg + 4 * h) = w;
        }
      if (h == 0 && p.lse) p.lse[(int64_t)(q0 + jq) * Hq + head] = lse2 * kLn2;
    }
    return;
  }

  // split tile: publish the partial state of every row with device-coherent stores
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(p);
  if (qvalid) {
    const int64_t sh = (int64_t)(slot0 + jq) * G + wave;
    const uint32_t ob = (uint32_t)sh * 512u;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const u32x4 w = {__float_as_uint(o[db][4 * rg] * inv), __float_as_uint(o[db][4 * rg + 1] * inv),
                         __float_as_uint(o[db][4 * rg + 2] * inv),
                         __float_as_uint(o[db][4 * rg + 3] * inv)};
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, ob + 4u * (32 * db + 8 * rg + 4 * h), 0, kCoherent);
      }
    if (h == 0)
      __hip_atomic_store(p.part_lse + sh, lse2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  const int chunk = key0 / (p.header[5] * 16);
  const int base = slot0 - chunk * rows;
  if (tid == 0) {
    const int prev =
        __hip_atomic_fetch_add(p.counters + base, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == nchunk - 1;
    if (last) p.counters[base] = 0;
    s_flag = last;
  }
  __syncthreads();
  if (!s_flag || !qvalid) return;

  // last workgroup of the split: merge the chunks of every row; lane (h, jq)
  // owns dims 64 h .. 64 h + 63 of row q0 + jq
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;
  float gm = kNegInf, gl = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const int64_t sh = (int64_t)(base + c * rows + jq) * G + wave;
    const float s2 = __hip_atomic_load(p.part_lse + sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ob = (uint32_t)sh * 512u + 256u * h;
    u32x4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ob + 16 * i, 0, kCoherent);
    const float mn = fmaxf(gm, s2);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float f = fast_exp2(gm - ms);
    const float w = fast_exp2(s2 - ms);
    gl = gl * f + w;
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = acc[i] * f + w * __uint_as_float(raw[i >> 2][i & 3]);
    gm = mn;
  }
  const bool glive = gl > 0.f;
  const float ginv = glive ? 1.f / gl : 0.f;
  uint16_t* op = p.out + ((int64_t)(q0 + jq) * Hq + head) * 128 + 64 * h;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = Elt<DT>::pack(acc[8 * i + 2 * e] * ginv, acc[8 * i + 2 * e + 1] * ginv);
    *reinterpret_cast<u32x4*>(op + 8 * i) = w;
  }
  if (h == 0 && p.lse)
    p.lse[(int64_t)(q0 + jq) * Hq + head] = glive ? (gm + fast_log2(gl)) * kLn2 : kNegInf;
}

template <int DT>
hipError_t launch_dt(const AttnParams& p, int group, int grid, hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL((append_kernel<DT, 1>), dim3(grid), dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL((append_kernel<DT, 2>), dim3(grid), dim3(128), 0, s, p); break;
    case 4: hipLaunchKernelGGL((append_kernel<DT, 4>), dim3(grid), dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((append_kernel<DT, 8>), dim3(grid), dim3(512), 0, s, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AttnParams& p, int dtype, int group, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  return dtype == FA_BF16 ? launch_dt<FA_BF16>(p, group, max_tiles, s)
                          : launch_dt<FA_F16>(p, group, max_tiles, s);
}

}  // namespace pkfa
