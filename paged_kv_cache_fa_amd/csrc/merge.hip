// Log-sum-exp merge of attention states on gfx950.
//
// [Guide] "FlashInfer: GPU Kernels for LLM Inference (2026 Guide)", section
// "Cascade attention for shared prefixes": states computed over disjoint key
// sets are combined by merge_state / merge_states. For states (v_c, s_c):
//   s = log(sum_c exp(s_c)),   v = sum_c exp(s_c - s) v_c,
// evaluated here as a running (online) merge in fp32 so any number of states
// streams through registers; a state with s = -inf contributes nothing and
// all-empty input gives (0, -inf).
//
// These kernels are HBM-bound elementwise passes: each thread owns 8
// consecutive elements of one (row, head), loads 16/32 bytes per state and
// writes its 8 outputs once.
#include "device_common.h"
#include "kernels.h"

namespace pkfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBatch = 8;  // states of one (row, head) whose loads are in flight together

// 8 consecutive values of type DT (FA_F32 or a 16-bit type) <-> fp32.
template <int DT>
struct Vec8 {
  __device__ __forceinline__ static void load(const void* base, int64_t idx, float (&x)[8]) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = Elt<DT>::lo(u[i]);
      x[2 * i + 1] = Elt<DT>::hi(u[i]);
    }
  }
  __device__ __forceinline__ static void store(void* base, int64_t idx, const float (&x)[8]) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = Elt<DT>::pack(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx) = u;
  }
};

template <>
struct Vec8<FA_F32> {
  __device__ __forceinline__ static void load(const void* base, int64_t idx, float (&x)[8]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ static void store(void* base, int64_t idx, const float (&x)[8]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
    p[0] = make_float4(x[0], x[1], x[2], x[3]);
    p[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
};

// Running merge state in log2 units. A state with s = -inf leaves it as it
// is (f = 1, nothing added, whatever its v holds); the update has no branch,
// so the loads of several states can be in flight before the first is added.
struct Online {
  float m = kNegInf, sum = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void add(float s2, const float (&v)[8]) {
    const bool live = s2 != kNegInf;
    const float mn = live ? fmaxf(m, s2) : m;
    const float ms = mn == kNegInf ? 0.f : mn;
    const float f = fast_exp2(m - ms);  // m = -inf -> 0
    const float w = live ? fast_exp2(s2 - ms) : 0.f;
    sum = sum * f + w;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] * f + (live ? w * v[i] : 0.f);
    m = mn;
  }
  __device__ __forceinline__ void finish(float (&out)[8], float& lse2) const {
    const bool live = sum > 0.f;
    const float inv = live ? 1.f / sum : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = acc[i] * inv;
    lse2 = live ? m + fast_log2(sum) : kNegInf;
  }
};

template <int DT>
__global__ __launch_bounds__(256) void merge_state_kernel(const void* va, const float* sa,
                                                          const void* vb, const float* sb,
                                                          void* vo, float* so, int64_t n, int heads,
                                                          int head_dim) {
  const int chunks = head_dim / 8;
  const int64_t total = n * heads * chunks;
  for (int64_t it = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; it < total;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rh = it / chunks;
    const int64_t idx = rh * head_dim + (it % chunks) * 8;
    float a[8], b[8];
    Vec8<DT>::load(va, idx, a);
    Vec8<DT>::load(vb, idx, b);
    const float s_a = sa[rh], s_b = sb[rh];
    Online st;
    st.add(s_a * kLog2e, a);
    st.add(s_b * kLog2e, b);
    float o[8], lse2;
    st.finish(o, lse2);
    Vec8<DT>::store(vo, idx, o);
    if (so && (it % chunks) == 0) so[rh] = lse2 * kLn2;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void merge_states_kernel(const void* v, const float* s, int64_t n,
                                                           int k, int heads, int head_dim, void* vo,
                                                           float* so) {
  const int chunks = head_dim / 8;
  const int64_t total = n * heads * chunks;
  for (int64_t it = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; it < total;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rh = it / chunks;  // row * heads + head
    const int64_t row = rh / heads, h = rh % heads;
    const int d = (int)(it % chunks) * 8;
    Online st;
    // up to kBatch states requested at once, then merged in order
    for (int c0 = 0; c0 < k; c0 += kBatch) {
      float s2[kBatch], x[kBatch][8];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (c0 + i < k) {
          const int64_t sh = (row * k + c0 + i) * heads + h;
          Vec8<DT>::load(v, sh * head_dim + d, x[i]);
          s2[i] = s[sh] * kLog2e;
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (c0 + i < k) st.add(s2[i], x[i]);
    }
    float o[8], lse2;
    st.finish(o, lse2);
    Vec8<DT>::store(vo, rh * head_dim + d, o);
    if (so && d == 0) so[rh] = lse2 * kLn2;
  }
}

// One thread per (row, head, 8 dims): the prefix state is either the merge of
// the prefix plan's chunk partials (all prefix q tiles split alike: merge
// entry (q tile, kv head) = qt * num_kv_heads + hk) or its direct output.
template <int DT>
__global__ __launch_bounds__(256) void cascade_merge_kernel(
    const int32_t* header, const int32_t* merge, const float* part_o, const float* part_lse,
    const void* po, const float* pls, const void* so, const float* sls, void* vo, float* lo,
    const int32_t* suffix_header, int heads, int group, int num_kv_heads, int qo_tile) {
  const int num_merge = header[1];
  const int64_t n = suffix_header[2];  // the suffix plan's batch (graph replays follow re-plans)
  const int64_t total = n * heads * 16;
  for (int64_t it = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; it < total;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rh = it >> 4;
    const int64_t r = rh / heads;
    const int h = (int)(rh % heads);
    const int d = (int)(it & 15) * 8;
    Online st;
    // the suffix state is requested first; the prefix chunks then come in
    // batches of kBatch, all of a batch in flight at once
    float xs[8];
    Vec8<DT>::load(so, rh * 128 + d, xs);
    const float ss = sls[rh] * kLog2e;
    if (num_merge > 0) {
      const int hk = h / group, g = h % group;
      // one 16-byte load of the merge entry {q0, -, base, C}
      const u32x4 e = *reinterpret_cast<const u32x4*>(merge + ((int64_t)(r / qo_tile) * num_kv_heads + hk) * 4);
      const int q0 = (int)e[0], base = (int)e[2], C = (int)e[3];
      const int rows = (int)min((int64_t)qo_tile, n - q0);
      for (int c0 = 0; c0 < C; c0 += kBatch) {
        float s2[kBatch], x[kBatch][8];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          if (c0 + i < C) {
            const int64_t sh = (int64_t)(base + (c0 + i) * rows + (r - q0)) * group + g;
            Vec8<FA_F32>::load(part_o, sh * 128 + d, x[i]);
            s2[i] = part_lse[sh];
          }
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (c0 + i < C) st.add(s2[i], x[i]);
      }
    } else {
      float x[8];
      Vec8<DT>::load(po, rh * 128 + d, x);
      st.add(pls[rh] * kLog2e, x);
    }
    st.add(ss, xs);
    float o[8], lse2;
    st.finish(o, lse2);
    Vec8<DT>::store(vo, rh * 128 + d, o);
    if (lo && d == 0) lo[rh] = lse2 * kLn2;
  }
}

int grid_for(int64_t total) {
  const int64_t blocks = (total + 255) / 256;
  return (int)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                              void* vo, float* so, int64_t n, int heads, int head_dim, int dtype,
                              hipStream_t s) {
  const int64_t total = n * heads * (head_dim / 8);
  if (total <= 0) return hipSuccess;
  const int grid = grid_for(total);
  switch (dtype) {
    case FA_BF16:
      hipLaunchKernelGGL(merge_state_kernel<FA_BF16>, dim3(grid), dim3(256), 0, s, va, sa, vb, sb,
                         vo, so, n, heads, head_dim);
      break;
    case FA_F16:
      hipLaunchKernelGGL(merge_state_kernel<FA_F16>, dim3(grid), dim3(256), 0, s, va, sa, vb, sb,
                         vo, so, n, heads, head_dim);
      break;
    default:
      hipLaunchKernelGGL(merge_state_kernel<FA_F32>, dim3(grid), dim3(256), 0, s, va, sa, vb, sb,
                         vo, so, n, heads, head_dim);
  }
  return hipGetLastError();
}

hipError_t launch_merge_states(const void* v, const float* sv, int64_t n, int k, int heads,
                               int head_dim, int dtype, void* vo, float* so, hipStream_t s) {
  const int64_t total = n * heads * (head_dim / 8);
  if (total <= 0) return hipSuccess;
  const int grid = grid_for(total);
  switch (dtype) {
    case FA_BF16:
      hipLaunchKernelGGL(merge_states_kernel<FA_BF16>, dim3(grid), dim3(256), 0, s, v, sv, n, k,
                         heads, head_dim, vo, so);
      break;
    case FA_F16:
      hipLaunchKernelGGL(merge_states_kernel<FA_F16>, dim3(grid), dim3(256), 0, s, v, sv, n, k,
                         heads, head_dim, vo, so);
      break;
    default:
      hipLaunchKernelGGL(merge_states_kernel<FA_F32>, dim3(grid), dim3(256), 0, s, v, sv, n, k,
                         heads, head_dim, vo, so);
  }
  return hipGetLastError();
}

hipError_t launch_cascade_merge(const int32_t* prefix_header, const int32_t* prefix_merge,
                                const float* part_o, const float* part_lse, const void* prefix_out,
                                const float* prefix_lse, const void* suffix_out,
                                const float* suffix_lse, void* out, float* lse,
                                const int32_t* suffix_header, int64_t max_n, int heads, int group,
                                int num_kv_heads, int qo_tile, int dtype, hipStream_t s) {
  const int64_t total = max_n * heads * 16;
  if (total <= 0) return hipSuccess;
  const int grid = grid_for(total);
  if (dtype == FA_BF16)
    hipLaunchKernelGGL(cascade_merge_kernel<FA_BF16>, dim3(grid), dim3(256), 0, s, prefix_header,
                       prefix_merge, part_o, part_lse, prefix_out, prefix_lse, suffix_out,
                       suffix_lse, out, lse, suffix_header, heads, group, num_kv_heads, qo_tile);
  else
    hipLaunchKernelGGL(cascade_merge_kernel<FA_F16>, dim3(grid), dim3(256), 0, s, prefix_header,
                       prefix_merge, part_o, part_lse, prefix_out, prefix_lse, suffix_out,
                       suffix_lse, out, lse, suffix_header, heads, group, num_kv_heads, qo_tile);
  return hipGetLastError();
}

}  // namespace pkfa
