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
//  * tiles come in 8 bins, one per XCD: the planner deals each (request, kv
//    head) group to one bin, so the q tiles that read the same keys run side
//    by side on one XCD and share its L2;
//  * one 512-thread workgroup (8 waves, 2 per SIMD) per tile {request, kv
//    head, up to 256/G query positions, key chunk}. The tile's 256 query
//    columns are the G heads of the kv head's group x 256/G positions (GQA
//    packing): every K/V block staged in LDS feeds all of them, so a block is
//    fetched once per 256 columns. Wave w owns columns 32w .. 32w+31;
//  * blocks of 64 keys: waves 0-3 stage K and waves 4-7 stage V (one of each
//    per SIMD); each of their threads fetches 16 bytes of 4 token rows (one
//    row from each of the block's 4 pages, so every load's page is uniform
//    across the wave) through a per-page buffer resource that ends at the
//    last valid token: keys past the end read as zero. A block's registers
//    are written to LDS at the top of the next iteration (four LDS stages,
//    so a block is requested two iterations before its scores are needed),
//    one barrier per block;
//  * inside a block, key k sits in LDS slot 4 (k mod 16) + k / 16, so one
//    thread's 4 rows form 4 consecutive slots: V is stored transposed
//    (dim-major, 4 slots per 8-byte store) without any exchange. The
//    contraction over keys is order-free, and the mask maps slots back to
//    keys. Each lane's PV operand is one 16-byte LDS read, and V^T rows are
//    XOR-swizzled so that both the transposing stores and the operand reads
//    hit distinct banks;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: a lane owns one query column and 16 of
//    every 32 slots, so the online-softmax max / sum need one exchange
//    (lanes l and l^32) and the output rescale is lane-local. The reference
//    max only moves (with a rescale) when a wave-wide vote sees a score more
//    than 2^8 above it, so most blocks skip the rescale;
//  * O^T += V^T P^T reuses the score registers (rounded to the input type) as
//    the B operand;
//  * blocks that need no mask (all keys valid and below the first row's
//    causal limit) skip the masking step;
//  * a chunked (split) tile writes fp32 partial states; the last workgroup of
//    the split (agent-scope counter, reset by that workgroup) merges them by
//    log-sum-exp, unless the caller defers the merge to a later kernel (the
//    cascade combine, which merges prefix chunks and suffix in one pass).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pkfa {
namespace app {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Workgroups of WAVES waves (a template parameter): 8 in the append kernel
// and the wide one-launch form (one workgroup per CU, 2 waves per SIMD), 4 in
// the shared one-launch form, whose append workgroups share each CU with
// decode workgroups. A workgroup covers 32 WAVES query columns.
constexpr int kBlockKeys = 64;
constexpr int kKStride = 136;  // 16-bit elements per K slot row in LDS (128 dims + 8 pad)
constexpr int kKElems = kBlockKeys * kKStride;
constexpr int kCoherent = 16;          // cache policy sc1: device-coherent access
constexpr float kRescaleSlack = 8.0f;  // log2 units: probabilities stay <= 2^8

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

// V^T layout. Row d holds the 64 slots of dim d as 8 units of 16 bytes. The
// MFMA A operand of a lane of half h for slot tile kt, group kh is the 8
// slots {32 kt + 16 kh + 4 h + e, 32 kt + 16 kh + 8 + 4 h + e : e < 4}, i.e.
// the 4-slot groups tr and tr + 2 (tr = 8 kt + 4 kh + h): they share the
// 16-byte unit c = 4 kt + 2 kh + h (first and second half). Unit c of row d
// sits at position c ^ swz(d) of a row of kRow elements; swz depends on
// d mod 32 only (the 4 dim tiles of a lane differ by immediate offsets).
// Rows are 64 slots (128 bytes) with no padding, so four LDS stages of K and
// V^T fit beside each other. swz is linear over the bits of d mod 32:
// swz(d) = 2 d0 ^ 3 d1 ^ 5 d2 ^ 7 d3 ^ 2 d4 (d_i the bits of d). Of the
// swizzles measured on the LDS counters (SQ_LDS_BANK_CONFLICT and
// SQ_LDS_IDX_ACTIVE per instruction, the exact store and read patterns of
// this kernel, row strides of 128 to 192 bytes), it is one of those with no
// conflict cycles on the operand reads (3.9 LDS cycles per instruction,
// against 7.7 with conflicts) and the fewest cycles on the transposing
// 8-byte stores (4.0 per instruction, against 5.3 to 16).
struct VLayout {
  static constexpr int kRow = 64;
  static constexpr int kElems = 128 * kRow;
  static constexpr int kBufElems = kKElems + kElems;  // one LDS stage: K slots + V^T
  __device__ __forceinline__ static int swz(int d) {
    return ((d & 1) * 2) ^ (((d >> 1) & 1) * 3) ^ (((d >> 2) & 1) * 5) ^ (((d >> 3) & 1) * 7) ^
           (((d >> 4) & 1) * 2);
  }
  // swz(8 dg + 2 w + hi) = swz_base(dg) ^ swz_step(w, hi) for w < 4, hi < 2
  __device__ __forceinline__ static int swz_base(int dg) {
    return ((dg & 1) * 7) ^ (((dg >> 1) & 1) * 2);
  }
  __device__ __forceinline__ static constexpr int swz_step(int w, int hi) {
    return ((w & 1) * 3) ^ (((w >> 1) & 1) * 5) ^ (hi * 2);
  }
};

// Key (0..63 within the block) held in register r of score tile kt by a lane
// of half h: slot 32 kt + 8 (r / 4) + 4 h + r % 4, key = slot / 4 + 16 (slot % 4),
// i.e. reg_key0(kt, r) + h (a compile-time constant plus the lane half).
__device__ __forceinline__ constexpr int reg_key0(int kt, int r) {
  return 8 * kt + 2 * (r >> 2) + 16 * (r & 3);
}

// Max / sum of a value over the lane pair (l, l ^ 32), in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// STAGES: LDS buffers of the block loop, 4 (software pipeline: the scores of
// block j+1 beside the softmax of block j, stores a block ahead) or 2 (one
// block at a time, for a workgroup that shares its CU). A tile's rows must fit the workgroup's
// 32 WAVES / G positions (the planner's qo_tile).
template <int DT, int G, int STAGES, int WAVES>
__device__ __forceinline__ void append_tile(const AttnParams& p, int tile_id, uint16_t* smem,
                                            int& s_flag) {
  constexpr int kCols = 32 * WAVES;  // query columns of the workgroup
  constexpr int PT = kCols / G;      // query positions per tile
  using VL = VLayout;
  constexpr int kBufElems = VL::kBufElems;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int jq = lane & 31, h = lane >> 5;

  // tile fields, made wave-uniform
  const int32_t* t = p.tiles + tile_id * 8;
  const int tv = t[lane & 7];
  const int b = __builtin_amdgcn_readlane(tv, 0), hk = __builtin_amdgcn_readlane(tv, 1);
  const int q0 = __builtin_amdgcn_readlane(tv, 2), q1 = __builtin_amdgcn_readlane(tv, 3);
  const int key0 = __builtin_amdgcn_readlane(tv, 4);
  const int slot0 = __builtin_amdgcn_readlane(tv, 6), nchunk = __builtin_amdgcn_readlane(tv, 7);
  // paged: page offsets and last_page_len; ragged KV: the request's first and
  // end rows (a page is 16 rows from row kv_offsets[b] + 16 p)
  const bool ragged = p.kv_offsets != nullptr;
  const int32_t* kvp = ragged ? p.kv_offsets : p.kv_indptr;
  const int pv = lane == 0   ? kvp[b]
                 : lane == 1 ? kvp[b + 1]
                 : lane == 2 ? (ragged ? 0 : p.last_page_len[b])
                 : lane == 3 ? p.qo_indptr[b]
                             : p.qo_indptr[b + 1];
  const int pbeg = __builtin_amdgcn_readlane(pv, 0);
  const int span = __builtin_amdgcn_readlane(pv, 1) - pbeg;
  const int kv_len =
      ragged ? span : (span > 0 ? (span - 1) * 16 + __builtin_amdgcn_readlane(pv, 2) : 0);
  const int npages_req = ragged ? (span + 15) >> 4 : span;
  const int qo_beg = __builtin_amdgcn_readlane(pv, 3);
  const int qo_len = __builtin_amdgcn_readlane(pv, 4) - qo_beg;
  const int key1 = min(__builtin_amdgcn_readlane(tv, 5), kv_len);
  const int rows = q1 - q0;
  const int Hq = p.num_qo_heads;

  // this lane's query column: head hk*G + g, row q0 + pos
  const int col = 32 * wave + jq;
  const int g = col / PT, pos = col % PT;
  const int head = hk * G + g;
  const bool qvalid = pos < rows;
  // the mask mode comes from the uploaded plan (header word 4), so a captured
  // launch follows a re-plan that switches it
  const bool causal = __builtin_amdgcn_readfirstlane(p.header[4]) != 0;
  const int qpos_min = causal ? kv_len - qo_len + (q0 - qo_beg) : 0x7fffffff;
  const int qpos = causal ? qpos_min + pos : 0x7fffffff;

  // Q^T operand: 8 blocks of 16 dims, this lane supplies dims 16 kb + 8 h .. +8
  u32x4 qf[8];
  {
    const uint16_t* qp = p.q + ((int64_t)(q0 + pos) * Hq + head) * 128 + 8 * h;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      qf[kb] = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * kb) : u32x4{0, 0, 0, 0};
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = kNegInf, l = 0.f;  // per column: reference max (log2 units), this lane's sum
  const float scale = p.scale_log2;

  const int nblocks = key1 > key0 ? (key1 - key0 + kBlockKeys - 1) / kBlockKeys : 0;
  const int first_page = key0 >> 4;  // chunks start on a page boundary

  // --- K/V staging: the first half of the waves stage K, the second half V
  // (a wave-uniform role; one of each per SIMD). The 256 (token row tr of each
  // of the block's 4 pages, 16-byte dim group dg) pairs of a role are dealt
  // to its 32 WAVES threads in kPasses passes: pair st (st bits [1:0] and
  // [5:4] give dg, bits [3:2] and [7:6] give tr) is thread st mod 32 WAVES,
  // pass st / (32 WAVES). A wave reads 4 whole token rows per load, and 16
  // lanes that store together cover 4 dg x 4 tr.
  constexpr int kRoleThreads = 32 * WAVES;
  constexpr int kPasses = 256 / kRoleThreads;
  const bool stage_v = wave >= WAVES / 2;
  const int st0 = tid % kRoleThreads;
  const int dg = (st0 & 3) | ((st0 >> 2) & 12);
  int trp[kPasses];
#pragma unroll
  for (int r = 0; r < kPasses; ++r) {
    const int st = st0 + r * kRoleThreads;
    trp[r] = ((st >> 2) & 3) | ((st >> 4) & 12);
  }
  const uint32_t row_bytes = (uint32_t)p.token_stride * 2u;
  const int64_t head_off = (int64_t)hk * p.head_stride;
  const uint16_t* src = stage_v ? p.v : p.k;
  u32x4 stg[4 * kPasses];
  int pid[4];
  // page ids of a block: lanes 0..3 load them (index clamped to the request's
  // last page: a block past the end fetches nothing, see nbytes below), and
  // every lane takes them as wave-uniform values (scalar buffer resources)
  auto load_pid_vec = [&](int blk) -> int {
    const int pg = max(min(first_page + blk * 4 + (lane & 3), npages_req - 1), 0);
    return ragged ? pbeg + 16 * pg : p.kv_indices[pbeg + pg];
  };
  auto take_pids = [&](int v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pid[i] = __builtin_amdgcn_readlane(v, i);
  };
  auto fetch = [&](int blk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kstart = key0 + blk * kBlockKeys + 16 * i;
      const int nbytes =
          __builtin_amdgcn_readfirstlane(min(max(key1 - kstart, 0), 16) * (int)row_bytes);
      const int64_t base = (int64_t)pid[i] * p.page_stride + head_off;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(src + base), 0, nbytes, 0x00020000);
#pragma unroll
      for (int r = 0; r < kPasses; ++r)
        stg[4 * r + i] = __builtin_amdgcn_raw_buffer_load_b128(
            rs, (uint32_t)trp[r] * row_bytes + 16u * dg, 0, 0);
    }
  };
  auto store = [&](int buf) {
    uint16_t* sk = smem + buf * kBufElems;
    uint16_t* sv = sk + kKElems;
    if (!stage_v) {
#pragma unroll
      for (int r = 0; r < kPasses; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(sk + (4 * trp[r] + i) * kKStride + 8 * dg) = stg[4 * r + i];
      return;
    }
    // Dims d = 8 dg + 2 w and d + 1 go to V^T rows d, d + 1: the thread's 4
    // slots 4 tr .. 4 tr + 3 are the first (tr bit 1 clear) or second half of
    // unit 2 (tr >> 2) + (tr & 1), at position unit ^ swz(row) (tr bit 1 is
    // the same in every pass). u and the row base are recomputed here on
    // every call (the empty asm hides that they do not change), so the
    // compiler does not keep 8 loop-invariant addresses live through the
    // block loop.
    int vbase = 2 * VL::kRow * 8 * dg + 8 * ((trp[0] >> 1) & 1);
    asm volatile("" : "+v"(vbase));
    char* sv8 = reinterpret_cast<char*>(sv) + vbase;
#pragma unroll
    for (int r = 0; r < kPasses; ++r) {
      int u = (2 * (trp[r] >> 2) + (trp[r] & 1)) ^ VL::swz_base(dg);
      asm volatile("" : "+v"(u));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = stg[4 * r][w], a1 = stg[4 * r + 1][w], a2 = stg[4 * r + 2][w],
                       a3 = stg[4 * r + 3][w];
        const u32x2 lo = {__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                          __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
        const u32x2 hi = {__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                          __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
        *reinterpret_cast<u32x2*>(sv8 + 2 * w * 2 * VL::kRow + 16 * (u ^ VL::swz_step(w, 0))) =
            lo;
        *reinterpret_cast<u32x2*>(sv8 + (2 * w + 1) * 2 * VL::kRow +
                                  16 * (u ^ VL::swz_step(w, 1))) = hi;
      }
    }
  };

  // S^T of one 64-key block from its LDS buffer (two 32-slot halves, each a
  // chain of 8 MFMAs over the 128 dims). The K operands are read from LDS
  // KPRE at a time ahead of their MFMAs, so a chain waits for LDS 8 / KPRE
  // times.
  constexpr int KPRE = 4;
  auto scores_half = [&](const uint16_t* sk, int kt, f32x16& s_out) {
    const uint16_t* krow = sk + (32 * kt + jq) * kKStride + 8 * h;
    f32x16 acc = {};
#pragma unroll
    for (int k4 = 0; k4 < 8; k4 += KPRE) {
      u32x4 ka[KPRE];
#pragma unroll
      for (int i = 0; i < KPRE; ++i) ka[i] = *reinterpret_cast<const u32x4*>(krow + 16 * (k4 + i));
#pragma unroll
      for (int i = 0; i < KPRE; ++i) acc = Mfma<DT>::run(ka[i], qf[k4 + i], acc);
    }
    s_out = acc;
  };

  // The online softmax of one block, in three steps that both loops run in
  // the same order (so they give the same bits): the mask, the row max with
  // the (lazy) rescale of the running state, and the probabilities with
  // O^T += V^T P^T.
  auto mask_block = [&](f32x16 (&s)[2], int blk) {
    const int kb0 = key0 + blk * kBlockKeys;
    if (kb0 + kBlockKeys > key1 || kb0 + kBlockKeys - 1 > qpos_min) {  // wave-uniform
      // last visible key of this column, in-block, less the lane half
      const int lim = min(key1 - 1, qpos) - kb0 - h;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kt][r] = reg_key0(kt, r) > lim ? kNegInf : s[kt][r];
    }
  };
  auto row_max = [&](const f32x16 (&s)[2]) {
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = pair_max(mx);
    const float mxs = mx * scale;
    const bool need = mxs > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m - mxs) : 1.f;
      m = need ? mxs : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
  };
  auto exp_pv = [&](const f32x16 (&s)[2], const uint16_t* sv) {
    const float ms = m == kNegInf ? 0.f : m;
    // probabilities, packed to the input type as the B operand of P V (the
    // row sum is kept in fp32: the LSE must not carry the operand rounding)
    u32x4 pb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kt][8 * kh + 2 * e], scale, -ms));
          const float p1 = fast_exp2(__builtin_fmaf(s[kt][8 * kh + 2 * e + 1], scale, -ms));
          l += p0 + p1;
          pb[kt][kh][e] = Elt<DT>::pack(p0, p1);
        }
    // O^T += V^T P^T over the block's 4 slot groups of 16
    const uint16_t* vrow = sv + jq * VL::kRow;
    const int sw = VL::swz(jq);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int unit = (4 * kt + 2 * kh + h) ^ sw;
        u32x4 va[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          va[db] = *reinterpret_cast<const u32x4*>(vrow + 32 * db * VL::kRow + 8 * unit);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = Mfma<DT>::run(va[db], pb[kt][kh], o[db]);
      }
  };

  if constexpr (STAGES == 2) {
    // Two LDS buffers (the one-launch cascade / mixed-batch kernel, where an
    // append workgroup shares its CU with decode workers): block blk is
    // computed from buffer blk mod 2 while block blk+1 is in flight into
    // registers and the page ids of block blk+2 are loaded; one barrier per
    // block. The last iteration stages one block past the end (zero-size
    // buffer resources: nothing is read, zeros are stored).
    if (nblocks > 0) {
      take_pids(load_pid_vec(0));
      fetch(0);
      store(0);
      take_pids(load_pid_vec(1));
    }
    __syncthreads();
    for (int blk = 0; blk < nblocks; ++blk) {
      const int buf = blk & 1;
      const int pv = load_pid_vec(blk + 2);
      fetch(blk + 1);
      const uint16_t* sk = smem + buf * kBufElems;
      f32x16 sc[2];
      scores_half(sk, 0, sc[0]);
      scores_half(sk, 1, sc[1]);
      mask_block(sc, blk);
      row_max(sc);
      exp_pv(sc, sk + kKElems);
      store(buf ^ 1);
      take_pids(pv);
      __syncthreads();
    }
  } else {
    static_assert(STAGES == 4, "the block loop runs 2 or 4 LDS stages");
    // Software pipeline over four LDS buffers: block j is in buffer j mod 4.
    // Iteration j first stores block j+2 (requested at the top of iteration
    // j-1, so its loads have landed) into buffer (j+2) mod 4, which last held
    // block j-2 (read by every wave before the barrier that ended iteration
    // j-2), and requests block j+3 into the staging registers (its page ids
    // were loaded an iteration earlier). Then it runs block j's softmax and
    // P V beside block j+1's scores. The stores complete while the iteration
    // computes, away from the barrier that ends it, which publishes them.
    // Blocks past the end have zero-size buffer resources: they read nothing
    // and stage zeros, and their scores are never used.
    auto buf_of = [&](int j) { return smem + (j & 3) * kBufElems; };
    f32x16 sa[2], sb[2];
    if (nblocks > 0) {
      take_pids(load_pid_vec(0));
      fetch(0);
      store(0);
      take_pids(load_pid_vec(1));
      fetch(1);
      store(1);
      take_pids(load_pid_vec(2));
      fetch(2);
      take_pids(load_pid_vec(3));
    }
    __syncthreads();
    if (nblocks > 0) {
      scores_half(buf_of(0), 0, sa[0]);
      scores_half(buf_of(0), 1, sa[1]);
    }
    auto iteration = [&](int j, f32x16 (&s)[2], f32x16 (&s_next)[2]) {
      store((j + 2) & 3);
      const int pv = load_pid_vec(j + 4);
      fetch(j + 3);
      // block j's softmax and P V; block j+1's scores issued beside it:
      // half 0 before the row max, half 1 before the exponentials
      const uint16_t* sk_next = buf_of(j + 1);
      mask_block(s, j);
      scores_half(sk_next, 0, s_next[0]);
      row_max(s);
      scores_half(sk_next, 1, s_next[1]);
      exp_pv(s, buf_of(j) + kKElems);
      take_pids(pv);
      __syncthreads();
    };
    for (int j = 0; j < nblocks; j += 2) {
      iteration(j, sa, sb);
      if (j + 1 < nblocks) iteration(j + 1, sb, sa);
    }
  }

  // --- epilogue --------------------------------------------------------------
  // register r of o[db] holds dim 32 db + 8 (r/4) + 4 h + r%4 of this column;
  // each lane summed the probabilities of its own slots
  l = pair_sum(l);
  const bool live = l > 0.f;
  const float inv = live ? 1.f / l : 0.f;
  const float lse2 = live ? m + fast_log2(l) : kNegInf;
  if (slot0 < 0) {
    if (qvalid) {
      uint16_t* op = p.out + ((int64_t)(q0 + pos) * Hq + head) * 128;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const u32x2 w = {Elt<DT>::pack(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv),
                           Elt<DT>::pack(o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + 32 * db + 8 * rg + 4 * h) = w;
        }
      if (h == 0 && p.lse) p.lse[(int64_t)(q0 + pos) * Hq + head] = lse2 * kLn2;
    }
    return;
  }

  // split tile: publish the partial state of every column with device-coherent stores
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(p);
  if (qvalid) {
    const int64_t sh = (int64_t)(slot0 + pos) * G + g;
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
  if (p.defer_merge) return;  // a later kernel combines the partial states
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
  if (!s_flag) return;

  // last workgroup of the split: merge the chunks. The chunk-c states of this
  // tile are one run of rows G entries (entry pos G + g) of 512 bytes from
  // entry (base + c rows) G. First each entry's max and sum over the chunks
  // (thread = entry), then the weighted sum with the weights known, a wave
  // reading 2 whole entries per load: thread tid takes 16-byte unit tid mod 32
  // of entries tid / 32 + 2 WAVES r, r < 16.
  const int nent = rows * G;
  float* s_max = reinterpret_cast<float*>(smem);
  float* s_inv = s_max + kCols;
  if (tid < nent) {
    float mx = kNegInf, sum = 0.f;
#pragma unroll 1
    for (int c0 = 0; c0 < nchunk; c0 += 8) {
      float s2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = min(c0 + i, nchunk - 1);
        s2[i] = __hip_atomic_load(p.part_lse + (int64_t)(base + c * rows) * G + tid,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool live = c0 + i < nchunk && s2[i] != kNegInf;
        const float mn = live ? fmaxf(mx, s2[i]) : mx;
        const float ms = mn == kNegInf ? 0.f : mn;
        sum = sum * fast_exp2(mx - ms) + (live ? fast_exp2(s2[i] - ms) : 0.f);
        mx = mn;
      }
    }
    const bool live = sum > 0.f;
    s_max[tid] = mx == kNegInf ? 0.f : mx;
    s_inv[tid] = live ? 1.f / sum : 0.f;
    if (p.lse)
      p.lse[(int64_t)(q0 + tid / G) * Hq + hk * G + tid % G] =
          live ? (mx + fast_log2(sum)) * kLn2 : kNegInf;
  }
  __syncthreads();

  constexpr int kStep = 2 * WAVES;  // entries per load
  const int unit = tid & 31, e0 = tid >> 5;
  const __amdgpu_buffer_rsrc_t rl =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.part_lse, 0, 0x7fffffff, 0x00020000);
  // lane 2 r + hh (and 32 + 2 r + hh) fetches the weight of the wave's entry
  // 2 wave + hh + kStep r; round r reads it from there
  const int el = min(2 * wave + (lane & 1) + kStep * ((lane & 31) >> 1), nent - 1);
  const float mx_l = s_max[el], inv_l = s_inv[el];
  float acc[16][4];
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.f;
#pragma unroll 1
  for (int c = 0; c < nchunk; ++c) {
    const uint32_t ebase = (uint32_t)((base + c * rows) * G);  // wave-uniform
    u32x4 raw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t e = (uint32_t)min(e0 + kStep * r, nent - 1);
      raw[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, e * 512u + 16u * unit, ebase * 512u, kCoherent);
    }
    const float s2 = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)el * 4u, ebase * 4u, kCoherent));
    const float w_l = fast_exp2(s2 - mx_l) * inv_l;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float w = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (2 * r + h), __float_as_int(w_l)));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][i] += w * __uint_as_float(raw[r][i]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int e = e0 + kStep * r;
    if (e < nent) {
      uint16_t* op = p.out + ((int64_t)(q0 + e / G) * Hq + hk * G + e % G) * 128 + 4 * unit;
      *reinterpret_cast<u32x2*>(op) = u32x2{Elt<DT>::pack(acc[r][0], acc[r][1]),
                                            Elt<DT>::pack(acc[r][2], acc[r][3])};
    }
  }
}

// Workgroup i runs tiles of bin i mod 8 (the XCD the hardware gives it), at
// positions i / 8, i / 8 + gridDim.x / 8, ... of the bin.
// Workgroup `block` of `nblocks` runs the tiles of bin block mod 8, strided
// by nblocks / 8 (nblocks a multiple of 8).
template <int DT, int G, int STAGES, int WAVES>
__device__ __forceinline__ void append_worker(const AttnParams& p, int block, int nblocks,
                                              uint16_t* smem, int& s_flag) {
  const int x = block % kAppendBins, stride = nblocks / kAppendBins;
  const int t1 = p.worker_ptr[x + 1];
  for (int t = p.worker_ptr[x] + block / kAppendBins; t < t1; t += stride)
    append_tile<DT, G, STAGES, WAVES>(p, t, smem, s_flag);
}

}  // namespace app
}  // namespace pkfa
