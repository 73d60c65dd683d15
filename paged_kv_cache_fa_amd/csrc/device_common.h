// Device helpers shared by the gfx950 kernels: element types, packed dot
// products, DPP lane exchanges, fast exp2/log2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa.h"

namespace pkfa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-bit storage types. dot2: fp32 c + a.lo*b.lo + a.hi*b.hi over packed pairs.
template <int DT>
struct Elt;

template <>
struct Elt<FA_BF16> {
  __device__ __forceinline__ static float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
  __device__ __forceinline__ static float lo(uint32_t x) { return __uint_as_float(x << 16); }
  __device__ __forceinline__ static float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
  __device__ __forceinline__ static uint32_t pack(float a, float b) {
    // hardware round-to-nearest-even conversion (v_cvt_pk_bf16_f32)
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  // Two E4M3 codes (bytes 2W, 2W+1 of x) widened to a bf16 pair, exactly
  // (every E4M3 value is a bf16 value; scale operand 1).
  template <bool W>
  __device__ __forceinline__ static uint32_t from_e4m3(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, W));
  }
};

template <>
struct Elt<FA_F16> {
  __device__ __forceinline__ static float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
  }
  __device__ __forceinline__ static float lo(uint32_t x) {
    return (float)__builtin_bit_cast(f16x2_t, x).x;
  }
  __device__ __forceinline__ static float hi(uint32_t x) {
    return (float)__builtin_bit_cast(f16x2_t, x).y;
  }
  __device__ __forceinline__ static uint32_t pack(float a, float b) {
    f16x2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  // Two E4M3 codes widened to an fp16 pair, exactly (E4M3's range and
  // 3-bit mantissa fit fp16).
  template <bool W>
  __device__ __forceinline__ static uint32_t from_e4m3(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, W));
  }
};

// DPP lane exchange inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

// Sum over the 8 consecutive lanes of an aligned octet; every lane gets the sum.
__device__ __forceinline__ float octet_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Exchanges across lane bits 3, 4 and 5 without LDS: a row rotate by 8 (DPP)
// pairs lanes l and l^8 inside each row of 16; v_permlane16_swap /
// v_permlane32_swap on (x, x) return x of lanes l and l^16 (l^32) in some
// order, which is all a symmetric reduction needs.
constexpr int kDppRowRor8 = 0x128;
__device__ __forceinline__ float xor8(float x) { return dpp<kDppRowRor8>(x); }
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace pkfa
