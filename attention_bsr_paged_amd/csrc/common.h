// Device helpers for the gfx950 kernels: storage types, packed conversions,
// dot2 products, DPP lane exchanges and base-2 exponentials.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/abp.h"

namespace abp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
// LDS (group segment) address space, for the gfx950 LDS load / transpose builtins
#define ABP_LDS __attribute__((address_space(3)))
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Loads of data read once per run (K/V rows in decode): non-temporal, so the
// stream does not evict data that other work reuses from the caches.
// Measured on batch decode: 101.5 us against 112.3 us with ordinary loads.
__device__ __forceinline__ uint4 load_once(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ uint2 load_once(const uint2* p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)));
}

// Read-only arrays whose loads at wave-uniform addresses should go through the
// scalar unit (plan records, page tables). Only loads are done through it.
#define ABP_CONST_AS __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const ABP_CONST_AS T* const_as(const T* p) {
  return (const ABP_CONST_AS T*)(p);
}

struct BF16 {};  // storage tags
struct F16 {};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// unpack one 32-bit word holding two 16-bit values to float
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float lo_f32(uint32_t w);
template <typename T>
__device__ __forceinline__ float hi_f32(uint32_t w);

template <>
__device__ __forceinline__ float lo_f32<BF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <>
__device__ __forceinline__ float hi_f32<BF16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
template <>
__device__ __forceinline__ float lo_f32<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w).x;
}
template <>
__device__ __forceinline__ float hi_f32<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w).y;
}

// pack two floats (round to nearest even) into one word
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  f16x2_t v;
  v.x = (_Float16)a;
  v.y = (_Float16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// c + a.lo * b.lo + a.hi * b.hi with fp32 accumulation
template <typename T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <>
__device__ __forceinline__ float dot2<BF16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
template <>
__device__ __forceinline__ float dot2<F16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                c, false);
}

// byte-select of two words: (lo16 of a, lo16 of b) and (hi16 of a, hi16 of b)
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---------------------------------------------------------------------------
// DPP lane exchanges inside a row of 16 lanes
// ---------------------------------------------------------------------------
enum Dpp : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141, // lane i <- 7 - i within 8
  kDppMirror = 0x140,     // lane i <- 15 - i within 16
  kDppRor8 = 0x128,       // lane i <- (i + 8) mod 16  (= xor 8)
};

// Every lane of the patterns used here has a valid source lane, so the "old"
// operand is never selected (mov_dpp leaves it undefined, which lets the
// compiler fold the move into the consuming add as a DPP operand).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xf, 0xf, true);
}

// sum over the 16 lanes of a row; every lane of the row gets the total
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

// ---------------------------------------------------------------------------
// RoPE angle: sin / cos of 2*pi*frac(pos * f) where f = fhi + flo is the
// frequency in revolutions per position. pos < 2^24 is exact in fp32; the
// product's rounding error is recovered with an fma, so the reduced angle is
// accurate to ~1e-7 revolutions at any position.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_sincos(float pos, float fhi, float flo, float* s, float* c) {
  const float x = pos * fhi;
  const float err = __builtin_fmaf(pos, fhi, -x);
  float r = __builtin_amdgcn_fractf(x) + __builtin_fmaf(pos, flo, err);
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// ---------------------------------------------------------------------------
// 8 consecutive elements of a row as floats: one 16-byte access for fp16/bf16,
// two for fp32. DT is an abp_dtype value.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float v[8]) {
  if constexpr (DT == ABP_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    using T = typename std::conditional<DT == ABP_BF16, BF16, F16>::type;
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = lo_f32<T>(ws[j]);
      v[2 * j + 1] = hi_f32<T>(ws[j]);
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t off, const float v[8]) {
  if constexpr (DT == ABP_F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    using T = typename std::conditional<DT == ABP_BF16, BF16, F16>::type;
    uint4 w;
    w.x = pack2<T>(v[0], v[1]);
    w.y = pack2<T>(v[2], v[3]);
    w.z = pack2<T>(v[4], v[5]);
    w.w = pack2<T>(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = w;
  }
}

}  // namespace abp
