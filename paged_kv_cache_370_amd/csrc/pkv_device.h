// Device-side helpers shared by the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// Storage tags for cache / query element types.
struct F32 { using storage = float; static constexpr int bytes = 4; };
struct BF16 { using storage = uint16_t; static constexpr int bytes = 2; };
struct FP8 { using storage = uint8_t; static constexpr int bytes = 1; };

// ------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two OCP E4M3FN codes (bytes 0,1 of w, or 2,3 when HI) -> two floats, exact.
// gfx950's v_cvt_pk_f32_fp8 decodes the OCP encoding (the NaN code 0x7f/0xff
// gives NaN, subnormals are kept).
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  a = v[0];
  b = v[1];
}

// float -> OCP E4M3FN code: round to nearest even on the float32 bit pattern,
// magnitudes >= 448 (infinity included) saturate to 448, NaN -> 0x7f.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  const float af = __uint_as_float(a);
  uint32_t code;
  if (af >= 448.0f) {
    code = 0x7eu;
  } else if (af < 0.015625f) {
    // subnormal grid: multiples of 2^-9; the product is exact, rint is RNE.
    code = (uint32_t)__builtin_rintf(af * 512.0f);
  } else {
    // keep 3 mantissa bits, RNE, then move the exponent bias from 127 to 7
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

// --------------------------------------------------------- wave primitives
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] and [2,3,0,1], row
// half-mirror (lane i <-> 7-i within 8), row mirror (lane i <-> 15-i).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same
// bits (each step adds two operands in both orders, which commutes exactly).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xb1>(x);
  x += dpp<0x4e>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xb1>(x));
  x = fmaxf(x, dpp<0x4e>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// ----------------------------------------------------------- vector loads

template <int NWORDS>
struct Words { uint32_t w[NWORDS]; };

template <int NWORDS>
__device__ __forceinline__ Words<NWORDS> load_words(const void* p) {
  Words<NWORDS> r;
  if constexpr (NWORDS == 1) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NWORDS == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    static_assert(NWORDS % 4 == 0, "vector width");
#pragma unroll
    for (int i = 0; i < NWORDS / 4; ++i) {
      uint4 v = reinterpret_cast<const uint4*>(p)[i];
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  }
  return r;
}

// E consecutive elements of type CT held in words -> floats.
template <typename CT, int E>
__device__ __forceinline__ void words_to_f32(const uint32_t* w, float* f) {
  if constexpr (sizeof(typename CT::storage) == 4) {
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = __uint_as_float(w[e]);
  } else if constexpr (sizeof(typename CT::storage) == 2) {
#pragma unroll
    for (int e = 0; e < E / 2; ++e) { f[2 * e] = bf16_lo(w[e]); f[2 * e + 1] = bf16_hi(w[e]); }
  } else {
#pragma unroll
    for (int e = 0; e < E / 4; ++e) {
      fp8x2_to_f32<false>(w[e], f[4 * e], f[4 * e + 1]);
      fp8x2_to_f32<true>(w[e], f[4 * e + 2], f[4 * e + 3]);
    }
  }
}

}  // namespace pkv
