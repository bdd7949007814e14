// Device helpers shared by the quantizer and GEMM kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Largest E4M3FN magnitude and the floor applied to a group's max-abs so that
// an all-zero group has a finite, non-zero scale.
constexpr float kFp8Max = 448.0f;
constexpr float kAmaxFloor = 7.8886090522101181e-31f;  // 2^-100, exact in FP32

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two FP32 values -> two E4M3FN codes in the low (hi_half = false) or high
// (hi_half = true) 16 bits of `old`.  gfx950's v_cvt_pk_fp8_f32 rounds to
// nearest even and keeps the sign of zero but turns magnitudes above 464 into
// NaN, so the inputs are clamped to +-448 first: that is exactly saturation.
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old, bool hi_half) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kFp8Max), kFp8Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kFp8Max), kFp8Max);
  return hi_half ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
                 : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Four FP32 values (already multiplied by the group's inverse scale) -> one
// dword of codes, byte i = code of v_i.
__device__ __forceinline__ uint32_t pack4_e4m3(float v0, float v1, float v2, float v3) {
  int w = cvt2_e4m3(v0, v1, 0, false);
  w = cvt2_e4m3(v2, v3, w, true);
  return (uint32_t)w;
}

// Group scale rule: s = fl32(amax'/448) (stored), inv = fl32(448/amax').
// Both divisions are IEEE correctly rounded (the library is built without
// fast-math and with correctly rounded FP32 division).
__device__ __forceinline__ void group_scale(float amax, float& s, float& inv) {
  float a = __builtin_fmaxf(amax, kAmaxFloor);
  s = a / kFp8Max;
  inv = kFp8Max / a;
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of the
// row receives the result.  row_ror:n has DPP control 0x120 + n.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x128, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x122, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x121, 0xF, 0xF, false));
  return v;
}

// Max over the whole 64-lane wave; every lane receives the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// |x| as ordered integer bits (valid for finite values; larger magnitude ->
// larger integer).
__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

// Element loaders: 8 consecutive elements of type T from a 16-byte-aligned
// address (full), or element by element (n < 8 valid).
struct BF16In {
  typedef uint16_t elem;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static void load8(const elem* p, float v[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_to_f32(u.x & 0xFFFFu); v[1] = bf16_to_f32(u.x >> 16);
    v[2] = bf16_to_f32(u.y & 0xFFFFu); v[3] = bf16_to_f32(u.y >> 16);
    v[4] = bf16_to_f32(u.z & 0xFFFFu); v[5] = bf16_to_f32(u.z >> 16);
    v[6] = bf16_to_f32(u.w & 0xFFFFu); v[7] = bf16_to_f32(u.w >> 16);
  }
  __device__ __forceinline__ static float load1(const elem* p) { return bf16_to_f32(*p); }
};

struct F32In {
  typedef float elem;
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static void load8(const elem* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static float load1(const elem* p) { return *p; }
};

}  // namespace fp8q
