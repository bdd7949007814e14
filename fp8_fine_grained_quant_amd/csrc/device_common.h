// Device helpers shared by the quantizer and GEMM kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Largest E4M3FN magnitude and the floor applied to a group's max-abs so that
// an all-zero group has a finite, non-zero scale.
constexpr float kFp8Max = 448.0f;
constexpr float kAmaxFloor = 7.8886090522101181e-31f;  // 2^-100, exact in FP32

// A buffer-load vector offset at or above the range of every buffer
// descriptor built here (all ranges are below 2^31 bytes).  The range check
// of a raw buffer access covers the vector offset plus the instruction
// offset, so such a load performs no memory access and returns zeros; the
// GEMMs use it for loads that only keep every wave's load count per chunk
// equal.
constexpr uint32_t kNoAccess = 0x80000000u;

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

// The same for values of a group scaled by fl32(448/amax') of its own
// max-abs: |x| <= amax' gives |fl32(x * fl32(448/amax'))| <= 448 (1 + 2^-23),
// below the 464 from which the conversion turns to NaN, and the conversion
// rounds (448, 464) to 448.  The clamp can change no code, so it is left out
// (it was a sixth of the dual quantizer's vector instructions).
__device__ __forceinline__ uint32_t pack4_e4m3_grp(float v0, float v1, float v2, float v3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
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

// Lane L of every 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int L>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + L, 0xF, 0xF, false));
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming accesses: every input byte is read once and every output byte
// written once.
// NT = 1 marks the access non-temporal.  Measured on MI355X: it pays for
// inputs read once and for long output streams written in full segments (the
// stacked expert weights), and loses for outputs that the next kernel reads
// (they would have stayed in the 256 MB MALL) and for scattered short stores,
// so each kernel picks per access.
template <int NT>
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}
template <int NT>
__device__ __forceinline__ void st_stream8(void* p, uint32_t a, uint32_t b) {
  if (NT) __builtin_nontemporal_store(u32x2{a, b}, reinterpret_cast<u32x2*>(p));
  else *reinterpret_cast<u32x2*>(p) = u32x2{a, b};
}
template <int NT>
__device__ __forceinline__ void st_stream16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  if (NT) __builtin_nontemporal_store(u32x4{a, b, c, d}, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = u32x4{a, b, c, d};
}
template <int NT>
__device__ __forceinline__ void st_stream4(void* p, uint32_t a) {
  if (NT) __builtin_nontemporal_store(a, reinterpret_cast<uint32_t*>(p));
  else *reinterpret_cast<uint32_t*>(p) = a;
}

struct BF16In {
  typedef uint16_t elem;
  static constexpr int kBytes = 2;
  template <int NT = 0>
  __device__ __forceinline__ static void load8(const elem* p, float v[8]) {
    const u32x4 u = ld_stream16<NT>(p);
    v[0] = bf16_to_f32(u[0] & 0xFFFFu); v[1] = bf16_to_f32(u[0] >> 16);
    v[2] = bf16_to_f32(u[1] & 0xFFFFu); v[3] = bf16_to_f32(u[1] >> 16);
    v[4] = bf16_to_f32(u[2] & 0xFFFFu); v[5] = bf16_to_f32(u[2] >> 16);
    v[6] = bf16_to_f32(u[3] & 0xFFFFu); v[7] = bf16_to_f32(u[3] >> 16);
  }
  __device__ __forceinline__ static float load1(const elem* p) { return bf16_to_f32(*p); }
};

struct F32In {
  typedef float elem;
  static constexpr int kBytes = 4;
  template <int NT = 0>
  __device__ __forceinline__ static void load8(const elem* p, float v[8]) {
    const u32x4 a = ld_stream16<NT>(p), b = ld_stream16<NT>(p + 4);
    v[0] = __uint_as_float(a[0]); v[1] = __uint_as_float(a[1]); v[2] = __uint_as_float(a[2]); v[3] = __uint_as_float(a[3]);
    v[4] = __uint_as_float(b[0]); v[5] = __uint_as_float(b[1]); v[6] = __uint_as_float(b[2]); v[7] = __uint_as_float(b[3]);
  }
  __device__ __forceinline__ static float load1(const elem* p) { return *p; }
};

}  // namespace fp8q
