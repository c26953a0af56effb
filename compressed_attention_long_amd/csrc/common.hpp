// Device helpers shared by the CSA/HCA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -3.0e38f;   // "no logit yet"; finite so that differences stay finite

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, two values at once with gfx950's packed converter (v_cvt_pk_bf16_f32):
// round to nearest even.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- fp16

// fp32 -> IEEE binary16, two values (round to nearest even: the conversion's default mode);
// and back, exactly.
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t w) {
  const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
  return f32x2{(float)v[0], (float)v[1]};
}

// ---------------------------------------------------------------- fp8 e4m3fn (OCP)

// Two codes (bytes 0,1 or 2,3 of `w`) -> two fp32 values; gfx950's converter reads OCP E4M3FN.
__device__ __forceinline__ f32x2 fp8x2_lo(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false); }
__device__ __forceinline__ f32x2 fp8x2_hi(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true); }

// fp32 -> OCP E2M1 code (4 bits), round to nearest even on the E2M1 grid, saturating at
// +-6; written from the format definition: 1 sign, 2 exponent (bias 1), 1 mantissa bit,
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (the grid step is 0.5 below 2, 1 below 4, 2 above).
// Negative zero encodes as +0.
__device__ __forceinline__ uint32_t f32_to_fp4_e2m1(float x) {
  const float a = fminf(fabsf(x), 6.0f);
  uint32_t code;
  if (a < 2.0f) code = (uint32_t)rintf(a * 2.0f);              // 0..4 (4 = 2.0, exponent 2)
  else if (a < 4.0f) code = (uint32_t)rintf(a) + 2u;          // 2, 3, 4 -> codes 4, 5, 6
  else code = (uint32_t)rintf(a * 0.5f) + 4u;                 // 4, 6 -> codes 6, 7
  return code == 0 ? 0u : (code | ((__float_as_uint(x) >> 28) & 8u));
}

// ---------------------------------------------------------------- rotary

// (cos, sin) of pos * inv_freq, returned in fp32.  The angle is formed in fp64 and reduced
// modulo 2*pi there (k = nearest integer to angle / 2pi, then angle - k * 2pi with 2pi split
// into a 53-bit head and a tail, Cody-Waite style; for the positions here, k < 2^22, the
// reduction error is ~1e-16 rad).  The reduced angle |r| <= pi is then rounded to fp32
// (error <= 2^-23 rad) and its sine and cosine taken in fp32 (a few fp32 ulps): far below
// the bf16 rounding of the rotated values.
__device__ __forceinline__ void rope_cs(int64_t pos, double inv_freq, float& c, float& s) {
  const double ang = (double)pos * inv_freq;
  const double k = rint(ang * 0.15915494309189535);          // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, ang);                // 2 pi, head
  r = fma(-k, 2.4492935982947064e-16, r);                    // 2 pi, tail
  sincosf((float)r, &s, &c);
}

// ---------------------------------------------------------------- XCD-aware block order

// Blocks are dispatched round-robin over the 8 XCDs (block L lands on XCD L % 8).
// Remap so that each XCD works on one contiguous range of logical blocks: neighbours in
// logical order (which share input rows) then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t L, uint32_t total) {
  if ((total & 7u) != 0u) return L;
  return (L & 7u) * (total >> 3) + (L >> 3);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

}  // namespace csa
