// OCP MX formats on the device [OCP-MX]: e2m1 -> e4m3fn conversion (lossless), MXFP8
// quantisation (shared exponent floor(log2 amax) - 8, elements rounded to nearest even and
// saturated at +-448), all in integer arithmetic so subnormal inputs and outputs are exact
// whatever the floating-point denormal mode.
#pragma once

#include "common.h"

namespace bitmoe {

// Eight e4m3fn magnitude bytes of the e2m1 values 0, 0.5, 1, 1.5, 2, 3, 4, 6 (by the low three
// bits of the nibble); the nibble's sign bit becomes bit 7.
constexpr uint32_t kE2m1ToE4m3Lo = 0x3C383000u;
constexpr uint32_t kE2m1ToE4m3Hi = 0x4C484440u;

// One code word (8 nibbles, element 2i in the low nibble of byte i) -> 8 e4m3fn bytes.
__device__ __forceinline__ void e2m1x8_to_e4m3(uint32_t w, uint32_t& out0, uint32_t& out1) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // even / odd elements
  const uint32_t elo = byte_perm(kE2m1ToE4m3Hi, kE2m1ToE4m3Lo, lo & 0x07070707u) | ((lo & 0x08080808u) << 4);
  const uint32_t ehi = byte_perm(kE2m1ToE4m3Hi, kE2m1ToE4m3Lo, hi & 0x07070707u) | ((hi & 0x08080808u) << 4);
  out0 = byte_perm(ehi, elo, 0x05010400u);  // elements 0..3
  out1 = byte_perm(ehi, elo, 0x07030602u);  // elements 4..7
}

// Position of the most significant set bit of v > 0.
__device__ __forceinline__ int msb32(uint32_t v) { return 31 - __clz((int)v); }

// e4m3fn byte (without sign) of the positive value M * 2^F (M > 0 an integer below 2^25),
// rounded to nearest even, saturated at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_mag_rne(uint32_t M, int F) {
  const int m = msb32(M);
  const int fl = m + F;                 // floor(log2(value))
  if (fl > 8) return 0x7Eu;
  int sh;                               // right shift that leaves the result's unit in bit 0
  int ebase;                            // biased exponent of a normal result before carry
  if (fl >= -6) {                       // normal: keep 4 significant bits
    sh = m - 3;
    ebase = fl + 7;
  } else {                              // subnormal: units of 2^-9
    sh = -(F + 9);
    ebase = 0;
  }
  uint32_t q;
  if (sh <= 0) {
    q = M << (-sh);
  } else if (sh > 25) {
    q = 0;
  } else {
    q = M >> sh;
    const uint32_t rem = M & ((1u << sh) - 1u), half = 1u << (sh - 1);
    q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  }
  uint32_t byte;
  if (ebase == 0) {
    byte = q;                           // q == 8 is the smallest normal, 0x08
  } else {
    // q in [8, 16]: 16 carries into the exponent
    byte = q == 16u ? (uint32_t)(ebase + 1) << 3 : ((uint32_t)ebase << 3) | (q - 8u);
  }
  return byte > 0x7Eu ? 0x7Eu : byte;
}

// floor(log2 |v|) of a bf16 magnitude (15 bits, > 0), and of an fp32 magnitude (31 bits, > 0).
__device__ __forceinline__ int floor_log2_bf16(uint32_t mag) {
  const uint32_t eb = mag >> 7;
  return eb ? (int)eb - 127 : msb32(mag) - 133;
}
__device__ __forceinline__ int floor_log2_f32(uint32_t mag) {
  const uint32_t eb = mag >> 23;
  return eb ? (int)eb - 127 : msb32(mag) - 149;
}

// Shared MX exponent of a block from floor(log2 amax) (amax > 0); -127 for an all-zero block.
__device__ __forceinline__ int mx_shared_exp(int fl_amax, bool zero) {
  if (zero) return -127;
  const int s = fl_amax - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// e4m3fn byte of bf16 bits b times 2^-shared.
__device__ __forceinline__ uint32_t bf16_to_e4m3_scaled(uint32_t b, int shared) {
  const uint32_t sgn = (b >> 8) & 0x80u, mag = b & 0x7FFFu;
  if (mag == 0) return sgn;
  const uint32_t eb = mag >> 7, mb = mag & 0x7Fu;
  const uint32_t M = eb ? (mb | 0x80u) : mb;
  const int E0 = eb ? (int)eb - 134 : -133;
  return sgn | e4m3_mag_rne(M, E0 - shared);
}

// Four e4m3fn bytes (v0 in the low byte) of fp32 values times 2^-shared (finite values,
// shared in [-127, 127]), rounded to nearest even and saturated at 448.  gfx950's fp8
// conversion (OCP e4m3fn, round to nearest even) of the value scaled by ldexp -- exact for every
// result at or above 2^-126, and anything smaller rounds to zero either way -- and clamped to
// +-448 first.  Checked on the device equal to e4m3_mag_rne of the exact value for every finite
// fp32 input and every shared exponent.
__device__ __forceinline__ float e4m3_prescale(float v, int shared) {
  return __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(v, -shared), 448.0f, -448.0f);
}
__device__ __forceinline__ uint32_t e4m3x4_scaled(float v0, float v1, float v2, float v3, int shared) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale(v0, shared), e4m3_prescale(v1, shared), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prescale(v2, shared), e4m3_prescale(v3, shared), lo, true);
}

}  // namespace bitmoe
