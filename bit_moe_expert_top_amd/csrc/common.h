// Device-side helpers shared by the gfx950 kernels of the low-bit MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (the compiler's bf16
// conversion), which equals the integer rounding (u + 0x7FFF + bit 16 of u) >> 16 for every
// finite fp32 input (checked on the device over all 2^32 bit patterns).  Finite inputs only.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two of them packed, a in the low half: one instruction
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies A row l%16 and B column
// l%16, each for the 8 k-slots 8*(l/16) .. 8*(l/16)+7 (two bf16 per 32-bit word, low half
// first); it receives D rows 4*(l/16) .. +3 of column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_perm_b32: byte j of the result is byte sel.byte[j] of the 8-byte value {hi:lo}
// (0..3 pick from `lo`, 4..7 from `hi`).
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Raw buffer loads: a uniform base + byte size (the "resource") and a per-lane 32-bit byte
// offset.  A lane whose offset is >= the size reads zeros and makes no memory request, so
// inactive lanes need no branch (the load stays unconditional).
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr uint32_t kOffNone = 0x80000000u;  // an offset past any buffer this library makes
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(buf_rsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x4 buf_load16s(buf_rsrc r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

__device__ __forceinline__ int wave_lane() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, <= 1024).
// `tmp` needs NT/64 + 1 ints of shared memory.  Returns the exclusive prefix of `v`;
// *total receives the block total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = wave_lane(), w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) tmp[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < NT / kWave; ++i) {
      int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
    tmp[NT / kWave] = run;
  }
  __syncthreads();
  int res = tmp[w] + incl - v;
  *total = tmp[NT / kWave];
  __syncthreads();
  return res;
}

}  // namespace bitmoe
