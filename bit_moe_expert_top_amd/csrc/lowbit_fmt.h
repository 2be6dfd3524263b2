// Low-bit expert formats on the device: loading packed codes and scales, decoding them into
// bf16 MFMA operands, and the k-slot order those operands use.
//
// Both formats decode to EXACT bf16 weights (level * scale needs at most 7 significant bits),
// so the MFMA sees the same values the format defines.  MFMA only needs its two operands to
// agree on which k sits in which slot, so each format decodes in the order cheapest for its
// bit layout and the token operand (x, and h for FC2) is stored in that same order: within
// every 32 consecutive k, slot s holds k = slot_k(s) and k = c sits in slot pos32(c).
//
// A lane's unit of work ("step") is 64 consecutive k of one weight row: 8 operands of 8 bf16.
// Operand o of a step pairs with bytes [16 o, 16 o + 16) of the lane's 128-byte slice of the
// token operand.
#pragma once

#include "common.h"

namespace bitmoe {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Scale bytes of one super-step (NB = bytes per step * steps per super-step, 1..16).
template <int NB>
struct ScaleBytes {
  uint32_t v[NB >= 4 ? NB / 4 : 1];
};
template <int NB>
__device__ __forceinline__ ScaleBytes<NB> load_scale_bytes_s(buf_rsrc r, uint32_t off, uint32_t soff) {
  ScaleBytes<NB> s;
  if constexpr (NB == 1) {
    s.v[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, (int)soff, 0);
  } else if constexpr (NB == 2) {
    s.v[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, (int)soff, 0);
  } else if constexpr (NB == 4) {
    s.v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, (int)soff, 0);
  } else if constexpr (NB == 8) {
    const uint64_t t = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, 0));
    s.v[0] = (uint32_t)t;
    s.v[1] = (uint32_t)(t >> 32);
  } else {
    const u32x4 t = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0));
    s.v[0] = t[0];
    s.v[1] = t[1];
    s.v[2] = t[2];
    s.v[3] = t[3];
  }
  return s;
}
template <int NB>
__device__ __forceinline__ ScaleBytes<NB> load_scale_bytes(buf_rsrc r, uint32_t off) {
  ScaleBytes<NB> s;
  if constexpr (NB == 1) {
    s.v[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
  } else if constexpr (NB == 2) {
    s.v[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  } else if constexpr (NB == 4) {
    s.v[0] = buf_load4(r, off);
  } else if constexpr (NB == 8) {
    const uint64_t t = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    s.v[0] = (uint32_t)t;
    s.v[1] = (uint32_t)(t >> 32);
  } else {
    const u32x4 t = buf_load16(r, off);
    s.v[0] = t[0];
    s.v[1] = t[1];
    s.v[2] = t[2];
    s.v[3] = t[3];
  }
  return s;
}

// =====================================================================================
// 2-bit codebook [Moet-QA]: codes u32[rows][K/16] (code i of a word at bits [2i, 2i+2)),
// level {-4,-1,1,4}[code], one bf16 scale per 32 along K.
//
// The levels are +-1 and +-4, so level*scale is the scale's bf16 with the sign flipped and/or
// 2 added to the exponent: every weight of a group has the scale's low byte, and a byte table
// of the four high bytes {-4s, -s, s, 4s} is looked up with one v_perm_b32 per four codes
// (masking a word shifted by 2u with 0x03030303 leaves codes u, 4+u, 8+u, 12+u one per byte:
// a selector).  Two more v_perm_b32 interleave the low byte, taken straight from the scale
// word: ~1.2 VALU operations per weight.  The table itself is one v_perm_b32 (byte broadcast
// of the high byte and of its sign-flipped copy) and one add per group.
// Slot order: within every 16 k, slots hold k = 0,4,8,12, 1,5,9,13, 2,6,10,14, 3,7,11,15.
// =====================================================================================
struct W2Fmt {
  static constexpr int kId = 1;
  static constexpr int kStepCodeBytes = 16;  // 64 codes
  static constexpr int kStepScaleBytes = 4;  // 2 bf16
  __host__ __device__ static constexpr uint32_t code_bytes(uint32_t k) { return k / 4; }
  __host__ __device__ static constexpr uint32_t scale_bytes(uint32_t k) { return k / 16; }

  struct Codes { u32x4 w; };
  // lut[g]: the four high bytes of group g; sw: the scale word (bf16 of group g in half g)
  struct Tab { uint32_t lut[2], sw; };

  __device__ static __forceinline__ Codes load_codes(buf_rsrc r, uint32_t off) { return {buf_load16(r, off)}; }
  __device__ static __forceinline__ Codes load_codes_s(buf_rsrc r, uint32_t off, uint32_t soff) {
    return {buf_load16s(r, off, soff)};
  }

  // high bytes {-4s, -s, s, 4s} of group g: bytes (hb^0x80)+1, hb^0x80, hb, hb+1 (the sign
  // flip, the exponent +2 in the high byte); x = sw with both sign bits flipped
  template <int g>
  __device__ static __forceinline__ uint32_t lut_of(uint32_t x, uint32_t sw) {
    return byte_perm(x, sw, g == 0 ? 0x01010505u : 0x03030707u) + 0x01000001u;
  }
  // the step's scale word: bf16 of k [0,32) in the low half, of k [32,64) in the high half
  __device__ static __forceinline__ Tab table(uint32_t sw) {
    Tab t;
    const uint32_t x = sw ^ 0x80008000u;
    t.lut[0] = lut_of<0>(x, sw);
    t.lut[1] = lut_of<1>(x, sw);
    t.sw = sw;
    return t;
  }
  template <int NB>
  __device__ static __forceinline__ uint32_t step_scale(const ScaleBytes<NB>& s, int step) { return s.v[step]; }

  // half 0 covers u = 0, 1 and half 1 u = 2, 3; per u: dwords (code u, 4+u), (8+u, 12+u);
  // the low byte of group g is byte 2g of the scale word sw
  template <int g>
  __device__ static __forceinline__ u32x4 decode_word(uint32_t w, int half, uint32_t lut, uint32_t sw) {
    u32x4 r;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int sh = 2 * (2 * half + u);
      const uint32_t hb = byte_perm(0u, lut, (w >> sh) & 0x03030303u);
      r[2 * u] = byte_perm(sw, hb, g == 0 ? 0x01040004u : 0x01060006u);
      r[2 * u + 1] = byte_perm(sw, hb, g == 0 ? 0x03040204u : 0x03060206u);
    }
    return r;
  }
  // operand o (0..7) of a step: word o/2, half o%2 (o is a constant after unrolling)
  __device__ static __forceinline__ u32x4 decode(const Codes& c, const Tab& t, int o) {
    const int wd = o >> 1;
    return wd < 2 ? decode_word<0>(c.w[wd], o & 1, t.lut[0], t.sw) : decode_word<1>(c.w[wd], o & 1, t.lut[1], t.sw);
  }
  // slot of k = c (0..31) in its 32-k block, and the k held by slot s
  __host__ __device__ static constexpr int pos32(int c) {
    return (c & 16) + 4 * ((c & 15) & 3) + ((c & 15) >> 2);
  }
  __host__ __device__ static constexpr int slot_k(int s) {
    return (s & 16) + 4 * ((s & 15) & 3) + ((s & 15) >> 2);  // the 4x4 transpose is an involution
  }

  // 32 codes (one group) for the GEMM's LDS tiles: words w[0], w[1], the group's bf16 scale.
  static constexpr int kFieldWords = 2;
  __device__ static __forceinline__ Tab table32(uint32_t s16) {
    Tab t;
    t.lut[0] = lut_of<0>(s16 ^ 0x8000u, s16);
    t.lut[1] = t.lut[0];
    t.sw = s16;
    return t;
  }
  __device__ static __forceinline__ u32x4 decode32(const uint32_t* w, const Tab& t, int op) {
    return decode_word<0>(w[op >> 1], op & 1, t.lut[0], t.sw);
  }
};

// =====================================================================================
// 3-bit, eight levels [Strata-R9700] path 6: codes u32[rows][K/32*3], the three words of a
// 32-code field form one LSB-first 96-bit value with code i at bits [3i, 3i+3); level
// {-8,-5,-3,-1,1,3,5,8}[code]; one e4m3fn scale byte per 64 along K, weight = level*e4m3/64.
//
// Per group a lane builds byte tables of the eight exact bf16 values level*scale (high and
// low bytes, 2 x 2 dwords).  Codes reach selector bytes without per-code work: in the 12
// bytes B0..B11 of a field, byte j holds whole codes at bit offsets j%3 and j%3+3, and the
// codes at bits 6 and 15 of every 3-byte period straddle two bytes.  One v_perm_b32 gathers
// two same-offset byte pairs per dword ([B0,B9 | B2,B8], [B3,B6 | B1,B4], [B7,B10 | B5,B11]);
// a packed 16-bit shift (one amount per pair) and a 0x07 mask per byte then yield four codes,
// twice per gathered dword.  The straddling codes become whole-byte codes at offsets 4 and 5
// of the field shifted right by 2 bits (two v_alignbit_b32), gathered the same way.  Each
// selector dword is looked up in the high- and low-byte tables (two v_perm_b32) and
// interleaved into two bf16 pairs (two more): ~2 VALU operations per weight.
// =====================================================================================
static __constant__ uint8_t kW3SlotK[32] = {0, 24, 6, 22, 1, 25, 7, 23, 8, 16, 3, 11, 9, 17, 4, 12,
                                            19, 27, 14, 30, 20, 28, 15, 31, 2, 10, 5, 13, 18, 26, 21, 29};
static __constant__ uint8_t kW3Pos[32] = {0, 4, 24, 10, 14, 26, 2, 6, 8, 12, 25, 11, 15, 27, 18, 22,
                                          9, 13, 28, 16, 20, 30, 3, 7, 1, 5, 29, 17, 21, 31, 19, 23};

struct W3Fmt {
  static constexpr int kId = 2;
  static constexpr int kStepCodeBytes = 24;  // 64 codes (two fields)
  static constexpr int kStepScaleBytes = 1;  // one e4m3 byte
  __host__ __device__ static constexpr uint32_t code_bytes(uint32_t k) { return k / 32 * 12; }
  __host__ __device__ static constexpr uint32_t scale_bytes(uint32_t k) { return k / 64; }

  struct Codes { u32x4 a; uint32_t b0, b1; };
  struct Tab { uint32_t hb1, hb0, lb1, lb0; };

  __device__ static __forceinline__ Codes load_codes_s(buf_rsrc r, uint32_t off, uint32_t soff) {
    Codes c;
    c.a = buf_load16s(r, off, soff);
    const uint64_t t = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off + 16u), (int)soff, 0));
    c.b0 = (uint32_t)t;
    c.b1 = (uint32_t)(t >> 32);
    return c;
  }
  __device__ static __forceinline__ Codes load_codes(buf_rsrc r, uint32_t off) {
    Codes c;
    c.a = buf_load16(r, off);
    const uint64_t t = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off + 16u), 0, 0));
    c.b0 = (uint32_t)t;
    c.b1 = (uint32_t)(t >> 32);
    return c;
  }

  // fp32 bits of e4m3fn(b) / 64 (finite bytes): normal numbers by rebiasing the exponent
  // (7 + 6 -> 127: add 114), subnormals m * 2^-9 / 64 = m * 2^-15 exactly.
  __device__ static __forceinline__ uint32_t scale_f32_bits(uint32_t b) {
    const uint32_t mag = b & 0x7Fu;
    const uint32_t nrm = (mag << 20) + (114u << 23);
    const uint32_t sub = __float_as_uint((float)mag * 0x1p-15f);
    return ((mag >> 3) ? nrm : sub) | ((b & 0x80u) << 24);
  }
  __device__ static __forceinline__ Tab table(uint32_t b) {
    const float s = __uint_as_float(scale_f32_bits(b));
    const uint32_t f1 = __float_as_uint(s), f3 = __float_as_uint(3.0f * s);
    const uint32_t f5 = __float_as_uint(5.0f * s), f8 = __float_as_uint(8.0f * s);
    const uint32_t p13 = byte_perm(f3, f1, 0x07030602u);  // [lo1, lo3, hi1, hi3]
    const uint32_t p58 = byte_perm(f8, f5, 0x07030602u);  // [lo5, lo8, hi5, hi8]
    Tab t;
    t.lb1 = byte_perm(p58, p13, 0x05040100u);             // levels 1, 3, 5, 8
    t.hb1 = byte_perm(p58, p13, 0x07060302u);
    t.lb0 = byte_perm(0u, t.lb1, 0x00010203u);            // levels -8, -5, -3, -1
    t.hb0 = byte_perm(0u, t.hb1, 0x00010203u) ^ 0x80808080u;
    return t;
  }
  template <int NB>
  __device__ static __forceinline__ uint32_t step_scale(const ScaleBytes<NB>& s, int step) {
    return (s.v[step >> 2] >> (8 * (step & 3))) & 0xFFu;
  }

  __device__ static __forceinline__ uint32_t sel(uint32_t v, uint16_t a, uint16_t b) {
    const u16x2 r = __builtin_bit_cast(u16x2, v) >> u16x2{a, b};
    return __builtin_bit_cast(uint32_t, r) & 0x07070707u;
  }
  __device__ static __forceinline__ void lookup(uint32_t s, const Tab& t, uint32_t& d0, uint32_t& d1) {
    const uint32_t hb = byte_perm(t.hb1, t.hb0, s), lb = byte_perm(t.lb1, t.lb0, s);
    d0 = byte_perm(hb, lb, 0x05010400u);
    d1 = byte_perm(hb, lb, 0x07030602u);
  }
  // operand op (0..3) of the field (w0, w1, w2); op is a constant after unrolling
  __device__ static __forceinline__ u32x4 decode_field(uint32_t w0, uint32_t w1, uint32_t w2, int op,
                                                      const Tab& t) {
    uint32_t s0, s1;
    if (op == 0) {
      const uint32_t z = byte_perm(w2, w0, 0x04020500u);  // [B0, B9, B2, B8]
      s0 = sel(z, 0, 2);
      s1 = sel(z, 3, 5);
    } else if (op == 1) {
      const uint32_t x = byte_perm(w1, w0, 0x04010603u);  // [B3, B6, B1, B4]
      s0 = sel(x, 0, 1);
      s1 = sel(x, 3, 4);
    } else if (op == 2) {
      const uint32_t y = byte_perm(w2, w1, 0x07010603u);  // [B7, B10, B5, B11]
      s0 = sel(y, 1, 2);
      s1 = sel(y, 4, 5);
    } else {
      const uint32_t a0 = __builtin_amdgcn_alignbit(w1, w0, 2u), a1 = __builtin_amdgcn_alignbit(w2, w1, 2u);
      const uint32_t a2 = w2 >> 2;
      s0 = sel(byte_perm(a1, a0, 0x04010300u), 4, 5);     // [S0, S3, S1, S4] of (field >> 2)
      s1 = sel(byte_perm(a2, a1, 0x06030502u), 4, 5);     // [S6, S9, S7, S10]
    }
    uint32_t d0, d1, d2, d3;
    lookup(s0, t, d0, d1);
    lookup(s1, t, d2, d3);
    return u32x4{d0, d1, d2, d3};
  }
  __device__ static __forceinline__ u32x4 decode(const Codes& c, const Tab& t, int o) {
    return o < 4 ? decode_field(c.a[0], c.a[1], c.a[2], o & 3, t) : decode_field(c.a[3], c.b0, c.b1, o & 3, t);
  }
  __device__ static __forceinline__ int pos32(int c) { return kW3Pos[c]; }
  __device__ static __forceinline__ int slot_k(int s) { return kW3SlotK[s]; }

  // one field for the GEMM's LDS tiles: words w[0..2], the scale byte of its group
  static constexpr int kFieldWords = 3;
  __device__ static __forceinline__ Tab table32(uint32_t b) { return table(b); }
  __device__ static __forceinline__ u32x4 decode32(const uint32_t* w, const Tab& t, int op) {
    return decode_field(w[0], w[1], w[2], op, t);
  }
};

// =====================================================================================
// MXFP4 residual of a 2-bit expert ([Moet-QA]: the FP4 delta cache above the 2-bit weights;
// [OCP-MX] e2m1 elements, one e8m0 scale per 32 along K): codes u8[rows][K/2] (element 2i in
// the low nibble), scales u8[rows][K/32].  Decoded to exact bf16 values e2m1 * 2^(scale - 127)
// in the 2-bit format's k-slot order, so that its MFMAs share the token operand of the 2-bit
// pass and accumulate into the same sums (the residual is added before SwiGLU).
//
// Per 32-k group a lane builds byte tables of the eight magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
// times the scale (high and low bytes, 2 x 2 dwords: the bf16 bits of each magnitude plus
// (scale - 127) << 7, one packed 16-bit add per pair; magnitude 0 stays 0).  The bytes of a
// 16-k block holding the slot's k (even bytes for slots 0-7 -- k 0,4,8,12 in the low nibbles,
// k 1,5,9,13 in the high ones -- odd bytes for slots 8-15) are gathered by one v_perm_b32; the
// magnitudes masked into selector bytes are looked up in both tables, the nibble's sign bit is
// xor-ed into the high byte, and two v_perm_b32 interleave high and low bytes into bf16 pairs.
// Exact for scale bytes in [2, 252] (every nonzero value then a normal bf16).
// =====================================================================================
struct Fp4Fmt {
  static constexpr int kId = 3;
  static constexpr int kStepCodeBytes = 32;  // 64 codes
  static constexpr int kStepScaleBytes = 2;  // 2 e8m0 bytes
  __host__ __device__ static constexpr uint32_t code_bytes(uint32_t k) { return k / 2; }
  __host__ __device__ static constexpr uint32_t scale_bytes(uint32_t k) { return k / 32; }

  struct Codes { u32x4 a, b; };
  struct GTab { uint32_t hb0, hb1, lb0, lb1; };  // magnitudes 0-3 / 4-7, high / low bytes
  struct Tab { GTab g[2]; };                      // the step's two groups

  __device__ static __forceinline__ Codes load_codes(buf_rsrc r, uint32_t off) {
    return {buf_load16(r, off), buf_load16(r, off + 16u)};
  }
  __device__ static __forceinline__ Codes load_codes_s(buf_rsrc r, uint32_t off, uint32_t soff) {
    return {buf_load16s(r, off, soff), buf_load16s(r, off + 16u, soff)};
  }
  __device__ static __forceinline__ GTab group_table(uint32_t e) {
    // bf16 bits of the magnitudes at scale 1, in pairs; + (e - 127) << 7 on every nonzero one
    const uint16_t x = (uint16_t)((e - 127u) << 7);
    const u16x2 p0 = u16x2{0, 0x3F00} + u16x2{0, x};
    const u16x2 p1 = u16x2{0x3F80, 0x3FC0} + u16x2{x, x};
    const u16x2 p2 = u16x2{0x4000, 0x4040} + u16x2{x, x};
    const u16x2 p3 = u16x2{0x4080, 0x40C0} + u16x2{x, x};
    const uint32_t d0 = __builtin_bit_cast(uint32_t, p0), d1 = __builtin_bit_cast(uint32_t, p1);
    const uint32_t d2 = __builtin_bit_cast(uint32_t, p2), d3 = __builtin_bit_cast(uint32_t, p3);
    GTab t;
    t.hb0 = byte_perm(d1, d0, 0x07050301u);
    t.lb0 = byte_perm(d1, d0, 0x06040200u);
    t.hb1 = byte_perm(d3, d2, 0x07050301u);
    t.lb1 = byte_perm(d3, d2, 0x06040200u);
    return t;
  }
  // the step's scale bytes: group 0 in bits [0, 8), group 1 in bits [8, 16)
  __device__ static __forceinline__ Tab table(uint32_t sw) {
    Tab t;
    t.g[0] = group_table(sw & 0xFFu);
    t.g[1] = group_table((sw >> 8) & 0xFFu);
    return t;
  }
  template <int NB>
  __device__ static __forceinline__ uint32_t step_scale(const ScaleBytes<NB>& s, int step) {
    return (s.v[step >> 1] >> (16 * (step & 1))) & 0xFFFFu;
  }
  // four magnitudes (selector bytes) with their signs (bit 7 of each byte) -> two bf16 pairs
  __device__ static __forceinline__ void lookup(uint32_t m, uint32_t sg, const GTab& t, uint32_t& d0,
                                                uint32_t& d1) {
    const uint32_t hb = byte_perm(t.hb1, t.hb0, m) ^ sg, lb = byte_perm(t.lb1, t.lb0, m);
    d0 = byte_perm(hb, lb, 0x05010400u);
    d1 = byte_perm(hb, lb, 0x07030602u);
  }
  // operand o (0..7) of a step: 16-k block o / 2 (code dwords 2(o/2), 2(o/2)+1), slots 8(o%2) ..
  __device__ static __forceinline__ u32x4 decode(const Codes& c, const Tab& t, int o) {
    const int j = o >> 1;
    const uint32_t d_lo = j < 2 ? c.a[2 * j] : c.b[2 * j - 4];
    const uint32_t d_hi = j < 2 ? c.a[2 * j + 1] : c.b[2 * j - 3];
    const uint32_t g = byte_perm(d_hi, d_lo, (o & 1) ? 0x07050301u : 0x06040200u);
    const GTab& tb = t.g[j >> 1];
    uint32_t d0, d1, d2, d3;
    lookup(g & 0x07070707u, (g << 4) & 0x80808080u, tb, d0, d1);   // low nibbles
    lookup((g >> 4) & 0x07070707u, g & 0x80808080u, tb, d2, d3);  // high nibbles
    return u32x4{d0, d1, d2, d3};
  }
  __host__ __device__ static constexpr int pos32(int c) { return W2Fmt::pos32(c); }
  __host__ __device__ static constexpr int slot_k(int s) { return W2Fmt::slot_k(s); }
};


// x stored in the k-slot order of the weight format (the token operand of the low-bit FFN
// kernels), one chunk per thread:
//   2-bit: xp[t][16c + p] = x[t][16c + 4*(p%4) + p/4] for chunk c of 16 k (byte selects);
//   3-bit: xp[t][32c + s] = x[t][32c + slot_k(s)] for chunk c of 32 k.
__device__ __forceinline__ void x_chunk_to_slots(const uint4* __restrict__ x, int c, int fmt,
                                                 uint4* __restrict__ xp) {
  if (fmt == W2Fmt::kId) {
    const uint4 a = x[2 * c], b = x[2 * c + 1];  // dwords d0..d3 = a, d4..d7 = b
    constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;
    uint4 o0, o1;
    o0.x = byte_perm(a.z, a.x, LO);  // (x0, x4)
    o0.y = byte_perm(b.z, b.x, LO);  // (x8, x12)
    o0.z = byte_perm(a.z, a.x, HI);  // (x1, x5)
    o0.w = byte_perm(b.z, b.x, HI);  // (x9, x13)
    o1.x = byte_perm(a.w, a.y, LO);  // (x2, x6)
    o1.y = byte_perm(b.w, b.y, LO);  // (x10, x14)
    o1.z = byte_perm(a.w, a.y, HI);  // (x3, x7)
    o1.w = byte_perm(b.w, b.y, HI);  // (x11, x15)
    xp[2 * c] = o0;
    xp[2 * c + 1] = o1;
  } else {
    uint32_t in[16], o[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 v = x[4 * c + u];
      in[4 * u] = v.x;
      in[4 * u + 1] = v.y;
      in[4 * u + 2] = v.z;
      in[4 * u + 3] = v.w;
    }
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const int k0 = W3Fmt::slot_k(2 * d), k1 = W3Fmt::slot_k(2 * d + 1);
      const uint32_t lo = (in[k0 >> 1] >> (16 * (k0 & 1))) & 0xFFFFu;
      const uint32_t hi = (in[k1 >> 1] >> (16 * (k1 & 1))) & 0xFFFFu;
      o[d] = lo | (hi << 16);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) xp[4 * c + u] = make_uint4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3]);
  }
}

}  // namespace bitmoe
