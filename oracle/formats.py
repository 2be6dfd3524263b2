"""Element and weight formats of the oracle (fp64 values from packed bytes).

Test infrastructure only (see the package docstring).  Every decoder follows a format
definition, element by element; none is shared with the HIP library.
"""
from __future__ import annotations

import numpy as np

# [Moet-QA] section on 2-bit expert quantisation: experts use the sign-symmetric
# 4-level codebook {-4, -1, 1, 4}.  Reading: code c = 0, 1, 2, 3 selects the levels
# in the listed (ascending) order.
W2_LEVELS = np.array([-4.0, -1.0, 1.0, 4.0])

# [Strata-R9700] path 6: the 3-bit expert format has the 8 levels below, code c = 0..7
# selects them in the listed order.
W3_LEVELS = np.array([-8.0, -5.0, -3.0, -1.0, 1.0, 3.0, 5.0, 8.0])

# [OCP-MX] e2m1 magnitudes for the 3 low bits of a nibble; bit 3 is the sign.
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

E4M3_MAX = 448.0


# ---------------------------------------------------------------- element decoders
def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64: the bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_value(byte) -> np.ndarray:
    """[OCP-MX] e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN."""
    b = np.asarray(byte, dtype=np.uint8).astype(np.int64)
    s = np.where(b >> 7 == 1, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0**-6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (b & 7 == 7), np.nan, mag)
    return s * mag


def e8m0_value(byte) -> np.ndarray:
    """[OCP-MX] e8m0 scale: 2^(b - 127); 255 is NaN."""
    b = np.asarray(byte, dtype=np.uint8).astype(np.float64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def e2m1_value(nibble) -> np.ndarray:
    """[OCP-MX] e2m1 nibble: bit 3 sign, bits 0-2 index the magnitudes 0..6."""
    n = np.asarray(nibble, dtype=np.uint8).astype(np.int64)
    s = np.where((n >> 3) & 1 == 1, -1.0, 1.0)
    return s * E2M1_MAG[n & 7]


# ---------------------------------------------------------------- element encoder
def e4m3fn_encode(v) -> np.ndarray:
    """fp64 -> e4m3fn byte, round to nearest, ties to even, saturating at +-448
    (the [OCP-MX] saturating conversion).  Keeps the sign of zero.  Inputs are finite.

    Written from the encoding: find the binade of |v|, round |v| to a multiple of that
    binade's step (2^-9 below 2^-6), and place exponent and mantissa fields."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v)), "e4m3fn_encode: non-finite input"
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    _, ex = np.frexp(a)                         # a = f * 2^ex, f in [0.5, 1)
    e_unb = ex.astype(np.int64) - 1             # floor(log2 a) for a > 0
    sub = (a < 2.0**-6)
    step = np.where(sub, 2.0**-9, np.exp2(e_unb - 3.0))
    q = np.round(a / step)                      # numpy rounds half to even
    val = q * step                              # rounded magnitude (exact)
    val = np.minimum(val, E4M3_MAX)
    # fields of the rounded magnitude
    _, ex2 = np.frexp(val)
    e2 = ex2.astype(np.int64) - 1
    is_sub = val < 2.0**-6
    mant_sub = np.round(val / 2.0**-9).astype(np.int64)                  # 0..7
    mant_nrm = np.round((val / np.exp2(e2.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    field = np.where(is_sub, mant_sub, ((e2 + 7) << 3) | mant_nrm)
    return ((sign << 7) | field).astype(np.uint8)


# ---------------------------------------------------------------- weight formats
def dequant_w2(codes, scales) -> np.ndarray:
    """2-bit codebook weights -> fp64 ``[rows][K]``.

    codes ``u32[rows][K/16]``: code i of a word sits at bits [2i, 2i+2) (LSB first;
    reading: sixteen codes per 32-bit word, in K order); level = ``W2_LEVELS[code]``.
    scales ``u16[rows][K/32]`` (bf16): one scale per 32 consecutive weights along K of
    one row.  Weight = level * scale ([Moet-QA] codebook; group-32 bf16 scales)."""
    codes = np.asarray(codes, dtype=np.uint32)
    rows, nw = codes.shape
    shifts = (2 * np.arange(16)).astype(np.uint32)
    c = (codes[:, :, None] >> shifts[None, None, :]) & np.uint32(3)
    lev = W2_LEVELS[c.reshape(rows, nw * 16).astype(np.int64)]
    s = np.repeat(bf16_value(scales), 32, axis=1)
    assert s.shape == lev.shape
    return lev * s


def unpack_w3_codes(codes) -> np.ndarray:
    """3-bit codes ``u32[rows][K/32*3]`` -> ``int[rows][K]``.  [Strata-R9700] path 6:
    32 codes in three 32-bit words.  Reading: the three words are one little-endian
    96-bit field (word j holds bits 32j..32j+31) and code i occupies bits [3i, 3i+3),
    so codes 10 and 21 straddle a word boundary."""
    codes = np.asarray(codes, dtype=np.uint32)
    rows, nw = codes.shape
    assert nw % 3 == 0
    g = codes.reshape(rows, nw // 3, 3).astype(np.uint64)
    out = np.empty((rows, nw // 3, 32), dtype=np.int64)
    for i in range(32):
        bit = 3 * i
        w, off = bit // 32, bit % 32
        v = g[:, :, w] >> np.uint64(off)
        if off + 3 > 32:
            v = v | (g[:, :, w + 1] << np.uint64(32 - off))
        out[:, :, i] = (v & np.uint64(7)).astype(np.int64)
    return out.reshape(rows, nw // 3 * 32)


def dequant_w3(codes, scales) -> np.ndarray:
    """3-bit 8-level weights -> fp64 ``[rows][K]``.  [Strata-R9700] path 6: levels
    ``W3_LEVELS``, "e4m3 scale/64".  Reading: one e4m3fn scale byte per 64 consecutive
    weights along K of one row, and weight = level * e4m3(scale) / 64."""
    lev = W3_LEVELS[unpack_w3_codes(codes)]
    s = np.repeat(e4m3fn_value(scales) / 64.0, 64, axis=1)
    assert s.shape == lev.shape
    return lev * s


def unpack_e2m1_nibbles(codes) -> np.ndarray:
    """MXFP4 codes ``u8[rows][K/2]`` -> nibbles ``[rows][K]``; element 2i is the low
    nibble of byte i (reading: the usual packed-fp4 order)."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, nb = codes.shape
    out = np.empty((rows, 2 * nb), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def dequant_mxfp4(codes, scales) -> np.ndarray:
    """MXFP4 weights -> fp64: e2m1 element times the e8m0 scale of its 32-block along K
    ([Moet-README]: the checkpoint's experts are MXFP4; [OCP-MX] for the encoding)."""
    v = e2m1_value(unpack_e2m1_nibbles(codes))
    s = np.repeat(e8m0_value(scales), 32, axis=1)
    assert s.shape == v.shape
    return v * s


def mxfp4_to_fp8(codes, scales):
    """[Day0-MXFP4] section 4: an expert held in MXFP4 is converted to FP8 just before it
    is used.  Reading: each e2m1 element becomes the e4m3fn byte of the *same value*
    (every e2m1 value, including -0, is exact in e4m3fn), laid out one byte per element
    ``u8[rows][K]``, and the e8m0 block scales are kept unchanged, so the converted
    expert is the same MX-scaled tensor in an FP8 element type (lossless)."""
    elems = e4m3fn_encode(e2m1_value(unpack_e2m1_nibbles(codes)))
    return elems, np.array(scales, dtype=np.uint8, copy=True)


def dequant_fp8(elems, scales) -> np.ndarray:
    """MX-scaled FP8 tensor (e4m3fn bytes ``[rows][K]``, e8m0 per 32 along K) -> fp64."""
    v = e4m3fn_value(elems)
    s = np.repeat(e8m0_value(scales), 32, axis=1)
    assert s.shape == v.shape
    return v * s


# ---------------------------------------------------------------- MXFP8 activations
def mxfp8_quantize(v):
    """[Moet-README] release notes of -r23: the prefill MoE quantises the SwiGLU output
    to MXFP8 before FC2; FP8 experts need FP8 activations into FC1 too (reading).

    [OCP-MX] conversion, blocks of 32 along the last axis: the shared exponent is
    floor(log2(max|v|)) - 8 (8 = the largest e4m3 exponent), each element is
    v / 2^shared rounded to e4m3fn (nearest-even, saturating).  An all-zero block gets
    scale byte 0.  Returns (element bytes ``u8[..., K]``, scale bytes ``u8[..., K/32]``)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % 32 == 0
    blk = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(amax)
    shared = np.where(amax > 0, ex.astype(np.int64) - 1 - 8, -127)
    shared = np.clip(shared, -127, 127)
    sbyte = (shared + 127).astype(np.uint8)
    scaled = blk / np.exp2(shared.astype(np.float64))[..., None]
    elems = e4m3fn_encode(scaled).reshape(v.shape)
    return elems, sbyte


def mxfp8_dequant(elems, sbytes) -> np.ndarray:
    """Inverse of ``mxfp8_quantize``'s encoding: e4m3fn value times 2^(scale-127)."""
    e = np.asarray(elems)
    K = e.shape[-1]
    val = e4m3fn_value(e).reshape(e.shape[:-1] + (K // 32, 32))
    return (val * e8m0_value(sbytes)[..., None]).reshape(e.shape)
