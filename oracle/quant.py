"""Quantisers of the oracle: float weights -> the packed expert formats.

Test infrastructure only (see the package docstring).  The pages give the 2-bit codebook
({-4, -1, 1, 4}, [Moet-QA] section on 2-bit expert quantisation) and judge low-bit experts
by how close they stay to the float weights ([Strata-R9700], the post comparing 3-bit and
2-bit experts by cosine similarity), but they do not say how codes and scales are chosen.
Reading taken here: per group (32 consecutive weights along K of one row, the format's
scale group), the least-squares fit of ``w ~ level[code] * s``, found the standard way by
alternating the two optimal half-steps (Lloyd iterations):

* codes for a fixed scale: the nearest level of ``w / s``;
* scale for fixed codes: ``s = sum(level * w) / sum(level^2)``.

It starts from ``s = max|w| / 4`` (the largest weight on the outer level), runs three
rounds, rounds the scale to bf16 (round to nearest even; the format stores bf16) and
assigns the final codes against that stored scale.  Every decision that picks an integer
(a code) or a stored value (the scale) is taken in fp32, in a fixed order, so the HIP
quantiser must reproduce it bit for bit: products ``level * w`` are exact (levels are +-1
and +-4), sums run k = 0..31 in order, ``2.5 * s`` and ``num / den`` are single IEEE fp32
roundings.  Nearest-level rule on fp32 ``w`` with ``t = 2.5 * s``: code 3 (+4) if w > t,
code 2 (+1) if 0 <= w <= t (so -0 and ties at +-t go to the smaller magnitude), code 1
(-1) if -t <= w < 0, code 0 (-4) if w < -t.  An all-zero group gets scale 0 and code 2.

MXFP4 ([OCP-MX] conversion, block 32 along K): shared exponent floor(log2(max|w|)) - 2
(2 = the largest e2m1 exponent), each element ``w / 2^shared`` rounded to the nearest e2m1
value, ties to the even mantissa, saturating at +-6; an all-zero block gets scale byte 0
(the same reading as the MXFP8 activations).

Inputs are finite fp32 arrays ``[rows][K]`` with K a multiple of 32.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_MAG

W2_ROUNDS = 3
# level of code c (the [Moet-QA] codebook in ascending order); kept apart from
# formats.W2_LEVELS on purpose: these are the fp32 multipliers the fit uses
_LEV32 = np.array([-4.0, -1.0, 1.0, 4.0], dtype=np.float32)


def bf16_rne_bits(v) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def w2_assign(w32: np.ndarray, s32: np.ndarray) -> np.ndarray:
    """Nearest codebook level of w / s for every weight (fp32 thresholds, see module doc).
    w32 ``f32[G][32]``, s32 ``f32[G]`` -> codes ``int[G][32]``."""
    t = (np.float32(2.5) * s32).astype(np.float32)[:, None]
    return np.where(w32 > t, 3, np.where(w32 >= 0, 2, np.where(w32 >= -t, 1, 0)))


def w2_refit(w32: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Least-squares scale for fixed codes, fp32, sums in k order."""
    lev = _LEV32[codes]
    num = np.zeros(w32.shape[0], dtype=np.float32)
    den = np.zeros(w32.shape[0], dtype=np.float32)
    for i in range(32):
        num = (num + lev[:, i] * w32[:, i]).astype(np.float32)
        den = (den + lev[:, i] * lev[:, i]).astype(np.float32)
    return (num / den).astype(np.float32)


def quantize_w2(w) -> tuple[np.ndarray, np.ndarray]:
    """fp32 ``[rows][K]`` -> (codes ``u32[rows][K/16]``, bf16 scales ``u16[rows][K/32]``)."""
    w32 = np.asarray(w, dtype=np.float32)
    rows, K = w32.shape
    assert K % 32 == 0 and np.all(np.isfinite(w32))
    g = w32.reshape(rows * K // 32, 32)
    amax = np.max(np.abs(g), axis=1).astype(np.float32)
    s = (amax / np.float32(4.0)).astype(np.float32)
    for _ in range(W2_ROUNDS):
        c = w2_assign(g, s)
        s = np.where(amax > 0, w2_refit(g, c), np.float32(0.0)).astype(np.float32)
    sb = bf16_rne_bits(s)
    sq = (sb.astype(np.uint32) << 16).view(np.float32)
    c = w2_assign(g, sq)
    c = np.where(amax[:, None] > 0, c, 2)
    words = np.zeros((g.shape[0], 2), dtype=np.uint64)
    for i in range(32):
        words[:, i // 16] |= c[:, i].astype(np.uint64) << np.uint64(2 * (i % 16))
    return words.astype(np.uint32).reshape(rows, K // 16), sb.reshape(rows, K // 32)


def e2m1_round(x) -> np.ndarray:
    """Magnitude-and-sign rounding of fp64 x to the nearest e2m1 value, ties to the even
    mantissa, saturating at 6; returns the nibble (bit 3 = sign of x, -0 keeps its sign)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    # candidates below and above: distances to every magnitude, nearest, then ties
    d = np.abs(a[..., None] - E2M1_MAG)
    best = np.min(d, axis=-1, keepdims=True)
    cand = d == best
    # among tied candidates take the one with an even mantissa field (index bit 0 == 0)
    idx = np.arange(8)
    even = cand & (idx % 2 == 0)
    pick = np.where(np.any(even, axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    sign = np.signbit(x).astype(np.uint8)
    return ((sign << 3) | pick.astype(np.uint8)).astype(np.uint8)


def quantize_mxfp4(w) -> tuple[np.ndarray, np.ndarray]:
    """fp32 ``[rows][K]`` -> (codes ``u8[rows][K/2]`` low nibble first, e8m0 ``u8[rows][K/32]``)."""
    w32 = np.asarray(w, dtype=np.float32)
    rows, K = w32.shape
    assert K % 32 == 0 and np.all(np.isfinite(w32))
    blk = w32.astype(np.float64).reshape(rows, K // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(amax)
    shared = np.where(amax > 0, ex.astype(np.int64) - 1 - 2, -127)
    shared = np.clip(shared, -127, 127)
    nib = e2m1_round(blk / np.exp2(shared.astype(np.float64))[..., None]).reshape(rows, K)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, (shared + 127).astype(np.uint8)
