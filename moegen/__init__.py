"""Seeded synthetic inputs for the low-bit MoE layer.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.  This module holds
none of the layer's arithmetic: it only draws random numbers and lays raw random bits
out in the packed storage formats (a uniformly random 32-bit word *is* sixteen
uniformly random 2-bit codes, so no packing logic is needed).  Decoding, routing and
every matmul live in the oracle and in the HIP library, never here.

Layers (shapes follow the five workloads the layer is exercised on):

========  =====  ===  =====  =====  ======  ============================================
name       E      k    H      I     format  routing / extra
========  =====  ===  =====  =====  ======  ============================================
tiny        8     2    256    512   2-bit   plain N(0,1) logits, T = 16
decode    384     8   4096   2048   2-bit   Zipf(s=1.1) logits, T = 1 / 8 / 64
prefill   384     8   4096   2048   2-bit   Zipf(s=1.1) logits, T = 8192 / 65536
mixed     384     8   4096   2048   2-bit   hottest 32 experts held in MXFP4, T = 4096
w3        512    10   2048    512   3-bit   Zipf(s=1.1) logits, T = 1 .. 4096
residual  384     8   4096   2048   2-bit   hottest 32 experts carry an MXFP4 residual
                                            (FP4 delta) on top of their 2-bit codes
========  =====  ===  =====  =====  ======  ============================================

Storage layouts (all row-major, K = reduction dim is contiguous):

* 2-bit:  ``codes u32[rows][K/16]``, ``scales u16[rows][K/32]`` (bf16 bit patterns)
* 3-bit:  ``codes u32[rows][K/32*3]``, ``scales u8[rows][K/64]`` (e4m3fn bytes)
* MXFP4:  ``codes u8[rows][K/2]``, ``scales u8[rows][K/32]`` (e8m0 bytes)
* W1 is ``[E][2I][H]`` (gate rows then up rows), W2 is ``[E][H][I]``.

Draws:

* x: N(0,1) in fp32, rounded to nearest-even bf16 (bit patterns, ``u16[T][H]``).
* logits: fp32 ``l[t,e] = z[t,e] - s*ln(rank[e])`` with z ~ N(0,1), s = 1.1 and
  ``rank`` a seeded permutation of 1..E (rank 1 = hottest); the tiny layer uses z alone.
* 2-bit codes: uniform 32-bit words.  2-bit scales: bf16 of sign * U(0.005, 0.02).
* 3-bit codes: uniform 32-bit words.  3-bit scales: e4m3fn bytes with random sign,
  biased exponent uniform in {5, 6, 7} and uniform mantissa, i.e. |scale|/64 in
  [0.0039, 0.0293] -- the same magnitude as the 2-bit scales, drawn as bytes so no
  e4m3 encoder is needed here.
* MXFP4: uniform nibbles (uniform bytes); e8m0 scale bytes uniform in {120, 121}.
* MXFP4 residual (residual layer): uniform nibbles; e8m0 scale bytes uniform in {116, 117}
  (2^-11, 2^-10: a correction about an order of magnitude below the 2-bit weights).
* Hot set (mixed and residual layers): the 32 experts of Zipf rank 1..32, hottest first.

Weights depend only on the layer (seed 1000 + layer index, then the expert id);
activations and logits also depend on T, so one layer serves every batch size.
"""
from __future__ import annotations

import numpy as np

LAYERS = {
    # name: (index, E, k, H, I, low-bit format, zipf exponent or None, n_hot, token counts)
    "tiny": (0, 8, 2, 256, 512, "w2", None, 0, (16,)),
    "decode": (1, 384, 8, 4096, 2048, "w2", 1.1, 0, (1, 8, 64)),
    "prefill": (2, 384, 8, 4096, 2048, "w2", 1.1, 0, (8192, 65536)),
    "mixed": (3, 384, 8, 4096, 2048, "w2", 1.1, 32, (4096,)),
    "w3": (4, 512, 10, 2048, 512, "w3", 1.1, 0, (1, 8, 64, 512, 4096)),
    "residual": (5, 384, 8, 4096, 2048, "w2", 1.1, 32, (1, 8, 64)),
}
# how the hot set is held: "replace" (the hot experts are MXFP4 instead of low-bit) or
# "residual" (their low-bit codes plus an MXFP4 residual)
HOT_MODE = {"mixed": "replace", "residual": "residual"}


def spec(name: str, **override) -> dict:
    """Shape and format of a layer as a dict; keyword overrides allow small variants."""
    idx, E, k, H, I, fmt, zipf, n_hot, Ts = LAYERS[name]
    d = dict(name=name, index=idx, E=E, k=k, H=H, I=I, fmt=fmt, zipf=zipf, n_hot=n_hot, Ts=Ts,
             hot_mode=HOT_MODE.get(name, "replace"))
    d.update(override)
    return d


def _rng(*words: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(w) for w in words]))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns the uint16 bit patterns.
    Inputs are finite, so the carry into the exponent is the correct result."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def zipf_ranks(sp: dict) -> np.ndarray:
    """rank[e] in 1..E (1 = hottest expert), a seeded permutation."""
    r = _rng(1000 + sp["index"], 7)
    return (r.permutation(sp["E"]) + 1).astype(np.int64)


def hot_ids(sp: dict) -> np.ndarray:
    """Expert ids of the hot set, hottest first (int32)."""
    if sp["n_hot"] == 0:
        return np.zeros(0, np.int32)
    ranks = zipf_ranks(sp)
    return np.argsort(ranks, kind="stable")[: sp["n_hot"]].astype(np.int32)


def _codes_scales(r: np.random.Generator, fmt: str, rows: int, K: int):
    if fmt == "w2":
        codes = r.integers(0, 2**32, size=(rows, K // 16), dtype=np.uint32)
        mag = r.uniform(0.005, 0.02, size=(rows, K // 32))
        sgn = np.where(r.integers(0, 2, size=mag.shape) == 1, -1.0, 1.0)
        scales = _f32_to_bf16_bits((sgn * mag).astype(np.float32))
        return codes, scales
    if fmt == "w3":
        codes = r.integers(0, 2**32, size=(rows, K // 32 * 3), dtype=np.uint32)
        sgn = r.integers(0, 2, size=(rows, K // 64), dtype=np.uint8)
        ex = r.integers(5, 8, size=(rows, K // 64), dtype=np.uint8)
        man = r.integers(0, 8, size=(rows, K // 64), dtype=np.uint8)
        scales = ((sgn << 7) | (ex << 3) | man).astype(np.uint8)
        return codes, scales
    if fmt in ("mxfp4", "mxfp4res"):
        codes = r.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
        lo = 120 if fmt == "mxfp4" else 116
        scales = r.integers(lo, lo + 2, size=(rows, K // 32), dtype=np.uint8)
        return codes, scales
    raise ValueError(fmt)


def expert(sp: dict, e: int, fmt: str | None = None) -> dict:
    """Packed weights of one expert: w1_codes/w1_scales ([2I] rows, K=H) and
    w2_codes/w2_scales ([H] rows, K=I).  ``fmt`` defaults to the layer's low-bit
    format; pass "mxfp4" for the hot-set copy of an expert, "mxfp4res" for its residual."""
    fmt = fmt or sp["fmt"]
    stream = {"w2": 1, "w3": 1, "mxfp4": 2, "mxfp4res": 4}[fmt]
    r = _rng(1000 + sp["index"], stream, e)
    H, I = sp["H"], sp["I"]
    c1, s1 = _codes_scales(r, fmt, 2 * I, H)
    c2, s2 = _codes_scales(r, fmt, H, I)
    return dict(w1_codes=c1, w1_scales=s1, w2_codes=c2, w2_scales=s2)


def weights(sp: dict) -> dict:
    """All experts stacked along a leading [E] axis (low-bit format), plus, for a layer
    with a hot set, ``hot_ids`` and the MXFP4 arrays stacked along [n_hot]."""
    E = sp["E"]
    first = expert(sp, 0)
    out = {key: np.empty((E,) + a.shape, a.dtype) for key, a in first.items()}
    for e in range(E):
        ex = first if e == 0 else expert(sp, e)
        for key, a in ex.items():
            out[key][e] = a
    hid = hot_ids(sp)
    out["hot_ids"] = hid
    if len(hid):
        hf = "mxfp4res" if sp.get("hot_mode") == "residual" else "mxfp4"
        h0 = expert(sp, int(hid[0]), hf)
        for key, a in h0.items():
            out["hot_" + key] = np.empty((len(hid),) + a.shape, a.dtype)
        for s, e in enumerate(hid):
            for key, a in expert(sp, int(e), hf).items():
                out["hot_" + key][s] = a
    return out


def batch(sp: dict, T: int) -> dict:
    """Router logits ``f32[T][E]`` and activations ``x`` (bf16 bits, ``u16[T][H]``)."""
    r = _rng(1000 + sp["index"], 3, T)
    z = r.standard_normal((T, sp["E"]), dtype=np.float32)
    if sp["zipf"] is None:
        logits = z
    else:
        pen = (sp["zipf"] * np.log(zipf_ranks(sp).astype(np.float64))).astype(np.float32)
        logits = (z - pen[None, :]).astype(np.float32)
    x = _f32_to_bf16_bits(r.standard_normal((T, sp["H"]), dtype=np.float32))
    return dict(logits=np.ascontiguousarray(logits), x=x)


def float_weights(rows: int, K: int, seed: int, spread: bool = True) -> np.ndarray:
    """Seeded fp32 float weights ``[rows][K]`` standing in for a trained expert matrix that is
    about to be quantised: N(0, 0.02^2), each row scaled by a factor 2^U(-3, 3) when `spread`
    (rows of different magnitude, as in real layers).  Random draws only."""
    r = _rng(2000, seed, rows, K)
    w = r.standard_normal((rows, K)) * 0.02
    if spread:
        w = w * np.exp2(r.uniform(-3.0, 3.0, size=(rows, 1)))
    return w.astype(np.float32)
