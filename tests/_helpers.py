"""Shared helpers of the GPU tests: device layers from the seeded generator, and the
oracle-side view of the same layer."""
from __future__ import annotations

import functools
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import moegen
from oracle import formats as OF
from oracle import moe as OM

FMT = {"w2": 1, "w3": 2}


@functools.lru_cache(maxsize=4)
def layer_arrays(name: str, **override):
    sp = moegen.spec(name, **override)
    return sp, moegen.weights(sp)


def device_layer(name: str, **override):
    from bit_moe_expert_top_amd import _lib as L

    sp, arrays = layer_arrays(name, **override)
    flags = L.MOE_FLAG_HOT_RESIDUAL if sp["hot_mode"] == "residual" else 0
    return sp, L.DeviceWeights(FMT[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, flags=flags)


def oracle_layer(name: str, **override):
    sp, arrays = layer_arrays(name, **override)
    return OM.Layer(sp["fmt"], arrays, hot_mode=sp["hot_mode"])


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_bits_host(t: torch.Tensor) -> np.ndarray:
    return host(t).view(np.uint16)


def max_err_over_rms(got, want) -> float:
    want = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - want)) / rms)


TOL_BF16 = 2e-2   # max |gpu - oracle| <= 2e-2 * rms(oracle) for bf16-computed layers
TOL_FP8 = 6e-2    # ... and 6e-2 * rms for layers with FP8 (MXFP8) experts, at the layer's own shape

# The FP8 matrix cores' dot products are not IEEE fp32 sums: one v_mfma_scale_f32_32x32x64_f8f6f4
# on random e4m3 operands deviated from the exact sum of its products by up to 3.2e-4 of the rms
# of such sums (measured on the device).  KAPPA bounds that deviation relative to
# sqrt(sum of squared products), with a factor of three to spare.
KAPPA = 1e-3


def fp8_h_bound(Xq, W1):
    """The oracle's h = SwiGLU(FC1) (fp64) for MXFP8 rows Xq of an FP8 expert, and a
    first-order bound of how far a computation whose FC1 sums carry an error of at most
    KAPPA * sqrt(sum of squared products) can move h: |dh| <= |silu'(g)| |u| dg + |silu(g)| du."""
    I = W1.shape[0] // 2
    a = OM.fc1(Xq, W1)
    s = np.sqrt(OM.fc1(Xq * Xq, W1 * W1))
    g, u = a[:, :I], a[:, I:]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    dh = KAPPA * (np.abs(dsilu * u) * s[:, :I] + np.abs(g * sig) * s[:, I:])
    return OM.swiglu(a), dh


def _e4m3_at_scale(v, shared):
    """The MXFP8 value of v with the given shared exponent (per element)."""
    return OF.e4m3fn_value(OF.e4m3fn_encode(v / np.exp2(shared))) * np.exp2(shared)


def mxfp8_flip_allowance(h, dh):
    """For rows h (f64[n][I]) and their bound dh: the oracle's MXFP8 values q of h, and per
    element the largest |q' - q| over the values q' that an h' with |h' - h| <= dh can give.  An
    element may round to the other side of an e4m3 midpoint; where the block's amax lies within
    its dh of a power of two, the whole block may take the neighbouring shared exponent."""
    n, I = h.shape
    el, sc = OF.mxfp8_quantize(h)
    q = OF.mxfp8_dequant(el, sc)
    E = np.repeat(sc.astype(np.float64) - 127.0, 32, axis=1)
    allow = np.maximum(np.abs(_e4m3_at_scale(h - dh, E) - q), np.abs(_e4m3_at_scale(h + dh, E) - q))
    hb = np.abs(h).reshape(n, I // 32, 32)
    am = hb.max(-1)
    dam = dh.reshape(n, I // 32, 32)[np.arange(n)[:, None], np.arange(I // 32)[None, :], hb.argmax(-1)]
    lo = np.floor(np.log2(np.maximum(am - dam, 1e-300)))
    hi = np.floor(np.log2(np.maximum(am + dam, 1e-300)))
    for r, b in zip(*np.nonzero((am > 0) & (lo != hi))):
        cols = slice(32 * b, 32 * b + 32)
        for dE in (-1.0, 1.0):
            for v in (h[r, cols] - dh[r, cols], h[r, cols] + dh[r, cols]):
                allow[r, cols] = np.maximum(allow[r, cols], np.abs(_e4m3_at_scale(v, E[r, cols] + dE) - q[r, cols]))
    return q, allow


def fp8_expert_rows(X, W1, W2):
    """The oracle's FFN of one FP8 expert on bf16-valued rows X (x and h quantised to MXFP8,
    as swiglu_ffn computes it), and per output element the allowance that the h elements'
    possible rounding flips carry through FC2: sum_j allow_j |W2[i, j]|."""
    h, dh = fp8_h_bound(OM.mxfp8_round_trip(X), W1)
    q, allow = mxfp8_flip_allowance(h, dh)
    return OM.fc2(q, W2), OM.fc2(allow, np.abs(W2))


def oracle_token_rows(lay, x_bits, ids, toks, k: int, threads: int = 8, allowance: dict | None = None) -> dict:
    """The oracle's expert outputs for the routed rows of the sampled tokens only:
    {(t, j): f64[H]} with y = FFN of expert ids[t, j] on token t.  Each expert's matrices are
    decoded once, experts in parallel (for sampled checks of large batches).  With a dict
    ``allowance``, the rows of FP8 experts also get their rounding-flip allowance there."""
    X = OF.bf16_value(x_bits)
    by_e: dict = {}
    for t in toks:
        for j in range(k):
            by_e.setdefault(int(ids[t, j]), []).append((int(t), j))

    def run(e):
        rows = by_e[e]
        Xr = X[[t for t, _ in rows]]
        if allowance is not None and lay.is_fp8(e):
            y, a = fp8_expert_rows(Xr, lay.dense(e, 1), lay.dense(e, 2))
            return rows, y, a
        return rows, OM.swiglu_ffn(Xr, lay.dense(e, 1), lay.dense(e, 2), lay.is_fp8(e)), None

    out = {}
    with ThreadPoolExecutor(threads) as ex:
        for rows, y, a in ex.map(run, list(by_e)):
            for i, tj in enumerate(rows):
                out[tj] = y[i]
                if a is not None:
                    allowance[tj] = a[i]
    return out


def oracle_fp8_allowance(lay, x_bits, k: int, offsets, perm, E: int, H: int) -> np.ndarray:
    """f64[T*k][H]: the rounding-flip allowance of every grouped row (0 for the rows of
    experts that do not compute in FP8)."""
    X = OF.bf16_value(x_bits)
    allow = np.zeros((len(perm), H))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0 and lay.is_fp8(e):
            allow[r0:r1] = fp8_expert_rows(X[perm[r0:r1] // k], lay.dense(e, 1), lay.dense(e, 2))[1]
    return allow


def max_err_beyond(got, want, allow) -> float:
    """max(|got - want| - allow) / rms(want): the error left once each element's allowance is
    taken off."""
    want = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - want) - allow) / rms)


def sample_tokens(T: int, n: int = 256, seed: int = 0) -> np.ndarray:
    """n distinct tokens of a batch of T (always the first and the last), seeded."""
    if T <= n:
        return np.arange(T)
    r = np.random.default_rng(seed + T)
    mid = r.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))
