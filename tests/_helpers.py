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
TOL_FP8 = 6e-2    # ... and 6e-2 * rms for layers with FP8 (MXFP8) experts


def oracle_token_rows(lay, x_bits, ids, toks, k: int, threads: int = 8) -> dict:
    """The oracle's expert outputs for the routed rows of the sampled tokens only:
    {(t, j): f64[H]} with y = FFN of expert ids[t, j] on token t.  Each expert's matrices are
    decoded once, experts in parallel (for sampled checks of large batches)."""
    X = OF.bf16_value(x_bits)
    by_e: dict = {}
    for t in toks:
        for j in range(k):
            by_e.setdefault(int(ids[t, j]), []).append((int(t), j))

    def run(e):
        rows = by_e[e]
        y = OM.swiglu_ffn(X[[t for t, _ in rows]], lay.dense(e, 1), lay.dense(e, 2), lay.is_fp8(e))
        return rows, y

    out = {}
    with ThreadPoolExecutor(threads) as ex:
        for rows, y in ex.map(run, list(by_e)):
            for tj, v in zip(rows, y):
                out[tj] = v
    return out


def sample_tokens(T: int, n: int = 256, seed: int = 0) -> np.ndarray:
    """n distinct tokens of a batch of T (always the first and the last), seeded."""
    if T <= n:
        return np.arange(T)
    r = np.random.default_rng(seed + T)
    mid = r.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))
