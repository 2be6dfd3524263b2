"""Shared helpers of the GPU tests: device layers from the seeded generator, and the
oracle-side view of the same layer."""
from __future__ import annotations

import functools

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
    return sp, L.DeviceWeights(FMT[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays)


def oracle_layer(name: str, **override):
    sp, arrays = layer_arrays(name, **override)
    return OM.Layer(sp["fmt"], arrays)


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
