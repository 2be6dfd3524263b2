"""GPU: moe_expert_ffn_noalloc (the library's static workspace, no allocation) gives the same
y_perm, bit for bit, as moe_expert_ffn with a caller workspace of the same size -- on two calls
in a row, the second with a smaller batch (the array keeps the first call's contents) -- and
rejects a batch whose workspace exceeds the static size.  Called through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import moegen
from oracle import moe as OM

from _helpers import device_layer, host, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


def _pair(L, dw, sp, T):
    b = moegen.batch(sp, T)
    k = sp["k"]
    ids, _ = OM.route(b["logits"], k)
    counts, offsets, perm, _ = L.moe_permute(to_dev(ids), sp["E"])
    x = to_dev(b["x"])
    y_ref = torch.full((T * k, sp["H"]), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    L.moe_expert_ffn(dw, x, k, counts, offsets, perm, y_perm=y_ref, ws=ws)
    y = torch.full_like(y_ref, float("nan"))
    L.moe_expert_ffn_noalloc(dw, x, k, counts, offsets, perm, y)
    torch.cuda.synchronize()
    return host(y), host(y_ref)


@pytest.mark.parametrize("name,Ts,override", [("tiny", (300, 7), {}), ("decode", (64, 1), {}),
                                              ("w3", (200, 3), {"E": 8, "k": 2, "H": 256, "I": 512}),
                                              ("mixed", (100, 16), {"E": 16, "k": 4, "H": 256, "I": 512, "n_hot": 4})])
def test_noalloc_matches_workspace_call(L, name, Ts, override):
    sp, dw = device_layer(name, **override)
    for T in Ts:  # the second call is smaller than the first
        y, y_ref = _pair(L, dw, sp, T)
        assert not np.isnan(y_ref).any()
        np.testing.assert_array_equal(y, y_ref, err_msg=f"{name} T={T}")


def test_noalloc_rejects_batches_beyond_the_static_workspace(L):
    sp, dw = device_layer("decode")
    T = 2048  # x in k-slot order 16 MiB alone: more than the static workspace
    assert L.moe_expert_ffn_ws_bytes(dw, T, sp["k"], 1) > L.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, sp["H"]), dtype=torch.int16, device="cuda")
    i = torch.zeros(sp["E"] + 1, dtype=torch.int32, device="cuda")
    p = torch.zeros(T * sp["k"], dtype=torch.int32, device="cuda")
    y = torch.zeros((1, 1), dtype=torch.float32, device="cuda")
    st = L.lib.moe_expert_ffn_noalloc(ctypes.byref(dw.c), x.data_ptr(), T, sp["k"], i.data_ptr(), i.data_ptr(),
                                      p.data_ptr(), y.data_ptr(), None)
    assert st == -3  # MOE_ERR_WORKSPACE, nothing enqueued
