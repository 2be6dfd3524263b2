"""GPU: moe_expert_ffn with the hot experts' preparation and MXFP4 -> FP8 conversion on a
second stream, concurrent with the low-bit stages ([Day0-MXFP4] section 4: the conversion of the next
experts runs on another stream while the current ones compute).  Same kernels on the same inputs: the output must be bit-equal to the
one-stream call, eagerly and replayed from a HIP graph."""
import pytest
import torch

import moegen

from _helpers import device_layer, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


MIXED_SMALL = {"E": 16, "k": 4, "H": 256, "I": 512, "n_hot": 4}


def _inputs(L, name, T, override):
    sp, dw = device_layer(name, **override)
    b = moegen.batch(sp, T)
    ids, _ = L.moe_route(to_dev(b["logits"]), sp["k"])
    counts, offsets, perm, inv = L.moe_permute(ids, sp["E"])
    return sp, dw, to_dev(b["x"]), counts, offsets, perm


@pytest.mark.parametrize("name,T,override,slots", [("mixed", 1, MIXED_SMALL, None), ("mixed", 100, MIXED_SMALL, None),
                                                   ("mixed", 300, MIXED_SMALL, 1), ("mixed", 256, {}, None),
                                                   ("mixed", 64, {}, 8), ("decode", 64, {}, None)])
def test_two_streams_equal_one_stream(L, name, T, override, slots):
    sp, dw, x, counts, offsets, perm = _inputs(L, name, T, override)
    k = sp["k"]
    nbytes = L.moe_expert_ffn_ws_bytes(dw, T, k, slots or 0)
    ws1 = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws1)
    print(f"{name} T={T} slots={slots}", flush=True)
    y1 = L.moe_expert_ffn(dw, x, k, counts, offsets, perm, ws=ws1)
    y2 = torch.full_like(y1, float("nan"))
    side = torch.cuda.Stream()
    L.moe_expert_ffn_two_streams(dw, x, k, counts, offsets, perm, y2, ws2, side)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_two_streams_graph_replay(L):
    sp, dw, x, counts, offsets, perm = _inputs(L, "mixed", 200, MIXED_SMALL)
    k = sp["k"]
    ws = torch.empty(L.moe_expert_ffn_ws_bytes(dw, 200, k, 0), dtype=torch.uint8, device="cuda")
    want = L.moe_expert_ffn(dw, x, k, counts, offsets, perm)
    y = torch.zeros_like(want)
    side = torch.cuda.Stream()
    L.moe_expert_ffn_two_streams(dw, x, k, counts, offsets, perm, y, ws, side)  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.moe_expert_ffn_two_streams(dw, x, k, counts, offsets, perm, y, ws, side)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), want.view(torch.int32)), rep
