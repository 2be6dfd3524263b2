"""GPU: moe_route_permute_prepare (routing, grouping and the FFN's preparation in one launch up to
16 tokens, in two above: the route kernel, then the rest) gives the same bits as moe_route + moe_permute + stage 0 of moe_expert_ffn: the ids, gates,
counts, offsets, perm and inv, the whole FFN workspace after the preparation, and the layer
output once stages 1 .. n-1 and the combine have run.  The three-call path is checked against the
oracle by the parity tests at these layers and sizes."""
import pytest
import torch

import moegen

from _helpers import device_layer, to_dev

pytestmark = pytest.mark.gpu

FILL = 0xA5
MIXED_SMALL = {"E": 16, "k": 4, "H": 256, "I": 512, "n_hot": 4}


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


def _rest(L, dw, x, k, counts, offsets, perm, inv, gw, ws, T):
    n = L.moe_expert_ffn_num_stages(dw, T, k, ws.numel())
    y = torch.zeros((T * k, dw.H), dtype=torch.float32, device="cuda")
    for st in range(1, n):
        L.moe_expert_ffn_stage(dw, x, k, counts, offsets, perm, y, ws, st)
    return y, L.moe_combine(y, inv, gw, out_fp32=True)


@pytest.mark.parametrize("name,T,override", [("tiny", 1, {}), ("tiny", 16, {}), ("decode", 1, {}),
                                             ("decode", 3, {}), ("decode", 8, {}), ("decode", 16, {}),
                                             ("w3", 1, {}), ("w3", 16, {}), ("residual", 8, {}),
                                             ("mixed", 5, MIXED_SMALL), ("mixed", 16, {}),
                                             # two launches: 17 tokens, the decode batch, the
                                             # grouped-GEMM list (T >= 128), the largest batch
                                             # (R = T*k = 4096 rows)
                                             ("tiny", 100, {}), ("decode", 17, {}), ("decode", 64, {}),
                                             ("decode", 128, {}), ("decode", 512, {}), ("w3", 64, {}),
                                             ("residual", 64, {}), ("mixed", 64, MIXED_SMALL)])
def test_front_equals_three_calls(L, name, T, override):
    sp, dw = device_layer(name, **override)
    k = sp["k"]
    b = moegen.batch(sp, T)
    logits, x = to_dev(b["logits"]), to_dev(b["x"])
    nbytes = L.moe_expert_ffn_ws_bytes(dw, T, k)
    print(f"[front] {name} T={T} k={k} ws={nbytes}", flush=True)
    # three calls
    ids_a, gw_a = L.moe_route(logits, k)
    counts_a, offsets_a, perm_a, inv_a = L.moe_permute(ids_a, sp["E"])
    ws_a = torch.full((nbytes,), FILL, dtype=torch.uint8, device="cuda")
    y0 = torch.zeros((T * k, dw.H), dtype=torch.float32, device="cuda")
    L.moe_expert_ffn_stage(dw, x, k, counts_a, offsets_a, perm_a, y0, ws_a, 0)
    # one launch
    ws_b = torch.full((nbytes,), FILL, dtype=torch.uint8, device="cuda")
    ids_b, gw_b, counts_b, offsets_b, perm_b, inv_b = L.moe_route_permute_prepare(dw, logits, x, k, ws_b)
    torch.cuda.synchronize()
    for a, bb, what in ((ids_a, ids_b, "ids"), (gw_a.view(torch.int32), gw_b.view(torch.int32), "gates"),
                        (counts_a, counts_b, "counts"), (offsets_a, offsets_b, "offsets"), (perm_a, perm_b, "perm"),
                        (inv_a, inv_b, "inv")):
        assert torch.equal(a, bb), what
    assert torch.equal(ws_a, ws_b), "workspace after the preparation"
    y_a, out_a = _rest(L, dw, x, k, counts_a, offsets_a, perm_a, inv_a, gw_a, ws_a, T)
    y_b, out_b = _rest(L, dw, x, k, counts_b, offsets_b, perm_b, inv_b, gw_b, ws_b, T)
    torch.cuda.synchronize()
    assert torch.equal(y_a.view(torch.int32), y_b.view(torch.int32))
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32))


def test_front_empty_batch(L):
    sp, dw = device_layer("tiny")
    k = sp["k"]
    logits = torch.zeros((0, sp["E"]), dtype=torch.float32, device="cuda")
    x = torch.zeros((0, sp["H"]), dtype=torch.int16, device="cuda")
    ws = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    out = (torch.empty((0, k), dtype=torch.int32, device="cuda"), torch.empty((0, k), dtype=torch.float32, device="cuda"),
           torch.full((sp["E"],), 7, dtype=torch.int32, device="cuda"),
           torch.full((sp["E"] + 1,), 7, dtype=torch.int32, device="cuda"),
           torch.empty(0, dtype=torch.int32, device="cuda"), torch.empty(0, dtype=torch.int32, device="cuda"))
    _, _, counts, offsets, _, _ = L.moe_route_permute_prepare(dw, logits, x, k, ws, out=out)
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0
