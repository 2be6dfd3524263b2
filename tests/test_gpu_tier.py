"""GPU: the host-RAM expert tier.  [Moet-QA] (GPU as a cache of hot experts over host RAM) and
[Moet-README] (an LRU over a slot budget).

The experts live in pinned host memory and n_slots of them on the GPU; a batch runs on the
slots after its missing experts are copied in.  Each row's arithmetic is the same as with every
expert resident, so the tiered layer must give the resident layer's output bit for bit, over a
sequence of batches with misses and evictions; the slots must hold the host bytes exactly; and
the output must match the fp64 oracle within the layer tolerance."""
import numpy as np
import pytest
import torch

import moegen
from oracle import moe as OM

from _helpers import FMT, TOL_BF16, device_layer, host, layer_arrays, max_err_over_rms, oracle_layer, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


KEYS = ("w1_codes", "w1_scales", "w2_codes", "w2_scales")

# (layer, overrides, slots, tokens per batch): T * k <= slots, so every batch fits the budget
CASES = [("tiny", {}, 4, 2), ("decode", {}, 64, 8), ("w3", {"E": 16}, 12, 1), ("decode", {}, 8, 1)]


@pytest.mark.parametrize("name,override,slots,T", CASES)
def test_tiered_layer_matches_resident(L, name, override, slots, T):
    sp, arrays = layer_arrays(name, **override)
    _, dw = device_layer(name, **override)
    tl = L.TieredLayer(FMT[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, slots)
    k = sp["k"]
    nb = 12
    pool = moegen.batch(sp, nb * T)
    lg_all, x_all = to_dev(pool["logits"]), to_dev(pool["x"])
    loads = []
    for b in range(nb):
        lg, x = lg_all[b * T:(b + 1) * T].contiguous(), x_all[b * T:(b + 1) * T].contiguous()
        print(f"{name} slots={slots}: batch {b} (T={T})", flush=True)
        got = tl.forward(lg, x, k)
        want = L.layer_forward(dw, lg, x, k)
        assert torch.equal(got["ids"], want["ids"])
        assert torch.equal(got["out"].view(torch.int32), want["out"].view(torch.int32)), f"batch {b}"
        loads.append(got["n_load"])
        # every routed id maps to the slot that holds it
        sids, ids = host(got["slot_ids"]), host(got["ids"])
        assert np.array_equal(tl.state.expert_of_slot[sids], ids)
    # the slots hold the host bytes of their experts, bit for bit
    for s, e in enumerate(tl.state.expert_of_slot.tolist()):
        if e >= 0:
            for key in KEYS:
                assert torch.equal(tl.slot[key][s].cpu(), tl.host[key][e]), (key, s, e)
    print(f"{name}: experts loaded per batch {loads}", flush=True)
    assert tl.loaded == sum(loads) and loads[0] > 0


def test_tiered_layer_matches_oracle(L):
    sp, arrays = layer_arrays("decode")
    lay = oracle_layer("decode")
    tl = L.TieredLayer(FMT[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, 32)
    k, T = sp["k"], 4
    b = moegen.batch(sp, T)
    res = tl.forward(to_dev(b["logits"]), to_dev(b["x"]), k)
    ids, gates = OM.route(b["logits"], k)
    counts, offsets, perm, inv = OM.permute(ids, sp["E"])
    y = OM.expert_ffn(lay, b["x"], k, offsets, perm, experts=sorted(set(ids.reshape(-1).tolist())))
    want = OM.combine(np.nan_to_num(y), inv, gates, T, k)
    err = max_err_over_rms(host(res["out"]), want)
    print(f"tiered decode T={T}: max|err|/rms = {err:.4g}", flush=True)
    assert err <= TOL_BF16


def test_remap_bit_exact(L):
    rng = np.random.default_rng(5)
    E = 384
    table = rng.permutation(E).astype(np.int32)
    ids = rng.integers(0, E, size=(1000, 8)).astype(np.int32)
    got = L.moe_tier_remap(to_dev(ids), to_dev(table))
    np.testing.assert_array_equal(host(got), table[ids])


def test_batch_over_the_slot_budget_is_refused(L):
    sp, arrays = layer_arrays("tiny")
    tl = L.TieredLayer(FMT[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, 2)
    b = moegen.batch(sp, 16)
    with pytest.raises(L.MoeError):
        tl.forward(to_dev(b["logits"]), to_dev(b["x"]), sp["k"])
    assert tl.state.tick == 0 and tl.loaded == 0


def test_tiered_empty_batch(L):
    sp, arrays = layer_arrays("tiny")
    tl = L.TieredLayer(FMT[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, 4)
    x = torch.zeros((0, sp["H"]), dtype=torch.int16, device="cuda")
    lg = torch.zeros((0, sp["E"]), dtype=torch.float32, device="cuda")
    res = tl.forward(lg, x, sp["k"])
    assert res["out"].shape == (0, sp["H"]) and res["n_load"] == 0 and tl.loaded == 0


@pytest.mark.parametrize("name,override,slots,T", [("decode", {}, 24, 1), ("decode", {}, 96, 4),
                                                   ("w3", {"E": 32}, 24, 1), ("tiny", {}, 8, 2)])
def test_pipelined_tier_matches_resident(L, name, override, slots, T):
    """Batch i+1 routed, planned and loaded on a second stream while batch i computes: every
    output bit-equal to the all-resident layer; batch i's slots survive batch i+1's plan."""
    sp, arrays = layer_arrays(name, **override)
    _, dw = device_layer(name, **override)
    tl = L.TieredLayer(FMT[sp["fmt"]], sp["E"], sp["H"], sp["I"], arrays, slots)
    k, nb = sp["k"], 12
    pool = moegen.batch(sp, nb * T)
    lg_all, x_all = to_dev(pool["logits"]), to_dev(pool["x"])
    batches = [(lg_all[b * T:(b + 1) * T].contiguous(), x_all[b * T:(b + 1) * T].contiguous()) for b in range(nb)]
    print(f"{name} slots={slots} T={T}: {nb} pipelined batches", flush=True)
    outs = tl.forward_pipelined(batches, k)
    torch.cuda.synchronize()
    for b, (lg, x) in enumerate(batches):
        want = L.layer_forward(dw, lg, x, k)
        assert torch.equal(outs[b]["ids"], want["ids"])
        assert torch.equal(outs[b]["out"].view(torch.int32), want["out"].view(torch.int32)), f"batch {b}"
    loads = [o["n_load"] for o in outs]
    print(f"{name}: experts loaded per batch {loads}", flush=True)
    assert tl.loaded == sum(loads) and loads[0] > 0
