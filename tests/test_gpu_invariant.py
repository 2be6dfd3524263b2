"""GPU: batch-invariant mode (MOE_FLAG_BATCH_INVARIANT).  [Moet-README] (results table of the
DeepSeek-V4.1-Flash build, quality row): a request gives the same logits at any batch size.

A token's layer output must have the same bits whether it comes alone, in a small decode batch,
in a prefill-sized batch, or at another position of the batch; and the mode's outputs must still
match the fp64 oracle within the layer tolerance."""
import numpy as np
import pytest
import torch

import moegen
from oracle import moe as OM

from _helpers import TOL_BF16, TOL_FP8, device_layer, host, max_err_over_rms, oracle_layer, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


POOL = 600

# (layer, overrides): E=8 groups reach hundreds of rows (the grouped-GEMM path of the default
# mode); the 384-expert layers split K over 4 waves at one token; "mixed" adds FP8 hot experts.
CASES = [("tiny", {}), ("decode", {}), ("w3", {"E": 16}), ("mixed", {})]


def _batches(rng):
    """Index lists into the token pool: sizes across the decode / prefill boundaries, with
    tokens 17 and 599 in every batch at different positions."""
    out = [np.array([17]), np.array([599, 17])]
    for T in (5, 16, 17, 64, 129, 300):
        idx = rng.choice(np.setdiff1d(np.arange(POOL), [17, 599]), T - 2, replace=False)
        idx = np.insert(idx, rng.integers(0, T - 1), 17)
        idx = np.insert(idx, rng.integers(0, T), 599)
        out.append(idx)
    out.append(np.arange(POOL)[::-1].copy())
    return out


@pytest.mark.parametrize("name,override", CASES)
def test_same_bits_at_any_batch_size(L, name, override):
    sp, dw = device_layer(name, **override)
    dw.set_batch_invariant(True)
    k = sp["k"]
    b = moegen.batch(sp, POOL)
    x, lg = to_dev(b["x"]), to_dev(b["logits"])
    print(f"{name}: pool of {POOL} tokens", flush=True)
    full = L.layer_forward(dw, lg, x, k, out_fp32=True)["out"]
    fbits = full.view(torch.int32)
    for idx in _batches(np.random.default_rng(7)):
        ti = torch.from_numpy(idx).cuda()
        print(f"{name}: T={len(idx)}", flush=True)
        sub = L.layer_forward(dw, lg[ti].contiguous(), x[ti].contiguous(), k, out_fp32=True)["out"]
        same = torch.all(sub.view(torch.int32) == fbits[ti], dim=1)
        assert bool(same.all()), f"T={len(idx)}: {int((~same).sum())} tokens differ from the pool's bits"
    # the default mode on the same batches, for the record (it may differ: K split and GEMM path)
    dw.set_batch_invariant(False)
    full_d = L.layer_forward(dw, lg, x, k, out_fp32=True)["out"].view(torch.int32)
    one = L.layer_forward(dw, lg[17:18].contiguous(), x[17:18].contiguous(), k, out_fp32=True)["out"]
    print(f"{name}: default mode, token 17 alone vs in the pool: "
          f"{int((one.view(torch.int32)[0] != full_d[17]).sum())} of {sp['H']} outputs differ", flush=True)


@pytest.mark.parametrize("name,override,T,sample", [("tiny", {}, 300, None), ("decode", {}, 64, [0, 31, 63]),
                                                    ("decode", {}, 1, None), ("w3", {"E": 16}, 200, None),
                                                    ("mixed", {}, 256, [0, 128, 255])])
def test_invariant_mode_matches_oracle(L, name, override, T, sample):
    sp, dw = device_layer(name, **override)
    dw.set_batch_invariant(True)
    lay = oracle_layer(name, **override)
    k = sp["k"]
    b = moegen.batch(sp, T)
    res = L.layer_forward(dw, to_dev(b["logits"]), to_dev(b["x"]), k, out_fp32=True)
    ids, gates = OM.route(b["logits"], k)
    counts, offsets, perm, inv = OM.permute(ids, sp["E"])
    np.testing.assert_array_equal(host(res["perm"]), perm)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    experts = sorted(set(ids[toks].reshape(-1).tolist()))
    y = OM.expert_ffn(lay, b["x"], k, offsets, perm, experts=experts)
    want = OM.combine(np.nan_to_num(y), inv, gates, T, k)[toks]
    err = max_err_over_rms(host(res["out"])[toks], want)
    print(f"{name} T={T} invariant: max|err|/rms = {err:.4g}", flush=True)
    assert err <= (TOL_FP8 if sp["n_hot"] > 0 else TOL_BF16)


def test_invariant_mode_empty_batch_and_repeated_ids(L):
    """T = 0 is a no-op; repeated expert ids (groups larger than T) still give each row the bits
    it gets alone."""
    sp, dw = device_layer("tiny")
    dw.set_batch_invariant(True)
    x0 = torch.zeros((0, sp["H"]), dtype=torch.int16, device="cuda")
    lg0 = torch.zeros((0, sp["E"]), dtype=torch.float32, device="cuda")
    assert L.layer_forward(dw, lg0, x0, sp["k"])["out"].shape == (0, sp["H"])
    k, T = 4, 40
    b = moegen.batch(sp, T)
    x = to_dev(b["x"])
    ids = torch.from_numpy(np.random.default_rng(3).integers(0, 2, size=(T, k)).astype(np.int32)).cuda()
    counts, offsets, perm, inv = L.moe_permute(ids, sp["E"])
    y = L.moe_expert_ffn(dw, x, k, counts, offsets, perm)
    y_tok = y[inv.long()].view(T, k, sp["H"])  # row t*k+j of token t
    for t in (0, 17, 39):
        ids1 = ids[t:t + 1].contiguous()
        c1, o1, p1, i1 = L.moe_permute(ids1, sp["E"])
        y1 = L.moe_expert_ffn(dw, x[t:t + 1].contiguous(), k, c1, o1, p1)[i1.long()]
        assert torch.equal(y1.view(torch.int32), y_tok[t].view(torch.int32)), t


def test_invariant_mode_with_fewer_slots_than_hot_experts(L):
    """Hot experts converted and computed in batches of 5 slots: a token's bits do not depend on
    the batch it comes in, nor on the slot count."""
    sp, dw = device_layer("mixed")
    dw.set_batch_invariant(True)
    k = sp["k"]
    b = moegen.batch(sp, 300)
    x, lg = to_dev(b["x"]), to_dev(b["logits"])
    full = L.layer_forward(dw, lg, x, k, fp8_slots=5)["out"].view(torch.int32)
    full_all = L.layer_forward(dw, lg, x, k)["out"].view(torch.int32)
    assert torch.equal(full, full_all)
    for idx in (np.array([17]), np.arange(0, 300, 7)):
        ti = torch.from_numpy(idx).cuda()
        print(f"mixed, 5 slots: T={len(idx)}", flush=True)
        sub = L.layer_forward(dw, lg[ti].contiguous(), x[ti].contiguous(), k, fp8_slots=5)["out"]
        assert torch.equal(sub.view(torch.int32), full[ti])
