"""GPU parity: the HIP library (through the C ABI) against the fp64 CPU oracle on the same
seeded inputs.  Routing ids, counts, offsets, perm, inv and decoded weights must match bit
for bit; float outputs within max|gpu - oracle| <= tol * rms(oracle)."""
import numpy as np
import pytest
import torch

import moegen
from oracle import formats as OF
from oracle import moe as OM

from _helpers import (TOL_BF16, TOL_FP8, device_layer, host, max_err_beyond, max_err_over_rms,
                      oracle_fp8_allowance, oracle_layer, oracle_token_rows, sample_tokens, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


# ------------------------------------------------------------------ decoded weights
@pytest.mark.parametrize("name,experts,override", [("tiny", [0, 5, 7], {}), ("decode", [0, 383], {}),
                                                   ("w3", [0, 3, 15], {"E": 16}),
                                                   ("w3", [2, 7], {"E": 8, "k": 2, "H": 256, "I": 512})])
def test_debug_dequant_bit_exact(L, name, experts, override):
    """Both decoders (which 1, 2: the weight-streaming kernels'; 3, 4: the grouped GEMM's field
    decoder) give the format's weights bit for bit."""
    sp, dw = device_layer(name, **override)
    lay = oracle_layer(name, **override)
    for e in experts:
        for which in (1, 2, 3, 4):
            got = host(L.moe_debug_dequant(dw, e, which)).astype(np.float64)
            want = lay.dense(e, 1 if which in (1, 3) else 2)
            assert np.array_equal(got, want), (name, e, which, np.argwhere(got != want)[:5])


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (1, 384, 8), (64, 384, 8), (37, 512, 10), (5, 8, 8),
                                   (300, 100, 7), (4096, 384, 8), (3, 1024, 64), (2, 64, 1)])
def test_route_bit_exact_ids(L, T, E, k):
    r = np.random.default_rng(T * 31 + E)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[0, : E // 2] = 0.25          # ties
    if T > 1:
        lg[1, ::2] = -0.0
        lg[1, 1::2] = 0.0
    ids, gw = L.moe_route(to_dev(lg), k)
    want_ids, want_g = OM.route(lg, k)
    np.testing.assert_array_equal(host(ids), want_ids)
    np.testing.assert_allclose(host(gw), want_g, rtol=2e-6, atol=1e-7)


# ------------------------------------------------------------------ grouping
@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (1, 384, 8), (64, 384, 8), (37, 512, 10), (5, 8, 8),
                                   (511, 384, 8), (513, 384, 8), (4096, 512, 10), (65536, 384, 8),
                                   (1000, 1024, 3)])
def test_permute_bit_exact(L, T, E, k):
    r = np.random.default_rng(T + E + k)
    lg = r.standard_normal((T, E)).astype(np.float32) - 1.1 * np.log(np.arange(1, E + 1))[None, :].astype(np.float32)
    ids, _ = OM.route(lg, k)
    counts, offsets, perm, inv = L.moe_permute(to_dev(ids), E)
    wc, wo, wp, wi = OM.permute(ids, E)
    np.testing.assert_array_equal(host(counts), wc)
    np.testing.assert_array_equal(host(offsets), wo)
    np.testing.assert_array_equal(host(perm), wp)
    np.testing.assert_array_equal(host(inv), wi)


@pytest.mark.parametrize("T,E,k", [(5, 8, 8), (64, 384, 8), (700, 384, 8)])
def test_permute_leaves_out_ids_outside_range(L, T, E, k):
    """Rows whose id is outside [0, E) (here -1 and E + 3) are left out of the grouping: counts,
    offsets and the first offsets[E] entries of perm are those of the other rows (stable by row),
    and inv maps each of them back.  R = 40 (one wave), 512 (one workgroup), 5600 (several)."""
    r = np.random.default_rng(77 + T)
    ids = r.integers(0, E, size=(T, k)).astype(np.int32)
    bad = r.uniform(size=(T, k)) < 0.1
    ids[bad] = np.where(r.uniform(size=int(bad.sum())) < 0.5, -1, E + 3).astype(np.int32)
    counts, offsets, perm, inv = L.moe_permute(to_dev(ids), E)
    flat = ids.reshape(-1)
    valid = np.flatnonzero((flat >= 0) & (flat < E))
    order = valid[np.argsort(flat[valid], kind="stable")]
    want_counts = np.bincount(flat[valid], minlength=E)
    np.testing.assert_array_equal(host(counts), want_counts)
    np.testing.assert_array_equal(host(offsets), np.concatenate([[0], np.cumsum(want_counts)]))
    np.testing.assert_array_equal(host(perm)[:len(valid)], order)
    np.testing.assert_array_equal(host(inv)[order], np.arange(len(valid)))


def test_permute_empty_batch(L):
    ids = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    counts, offsets, perm, inv = L.moe_permute(ids, 8)
    assert host(counts).tolist() == [0] * 8 and host(offsets).tolist() == [0] * 9


# ------------------------------------------------------------------ combine
def test_combine_bf16_is_rne_of_fp32(L):
    r = np.random.default_rng(3)
    T, k, H = 33, 4, 512
    y = r.standard_normal((T * k, H)).astype(np.float32)
    inv = r.permutation(T * k).astype(np.int32)
    g = r.uniform(0, 1, (T, k)).astype(np.float32)
    o32 = host(L.moe_combine(to_dev(y), to_dev(inv), to_dev(g), out_fp32=True))
    o16 = host(L.moe_combine(to_dev(y), to_dev(inv), to_dev(g), out_fp32=False)).view(np.uint16)
    want = OM.combine(y, inv, g, T, k)
    assert max_err_over_rms(o32, want) < 1e-6
    np.testing.assert_array_equal(o16, torch.from_numpy(o32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------------ the whole layer
def _check_layer(L, name, T, sample=False, fp8_slots=None, **override):
    """The whole layer against the oracle: routing and grouping over every token, bit for bit;
    float outputs of every token, or (sample=True) of 256 seeded tokens (their k routed rows
    each: the expert outputs y_perm and the combined output), within TOL_BF16 * rms of the
    oracle.  For the rows of FP8 experts each element also has the allowance of the e4m3
    rounding flips of h that the matrix cores' sums may cause (see mxfp8_flip_allowance), and
    the combined output the gate-weighted sum of its rows' allowances."""
    sp, dw = device_layer(name, **override)
    lay = oracle_layer(name, **override)
    b = moegen.batch(sp, T)
    k = sp["k"]
    tol = TOL_BF16
    fp8 = sp["n_hot"] > 0 and sp["hot_mode"] != "residual"
    res = L.layer_forward(dw, to_dev(b["logits"]), to_dev(b["x"]), k, out_fp32=True, fp8_slots=fp8_slots)
    ids, gates = OM.route(b["logits"], k)
    counts, offsets, perm, inv = OM.permute(ids, sp["E"])
    np.testing.assert_array_equal(host(res["ids"]), ids)
    np.testing.assert_array_equal(host(res["counts"]), counts)
    np.testing.assert_array_equal(host(res["offsets"]), offsets)
    np.testing.assert_array_equal(host(res["perm"]), perm)
    np.testing.assert_array_equal(host(res["inv"]), inv)
    if sample:
        toks = sample_tokens(T)
        at = {}
        yt = oracle_token_rows(lay, b["x"], ids, toks, k, allowance=at if fp8 else None)
        rows = np.array([inv[t * k + j] for t in toks for j in range(k)])
        y_rows = np.stack([yt[(int(t), j)] for t in toks for j in range(k)])
        zero = np.zeros(sp["H"])
        a_rows = np.stack([at.get((int(t), j), zero) for t in toks for j in range(k)])
        out = np.zeros((len(toks), sp["H"]))
        a_out = np.zeros((len(toks), sp["H"]))
        for j in range(k):
            out += gates[toks, j:j + 1] * np.stack([yt[(int(t), j)] for t in toks])
            a_out += gates[toks, j:j + 1] * np.stack([at.get((int(t), j), zero) for t in toks])
    else:
        toks = np.arange(T)
        y = OM.expert_ffn(lay, b["x"], k, offsets, perm)
        out = OM.combine(y, inv, gates, T, k)
        rows = np.arange(T * k)
        y_rows = y
        a_rows = (oracle_fp8_allowance(lay, b["x"], k, offsets, perm, sp["E"], sp["H"]) if fp8
                  else np.zeros_like(y))
        a_out = OM.combine(a_rows, inv, gates, T, k) if T > 0 else np.zeros_like(out)
    got = host(res["out"])[toks]
    err = max_err_beyond(got, out, a_out)
    plain = max_err_over_rms(got, out)
    print(f"{name} T={T}: {len(toks)} tokens, max|err|/rms = {plain:.4g}, "
          f"beyond the FP8 allowance {err:.4g}", flush=True)
    assert err <= tol
    if fp8 and not override:
        # at the layer's own shape the flips stay inside the flat bound for FP8 layers as well
        assert plain <= TOL_FP8
    assert max_err_beyond(host(res["y_perm"])[rows], y_rows, a_rows) <= tol
    # bf16 output is the RNE of the same fp32 sums
    o16 = L.moe_combine(res["y_perm"], res["inv"], res["gates"], out_fp32=False)
    ref16 = res["out"].to(torch.bfloat16).view(torch.int16)
    assert torch.equal(o16, ref16)
    return res


@pytest.mark.parametrize("T", [16, 1, 5, 37, 64, 100, 128, 300, 1000])
def test_layer_tiny(L, T):
    _check_layer(L, "tiny", T)


def test_layer_tiny_k1_and_kE(L):
    _check_layer(L, "tiny", 9, k=1)
    _check_layer(L, "tiny", 9, k=8)


@pytest.mark.parametrize("T", [1, 2, 10, 40])
def test_ffn_repeated_expert_ids(L, T):
    """Ids supplied directly, with experts repeated within a token: a group then holds more
    than T rows, and the streaming path must still split it into items its token stage holds
    (at most 8 rows when K is split in 4, 16 when split in 2)."""
    # decode-sized experts (FC1 K = 4096, FC2 K = 2048) so every K split is taken
    name, k, ov = "tiny", 8, dict(H=4096, I=2048)
    sp, dw = device_layer(name, k=k, **ov)
    lay = oracle_layer(name, k=k, **ov)
    b = moegen.batch(sp, T)
    r = np.random.default_rng(1234 + T)
    ids = np.where(r.uniform(size=(T, k)) < 0.75, 3, r.integers(0, sp["E"], size=(T, k))).astype(np.int32)
    counts, offsets, perm, inv = OM.permute(ids, sp["E"])
    assert counts.max() > T  # the case under test
    c_d, o_d, p_d, i_d = L.moe_permute(to_dev(ids), sp["E"])
    np.testing.assert_array_equal(host(o_d), offsets)
    np.testing.assert_array_equal(host(p_d), perm)
    y = host(L.moe_expert_ffn(dw, to_dev(b["x"]), k, c_d, o_d, p_d))
    want = OM.expert_ffn(lay, b["x"], k, offsets, perm, experts=sorted(set(ids.reshape(-1).tolist())))
    err = max_err_over_rms(y, want)
    print(f"repeated ids T={T}: max|err|/rms = {err:.4g}", flush=True)
    assert err <= TOL_BF16


@pytest.mark.parametrize("T", [1, 8, 64])
def test_layer_decode(L, T):
    _check_layer(L, "decode", T)


def test_layer_decode_shape_gemm_path(L):
    _check_layer(L, "decode", 256, sample=True)


@pytest.mark.parametrize("T", [8192, 65536])
def test_layer_prefill(L, T):
    _check_layer(L, "prefill", T, sample=True)


# 3-bit experts: a small variant (many T, both kernels) and the full 512-expert shape
W3_SMALL = {"E": 8, "k": 2, "H": 256, "I": 512}


@pytest.mark.parametrize("T", [1, 5, 16, 37, 128, 300])
def test_layer_w3_small(L, T):
    _check_layer(L, "w3", T, **W3_SMALL)


@pytest.mark.parametrize("T,sample", [(1, False), (8, False), (64, False), (512, True), (4096, True)])
def test_layer_w3(L, T, sample):
    _check_layer(L, "w3", T, sample)


# ------------------------------------------------------------------ hot experts (MXFP4 -> FP8)
def test_mxfp4_to_fp8_bit_exact(L):
    r = np.random.default_rng(11)
    codes = r.integers(0, 256, size=(37, 160), dtype=np.uint8)
    codes[0, :16] = np.arange(16, dtype=np.uint8) * 17  # every nibble in both positions
    scales = r.integers(0, 256, size=(37, 10), dtype=np.uint8)
    elems, sc = L.moe_mxfp4_to_fp8(to_dev(codes), to_dev(scales))
    we, ws = OF.mxfp4_to_fp8(codes, scales)
    np.testing.assert_array_equal(host(elems), we)
    np.testing.assert_array_equal(host(sc), ws)


def test_mxfp8_quantize_bit_exact(L):
    r = np.random.default_rng(12)
    rows, K = 64, 256
    x = moegen._f32_to_bf16_bits((r.standard_normal((rows, K)) * np.exp2(r.integers(-20, 20, (rows, 1)))).astype(np.float32))
    x[0, :32] = 0                                   # all-zero block -> scale byte 0
    x[0, 32:64] = 0x8000                            # all -0
    x[1, :32] = r.integers(1, 0x80, 32)             # bf16 subnormals
    x[1, 32:64] = 0x7F7F                            # the largest bf16
    x[2, :32] = moegen._f32_to_bf16_bits(np.float32(1.8125) * np.ones(32, np.float32))  # ties at the top
    x[2, 40] = moegen._f32_to_bf16_bits(np.array([-448.0 * 1.0625], np.float32))[0]
    x[3, :] = moegen._f32_to_bf16_bits(np.float32(1e-3) * r.standard_normal(K).astype(np.float32))
    elems, sc = L.moe_mxfp8_quantize(to_dev(x))
    we, ws = OF.mxfp8_quantize(OF.bf16_value(x))
    np.testing.assert_array_equal(host(sc), ws)
    np.testing.assert_array_equal(host(elems), we)


MIXED_SMALL = {"E": 16, "k": 4, "H": 256, "I": 512, "n_hot": 4}


@pytest.mark.parametrize("T", [1, 16, 100, 300])
def test_layer_mixed_small(L, T):
    _check_layer(L, "mixed", T, **MIXED_SMALL)


def test_layer_mixed_small_fewer_slots_than_hot_experts(L):
    a = _check_layer(L, "mixed", 200, fp8_slots=1, **MIXED_SMALL)
    b = _check_layer(L, "mixed", 200, fp8_slots=3, **MIXED_SMALL)
    assert torch.equal(a["out"], b["out"])


@pytest.mark.parametrize("T,sample", [(64, False), (4096, True)])
def test_layer_mixed(L, T, sample):
    _check_layer(L, "mixed", T, sample)


# The FP8 GEMM keeps its three LDS stages running across a workgroup's tasks: the last steps of
# one task load the next task's first stages, and the buffer that holds a task's first stage
# moves by (K / 128) mod 3 from one task to the next (K / 128 < 3: no loads across tasks).
# Shapes that give each of these cases in FC1 (K = H) and in FC2 (K = I), with enough hot rows
# that every one of the 256 workgroups runs three tasks or more.
FP8_RING = [({"H": 768, "I": 768}, 16384),    # FC1 K/128 = 6 (mod 3 = 0), FC2 6 (0)
            ({"H": 512, "I": 1024}, 16384),   # FC1 4 (1), FC2 8 (2)
            ({"H": 1024, "I": 256}, 16384),   # FC1 8 (2), FC2 2 (< 3)
            ({"H": 256, "I": 512}, 32768)]    # FC1 2 (< 3), FC2 4 (1)


def _fp8_tasks(over, T):
    """Tasks of the FP8 FC1 and FC2 launches (items of <= 128 rows of a hot expert, times the
    column tiles: I / 128 for FC1, H / 256 for FC2)."""
    sp = moegen.spec("mixed", **over)
    ids, _ = OM.route(moegen.batch(sp, T)["logits"], sp["k"])
    counts = np.bincount(ids.ravel(), minlength=sp["E"])
    items = int(sum((counts[e] + 127) // 128 for e in moegen.hot_ids(sp)))
    return items * sp["I"] // 128, items * sp["H"] // 256


@pytest.mark.parametrize("dims,T", FP8_RING)
def test_layer_mixed_fp8_ring(L, dims, T):
    over = dict(E=16, k=4, n_hot=8, **dims)
    fc1, fc2 = _fp8_tasks(over, T)
    assert min(fc1, fc2) >= 3 * 256, (fc1, fc2)
    _check_layer(L, "mixed", T, True, **over)


def test_layer_mixed_fp8_ring_skipped_tasks(L):
    """Three FP8 slots for eight hot experts: every batch's launches skip the tasks of the
    experts outside the batch, so the next task a workgroup prefetches is often several strides
    ahead; the output is the same bits as with every expert in one batch."""
    over = dict(E=16, k=4, n_hot=8, H=768, I=768)
    a = _check_layer(L, "mixed", 16384, True, fp8_slots=3, **over)
    b = _check_layer(L, "mixed", 16384, True, **over)
    assert torch.equal(a["out"], b["out"])


def test_layer_deterministic(L):
    sp, dw = device_layer("tiny")
    b = moegen.batch(sp, 64)
    a = L.layer_forward(dw, to_dev(b["logits"]), to_dev(b["x"]), sp["k"])
    c = L.layer_forward(dw, to_dev(b["logits"]), to_dev(b["x"]), sp["k"])
    assert torch.equal(a["out"], c["out"]) and torch.equal(a["y_perm"], c["y_perm"])


def test_empty_batch_is_a_noop(L):
    sp, dw = device_layer("tiny")
    x = torch.zeros((0, sp["H"]), dtype=torch.int16, device="cuda")
    lg = torch.zeros((0, sp["E"]), dtype=torch.float32, device="cuda")
    res = L.layer_forward(dw, lg, x, sp["k"])
    assert res["out"].shape == (0, sp["H"])


# ------------------------------------------------------------------ hot experts as an FP4 residual
RES_SMALL = {"E": 16, "k": 4, "H": 256, "I": 512, "n_hot": 4}


@pytest.mark.parametrize("name,override", [("residual", {}), ("residual", RES_SMALL)])
def test_residual_dequant_bit_exact(L, name, override):
    """The streaming kernels' MXFP4 residual decoder (2-bit slot order) gives the MXFP4 weights of
    every hot slot bit for bit."""
    sp, dw = device_layer(name, **override)
    from _helpers import layer_arrays

    _, arrays = layer_arrays(name, **override)
    for s in (0, sp["n_hot"] - 1):
        for which in (1, 2):
            got = host(L.moe_debug_dequant(dw, s, 4 + which)).astype(np.float64)
            want = OF.dequant_mxfp4(arrays[f"hot_w{which}_codes"][s], arrays[f"hot_w{which}_scales"][s])
            assert np.array_equal(got, want), (name, s, which, np.argwhere(got != want)[:5])


@pytest.mark.parametrize("T", [1, 8, 64])
def test_layer_residual(L, T):
    _check_layer(L, "residual", T)


@pytest.mark.parametrize("T", [1, 16, 100, 300])
def test_layer_residual_small(L, T):
    """Hot experts with more than 32 rows (several items each) and, from 128 tokens, cold experts
    on the grouped GEMM beside hot experts on the streaming kernels."""
    _check_layer(L, "residual", T, **RES_SMALL)


def test_layer_residual_large_batch(L):
    _check_layer(L, "residual", 4096, sample=True)
