"""Pins of the oracle's routing, grouping, expert FFN and combine: brute force on tiny
inputs, closed forms, special cases that reduce to a dense MLP, and the expert-sum
identity.  None of these re-types the oracle's own formula."""
import math
import os

import numpy as np
import pytest
import torch

import moegen
from oracle import formats as F
from oracle import moe as M


# ------------------------------------------------------------------------ routing
def _brute_topk(row, k):
    """Pure-Python: sort (expert) by (-logit, id) with Python float comparison
    (-0.0 == 0.0) and take the first k."""
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 2), (8, 8), (5, 1), (16, 10), (3, 3)])
def test_route_matches_brute_force_with_ties(E, k):
    r = np.random.default_rng(10 + E + k)
    T = 40
    lg = r.standard_normal((T, E)).astype(np.float32)
    # inject ties: duplicated values, +-0, a row of all-equal logits
    lg[0] = 0.5
    lg[1, ::2] = 0.0
    lg[1, 1::2] = -0.0
    lg[2, :] = np.round(lg[2, :])
    lg[3, : E // 2] = lg[3, E - 1]
    ids, g = M.route(lg, k)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(lg[t], k), t


def test_route_gates_closed_forms():
    lg = np.array([[3.0, 1.0, 2.0, -1.0]], np.float32)
    ids, g = M.route(lg, 1)
    assert ids[0, 0] == 0 and g[0, 0] == 1.0
    ids, g = M.route(lg, 2)
    assert list(ids[0]) == [0, 2]
    assert abs(g[0, 0] - 1 / (1 + math.exp(-1.0))) < 1e-15
    assert abs(g[0, 1] - 1 / (1 + math.exp(1.0))) < 1e-15
    r = np.random.default_rng(11)
    lg = r.standard_normal((200, 64)).astype(np.float32) * 4
    for k in (1, 3, 8, 64):
        ids, g = M.route(lg, k)
        assert np.all(np.abs(g.sum(1) - 1) < 1e-14)
        assert np.all(np.diff(g, axis=1) <= 0)  # descending logits -> descending gates
        # gate ratio equals exp of the logit difference
        sel = np.take_along_axis(lg, ids.astype(np.int64), 1).astype(np.float64)
        np.testing.assert_allclose(g[:, 0] / g[:, -1], np.exp(sel[:, 0] - sel[:, -1]), rtol=1e-12)


def test_route_k_equals_E_is_a_full_sort():
    r = np.random.default_rng(12)
    lg = r.standard_normal((10, 7)).astype(np.float32)
    ids, _ = M.route(lg, 7)
    for t in range(10):
        assert sorted(ids[t]) == list(range(7))
        assert np.all(np.diff(lg[t, ids[t]]) <= 0)


# ---------------------------------------------------------------------- grouping
def _brute_permute(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    perm = [r for e in range(E) for r in range(len(flat)) if flat[r] == e]
    counts = [sum(1 for v in flat if v == e) for e in range(E)]
    return counts, perm


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (16, 8, 2), (33, 5, 5), (50, 384, 8), (0, 4, 2)])
def test_permute_matches_brute_force(T, E, k):
    r = np.random.default_rng(T * 7 + E)
    lg = r.standard_normal((T, E)).astype(np.float32)
    ids = M.route(lg, k)[0] if T else np.zeros((0, k), np.int32)
    counts, offsets, perm, inv = M.permute(ids, E)
    bc, bp = _brute_permute(ids, E)
    assert list(counts) == bc and list(perm) == bp
    R = T * k
    assert offsets[0] == 0 and offsets[E] == R and np.all(np.diff(offsets) == counts)
    assert sorted(perm.tolist()) == list(range(R))
    assert np.all(inv[perm] == np.arange(R)) and np.all(perm[inv] == np.arange(R))
    flat = ids.reshape(-1)
    for e in range(E):
        rows = perm[offsets[e]: offsets[e + 1]]
        assert np.all(flat[rows] == e) and np.all(np.diff(rows) > 0)


# ------------------------------------------------------------------- the experts
def test_silu_closed_forms():
    assert M.silu(np.array(0.0)) == 0.0
    x = np.linspace(-30, 30, 121)
    # silu(-x) = silu(x) - x  (x*sigmoid(x) - x = -x*sigmoid(-x))
    np.testing.assert_allclose(M.silu(-x), M.silu(x) - x, atol=1e-12)
    assert abs(M.silu(np.array(1.0)) - 1 / (1 + math.exp(-1))) < 1e-16
    assert M.silu(np.array(-800.0)) == 0.0


def _loop_ffn(x, W1, W2):
    """Pure-Python loops, tiny sizes only."""
    n, H = x.shape
    I = W1.shape[0] // 2
    y = [[0.0] * H for _ in range(n)]
    for r in range(n):
        h = []
        for o in range(I):
            g = sum(x[r][c] * W1[o][c] for c in range(H))
            u = sum(x[r][c] * W1[I + o][c] for c in range(H))
            h.append(g / (1 + math.exp(-g)) * u)
        for o in range(H):
            y[r][o] = sum(h[i] * W2[o][i] for i in range(I))
    return np.array(y)


def test_ffn_matches_python_loops():
    r = np.random.default_rng(13)
    n, H, I = 3, 32, 16
    x = r.standard_normal((n, H))
    W1 = r.standard_normal((2 * I, H)) * 0.3
    W2 = r.standard_normal((H, I)) * 0.3
    np.testing.assert_allclose(M.swiglu_ffn(x, W1, W2), _loop_ffn(x, W1, W2), rtol=1e-12, atol=1e-12)


def test_fc1_one_hot_is_a_weight_column():
    r = np.random.default_rng(14)
    W1 = r.standard_normal((64, 32))
    for h in (0, 7, 31):
        x = np.zeros((1, 32))
        x[0, h] = 1.0
        np.testing.assert_array_equal(M.fc1(x, W1)[0], W1[:, h])


def test_swiglu_gate_up_split():
    a = np.array([[0.0, 2.0, 5.0, -3.0]])  # I = 2: gate (0, 2), up (5, -3)
    np.testing.assert_allclose(M.swiglu(a), [[0.0, 2 / (1 + math.exp(-2)) * -3]], rtol=1e-15)


def _tiny_layer(fmt="w2", E=4, H=64, I=32, hot=0, seed=0):
    sp = moegen.spec("tiny", E=E, H=H, I=I, fmt=fmt, n_hot=hot, index=90 + seed)
    return sp, M.Layer(fmt, moegen.weights(sp))


def test_doubling_w2_scales_doubles_y_exactly():
    sp, layer = _tiny_layer()
    a2 = dict(layer.a)
    a2["w2_scales"] = (layer.a["w2_scales"].astype(np.uint32) + 0x80).astype(np.uint16)  # exponent + 1
    layer2 = M.Layer("w2", a2)
    x = moegen.batch(sp, 5)["x"]
    X = F.bf16_value(x)
    y1 = M.swiglu_ffn(X, layer.dense(1, 1), layer.dense(1, 2))
    y2 = M.swiglu_ffn(X, layer2.dense(1, 1), layer2.dense(1, 2))
    np.testing.assert_array_equal(y2, 2 * y1)


def test_single_expert_layer_is_a_dense_mlp_torch():
    """E = 1, k = 1: the layer reduces to one dense SwiGLU MLP; checked against torch
    (float64, an independent library) on the dense dequantised matrices."""
    sp, layer = _tiny_layer(E=1)
    b = moegen.batch(sp, 9)
    res = M.layer_forward(layer, b["logits"][:, :1], b["x"], 1)
    X = torch.from_numpy(F.bf16_value(b["x"]))
    W1 = torch.from_numpy(layer.dense(0, 1))
    W2 = torch.from_numpy(layer.dense(0, 2))
    a = torch.nn.functional.linear(X, W1)
    h = torch.nn.functional.silu(a[:, :32]) * a[:, 32:]
    y = torch.nn.functional.linear(h, W2).numpy()
    np.testing.assert_allclose(res["out"], y, rtol=1e-12, atol=1e-12)
    assert np.all(res["gates"] == 1.0)


def test_expert_sum_identity():
    """Every expert with identical bytes: out[t] = FFN(x_t) for any routing, because the
    gates of a token sum to one."""
    sp, layer = _tiny_layer(E=6)
    same = {key: (np.repeat(v[:1], v.shape[0], axis=0) if key.startswith("w") else v)
            for key, v in layer.a.items()}
    lay = M.Layer("w2", same)
    b = moegen.batch(sp, 12)
    res = M.layer_forward(lay, b["logits"], b["x"], 3)
    X = F.bf16_value(b["x"])
    want = M.swiglu_ffn(X, lay.dense(0, 1), lay.dense(0, 2))
    np.testing.assert_allclose(res["out"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_k1_output_is_the_chosen_expert():
    sp, layer = _tiny_layer(E=4)
    b = moegen.batch(sp, 10)
    res = M.layer_forward(layer, b["logits"], b["x"], 1)
    X = F.bf16_value(b["x"])
    for t in range(10):
        e = int(np.argmax(b["logits"][t]))
        want = M.swiglu_ffn(X[t: t + 1], layer.dense(e, 1), layer.dense(e, 2))[0]
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-13, atol=1e-15)


def test_combine_hand_example():
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0], [0.5, 0.25]])
    inv = np.array([2, 0, 1, 3])  # token 0 -> rows 2, 0; token 1 -> rows 1, 3
    g = np.array([[0.75, 0.25], [0.5, 0.5]])
    out = M.combine(y, inv, g, 2, 2)
    np.testing.assert_array_equal(out, [[75.25, 150.5], [5.25, 10.125]])


def test_fp8_expert_models_mxfp8_activations():
    """A hot expert computes from the converted FP8 weights with MXFP8 x and h: it equals
    the dense MLP on round-tripped activations, and differs from the unquantised one."""
    sp, layer = _tiny_layer(E=4, hot=2)
    hot = [int(e) for e in layer.a["hot_ids"]]
    assert layer.is_fp8(hot[0]) and not layer.is_fp8([e for e in range(4) if e not in hot][0])
    e = hot[0]
    W1, W2 = layer.dense(e, 1), layer.dense(e, 2)
    np.testing.assert_array_equal(W1, F.dequant_mxfp4(layer.a["hot_w1_codes"][0], layer.a["hot_w1_scales"][0]))
    X = F.bf16_value(moegen.batch(sp, 4)["x"])
    y = M.swiglu_ffn(X, W1, W2, fp8=True)
    xq = F.mxfp8_dequant(*F.mxfp8_quantize(X))
    a = xq @ W1.T
    h = a[:, :32] / (1 + np.exp(-a[:, :32])) * a[:, 32:]
    hq = F.mxfp8_dequant(*F.mxfp8_quantize(h))
    np.testing.assert_allclose(y, hq @ W2.T, rtol=1e-13, atol=1e-13)
    assert np.max(np.abs(y - M.swiglu_ffn(X, W1, W2))) > 1e-3 * np.max(np.abs(y))


def test_expert_subset_rows():
    sp, layer = _tiny_layer(E=4)
    b = moegen.batch(sp, 8)
    full = M.layer_forward(layer, b["logits"], b["x"], 2)
    part = M.expert_ffn(layer, b["x"], 2, full["offsets"], full["perm"], experts=[1])
    lo, hi = full["offsets"][1], full["offsets"][2]
    np.testing.assert_array_equal(part[lo:hi], full["y_perm"][lo:hi])
    assert np.all(np.isnan(part[:lo])) and np.all(np.isnan(part[hi:]))


# ------------------------------------------------------------- FP4 residual (delta cache)
RES_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "residual.txt")


def _res_golden():
    out = []
    for line in open(RES_GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        words, scale, byte, e8 = lhs.split()
        out.append(([int(w, 16) for w in words.split(",")], int(scale, 16), int(byte, 16), int(e8),
                    [float(v) for v in rhs.split(",")]))
    return out


def _residual_layer(E=4, H=64, I=32, hot=2, seed=0):
    sp = moegen.spec("tiny", E=E, H=H, I=I, n_hot=hot, index=95 + seed, hot_mode="residual")
    return sp, M.Layer("w2", moegen.weights(sp), hot_mode="residual")


@pytest.mark.parametrize("words,scale,byte,e8,vals", _res_golden())
def test_residual_hand_worked_rows(words, scale, byte, e8, vals):
    """One hot-expert row (32 weights): 2-bit weights plus the MXFP4 residual, against the
    hand-derived values in tests/golden/residual.txt."""
    a = {"w1_codes": np.array(words, np.uint32).reshape(1, 1, 2), "w1_scales": np.array([[[scale]]], np.uint16),
         "w2_codes": np.zeros((1, 1, 2), np.uint32), "w2_scales": np.zeros((1, 1, 1), np.uint16),
         "hot_ids": np.array([0], np.int32),
         "hot_w1_codes": np.full((1, 1, 16), byte, np.uint8), "hot_w1_scales": np.array([[[e8]]], np.uint8),
         "hot_w2_codes": np.zeros((1, 1, 16), np.uint8), "hot_w2_scales": np.zeros((1, 1, 1), np.uint8)}
    lay = M.Layer("w2", a, hot_mode="residual")
    np.testing.assert_array_equal(lay.dense(0, 1)[0] * 2.0**7, np.array(vals))


def test_residual_zero_delta_is_the_2bit_layer():
    """All residual nibbles zero (any scale): the layer is the 2-bit layer, bit for bit."""
    sp, lay = _residual_layer(E=6, hot=3)
    a0 = dict(lay.a)
    for key in ("hot_w1_codes", "hot_w2_codes"):
        a0[key] = np.zeros_like(a0[key])
    zero = M.Layer("w2", a0, hot_mode="residual")
    plain = M.Layer("w2", {k_: v for k_, v in lay.a.items() if not k_.startswith("hot_")})
    b = moegen.batch(sp, 11)
    r0 = M.layer_forward(zero, b["logits"], b["x"], 2)
    r1 = M.layer_forward(plain, b["logits"], b["x"], 2)
    np.testing.assert_array_equal(r0["out"], r1["out"])
    assert any(int(e) in set(r0["ids"].reshape(-1).tolist()) for e in lay.a["hot_ids"])


def test_residual_zero_2bit_scales_give_the_mxfp4_weights():
    sp, lay = _residual_layer()
    a0 = dict(lay.a)
    for key in ("w1_scales", "w2_scales"):
        a0[key] = np.zeros_like(a0[key])
    z = M.Layer("w2", a0, hot_mode="residual")
    for s, e in enumerate(lay.a["hot_ids"]):
        for which in (1, 2):
            want = F.dequant_mxfp4(lay.a[f"hot_w{which}_codes"][s], lay.a[f"hot_w{which}_scales"][s])
            np.testing.assert_array_equal(z.dense(int(e), which), want)


def _bits_w2(words, scales, K):
    """2-bit weights by Python bit loops (not the oracle's unpacking)."""
    rows = words.shape[0]
    out = np.zeros((rows, K))
    for r in range(rows):
        for k in range(K):
            c = (int(words[r, k // 16]) >> (2 * (k % 16))) & 3
            s = np.array([int(scales[r, k // 32]) << 16], np.uint32).view(np.float32)[0]
            out[r, k] = (-4.0, -1.0, 1.0, 4.0)[c] * float(s)
    return out


def _bits_mxfp4(codes, scales, K):
    """MXFP4 weights by Python bit loops."""
    mag = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
    rows = codes.shape[0]
    out = np.zeros((rows, K))
    for r in range(rows):
        for k in range(K):
            n = (int(codes[r, k // 2]) >> (4 * (k % 2))) & 15
            v = mag[n & 7] * (-1.0 if n & 8 else 1.0)
            out[r, k] = v * 2.0 ** (int(scales[r, k // 32]) - 127)
    return out


def test_residual_single_expert_layer_is_a_dense_mlp_torch():
    """E = 1, k = 1, the expert hot: the layer is one SwiGLU MLP on W = W_2bit + W_mxfp4, with
    both parts unpacked here by bit loops and the MLP evaluated by torch (float64)."""
    sp, lay = _residual_layer(E=1, hot=1, H=64, I=32)
    b = moegen.batch(sp, 7)
    res = M.layer_forward(lay, b["logits"][:, :1], b["x"], 1)
    a = lay.a
    W1 = _bits_w2(a["w1_codes"][0], a["w1_scales"][0], 64) + _bits_mxfp4(a["hot_w1_codes"][0], a["hot_w1_scales"][0], 64)
    W2 = _bits_w2(a["w2_codes"][0], a["w2_scales"][0], 32) + _bits_mxfp4(a["hot_w2_codes"][0], a["hot_w2_scales"][0], 32)
    X = torch.from_numpy(F.bf16_value(b["x"]))
    h = torch.nn.functional.linear(X, torch.from_numpy(W1))
    h = torch.nn.functional.silu(h[:, :32]) * h[:, 32:]
    y = torch.nn.functional.linear(h, torch.from_numpy(W2)).numpy()
    np.testing.assert_allclose(res["out"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    # the residual matters: without it the output moves
    plain = M.Layer("w2", {k_: v for k_, v in a.items() if not k_.startswith("hot_")})
    r0 = M.layer_forward(plain, b["logits"][:, :1], b["x"], 1)
    assert np.max(np.abs(r0["out"] - res["out"])) > 1e-3 * np.abs(y).max()


def test_residual_experts_compute_without_fp8_activations():
    sp, lay = _residual_layer()
    e = int(lay.a["hot_ids"][0])
    assert not lay.is_fp8(e) and e in lay.hot
    rep = M.Layer("w2", lay.a, hot_mode="replace")
    assert rep.is_fp8(e)
