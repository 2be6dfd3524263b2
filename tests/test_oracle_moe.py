"""Pins of the oracle's routing, grouping, expert FFN and combine: brute force on tiny
inputs, closed forms, special cases that reduce to a dense MLP, and the expert-sum
identity.  None of these re-types the oracle's own formula."""
import math

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
