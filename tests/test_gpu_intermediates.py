"""GPU: intermediate results of moe_expert_ffn read back from its workspace and compared with
the oracle ([Day0-MXFP4] section 4: the online conversion is checked on fixed inputs;
[Moet-README] release notes of -r23: FC1 + SwiGLU + MXFP8 quantisation of h, then FC2).

* the MXFP8 of x (the FP8 FC1 input of hot experts): bit-exact, it is fixed by the bf16 x;
* the FP8 slot image the convert stage writes: bit-exact against the oracle's MXFP4 -> FP8,
  for every hot expert with rows, and untouched for hot experts without rows;
* the MXFP8 of h that the FP8 FC1 epilogue writes: the GPU forms h in fp32 from the matrix
  cores' sums, the oracle in fp64, so a value lying next to a rounding midpoint of e4m3 (or an
  amax next to a power of two) may round the other way: at most 1e-4 of the elements (and of the
  scales) may differ, and every differing element is one e4m3 step from the oracle's.

Stages of moe_expert_ffn with a hot set: 0-4 the low-bit stages, 5 hot prepare (work list,
MXFP8 of x), then per batch of S hot experts: 6 + 3b convert, 7 + 3b FP8 FC1, 8 + 3b FP8 FC2."""
import numpy as np
import pytest
import torch

import moegen
from oracle import formats as OF
from oracle import moe as OM

from _helpers import device_layer, fp8_h_bound, host, layer_arrays, oracle_layer, to_dev

pytestmark = pytest.mark.gpu

MIXED_SMALL = {"E": 16, "k": 4, "H": 256, "I": 512, "n_hot": 4}
FILL = 0xA5  # the workspace is filled with this byte before the call


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


def _run_stages(L, dw, x, k, ids, last_stage, fp8_slots=None):
    """moe_permute, then stages 0 .. last_stage of moe_expert_ffn on a workspace filled with FILL."""
    counts, offsets, perm, inv = L.moe_permute(ids, dw.E)
    T = x.shape[0]
    slots = dw.n_hot if fp8_slots is None else fp8_slots
    nbytes = L.moe_expert_ffn_ws_bytes(dw, T, k, slots)
    ws = torch.full((nbytes,), FILL, dtype=torch.uint8, device="cuda")
    y = torch.zeros((T * k, dw.H), dtype=torch.float32, device="cuda")
    assert last_stage < L.moe_expert_ffn_num_stages(dw, T, k, nbytes)
    for st in range(last_stage + 1):
        L.moe_expert_ffn_stage(dw, x, k, counts, offsets, perm, y, ws, st)
    torch.cuda.synchronize()
    return ws, host(counts), host(offsets), host(perm)


def _region(L, dw, T, k, ws, region):
    off, n = L.moe_expert_ffn_ws_region(dw, T, k, ws.numel(), region)
    return host(ws[off:off + n])


def _ids_without(sp, T, missing, seed=5):
    """Routed ids of T tokens (distinct per token) that never pick the experts in `missing`."""
    r = np.random.default_rng(seed)
    allowed = np.array([e for e in range(sp["E"]) if e not in set(missing)])
    return np.stack([r.choice(allowed, size=sp["k"], replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("name,T,override", [("mixed", 300, MIXED_SMALL), ("mixed", 64, {})])
def test_xq_bit_exact(L, name, T, override):
    sp, dw = device_layer(name, **override)
    b = moegen.batch(sp, T)
    ids, _ = OM.route(b["logits"], sp["k"])
    ws, *_ = _run_stages(L, dw, to_dev(b["x"]), sp["k"], to_dev(ids), 5)
    we, wsc = OF.mxfp8_quantize(OF.bf16_value(b["x"]))
    np.testing.assert_array_equal(_region(L, dw, T, sp["k"], ws, L.MOE_WS_XQ).reshape(T, sp["H"]), we)
    np.testing.assert_array_equal(_region(L, dw, T, sp["k"], ws, L.MOE_WS_XQ_SCALES).reshape(T, -1), wsc)


@pytest.mark.parametrize("fp8_slots", [None, 1, 3])
def test_fp8_slot_image_bit_exact(L, fp8_slots):
    """Every hot expert with rows is converted into its slot of its batch, bit for bit; the slot
    of a hot expert without rows is not written (the convert stage skips it)."""
    sp, dw = device_layer("mixed", **MIXED_SMALL)
    _, arrays = layer_arrays("mixed", **MIXED_SMALL)
    hot = arrays["hot_ids"]
    T, k = 40, sp["k"]
    b = moegen.batch(sp, T)
    ids = _ids_without(sp, T, [int(hot[1])])       # hot expert of slot position 1 gets no rows
    layout = L.moe_fp8_slot_layout(sp["H"], sp["I"])
    S = sp["n_hot"] if fp8_slots is None else fp8_slots
    n_batches = (sp["n_hot"] + S - 1) // S
    want = {}
    for which in (1, 2):
        for s in range(sp["n_hot"]):
            want[which, s] = OF.mxfp4_to_fp8(arrays[f"hot_w{which}_codes"][s], arrays[f"hot_w{which}_scales"][s])
    for bt in range(n_batches):
        ws, counts, _, _ = _run_stages(L, dw, to_dev(b["x"]), k, to_dev(ids), 6 + 3 * bt, fp8_slots)
        assert counts[hot[1]] == 0 and all(counts[e] > 0 for i, e in enumerate(hot) if i != 1)
        slots = _region(L, dw, T, k, ws, L.MOE_WS_SLOTS)
        assert slots.size == S * layout["slot_bytes"]
        for j in range(S):
            # slot j holds the image of the latest batch <= bt whose expert there has rows
            writer = [bb * S + j for bb in range(bt + 1) if bb * S + j < sp["n_hot"] and counts[hot[bb * S + j]] > 0]
            img = slots[j * layout["slot_bytes"]:(j + 1) * layout["slot_bytes"]]
            for which, rows, K in ((1, 2 * sp["I"], sp["H"]), (2, sp["H"], sp["I"])):
                key = f"w{which}"
                el = img[layout[key]:layout[key] + rows * K].reshape(rows, K)
                sc = img[layout[key + "_scales"]:layout[key + "_scales"] + rows * (K // 32)].reshape(rows, -1)
                if not writer:
                    assert np.all(el == FILL) and np.all(sc == FILL), (bt, j, which)
                    continue
                we, wsc = want[which, writer[-1]]
                np.testing.assert_array_equal(el, we, err_msg=f"batch {bt} slot {j} expert {writer[-1]} W{which}")
                np.testing.assert_array_equal(sc, wsc, err_msg=f"batch {bt} slot {j} expert {writer[-1]} W{which} s")


def _hq_oracle(lay, x_bits, k, I, rows, perm, offsets):
    """The oracle's h (fp64) for the given grouped rows of hot experts -- x quantised to MXFP8,
    FC1 with the expert's FP8 image, SwiGLU -- and the bound dh of fp8_h_bound."""
    X = OF.bf16_value(x_bits)
    Xq = OF.mxfp8_dequant(*OF.mxfp8_quantize(X))
    expert_of = np.searchsorted(offsets, rows, side="right") - 1
    h = np.zeros((len(rows), I))
    dh = np.zeros((len(rows), I))
    for e in sorted(set(expert_of.tolist())):
        sel = np.nonzero(expert_of == e)[0]
        h[sel], dh[sel] = fp8_h_bound(Xq[perm[rows[sel]] // k], lay.dense(e, 1))
    return h, dh


# Reading of the h_q bar.  The matrix cores' FP8 dot products are not exact fp32 sums: one
# v_mfma_scale_f32_32x32x64_f8f6f4 on random e4m3 operands deviated from the exact sum of its 64
# products by up to 3.2e-4 of the rms of such sums (measured on the device), far above fp32
# rounding.  So a value of h that close to an e4m3 rounding midpoint may round the other way:
# measured on a few 1e-4 of the elements, not the 1e-4 an IEEE fp32 sum would give.  The test
# bounds the rate at 1e-3 and checks that every difference is one the arithmetic explains: the
# oracle's exact h lies within the error bound dh (KAPPA = 1e-3, three times the largest
# deviation measured) of the values that round to the GPU's element.  A block scale may differ only where the oracle's amax lies within dh of a
# power of two, and on at most 1e-4 of the blocks.
HQ_RATE = 1e-3


def _e4m3_grid():
    vals = OF.e4m3fn_value(np.arange(256, dtype=np.uint8))
    return np.unique(vals[np.isfinite(vals)])


def _check_hq(h, dh, hq, hqs):
    """The h_q bar above; returns (element rate, differing elements, differing scales)."""
    we, wsc = OF.mxfp8_quantize(h)
    n, I = h.shape
    # scales: the shared exponent follows floor(log2 amax); a difference needs amax next to 2^e
    bad_s = hqs != wsc
    hb, db = np.abs(h.reshape(n, I // 32, 32)), dh.reshape(n, I // 32, 32)
    amax = np.max(hb, axis=-1)
    slack = db[np.arange(n)[:, None], np.arange(I // 32)[None, :], np.argmax(hb, axis=-1)]
    p2 = np.exp2(np.round(np.log2(np.where(amax > 0, amax, 1.0))))
    assert bad_s.mean() <= 1e-4, bad_s.mean()
    assert np.all(np.abs(amax - p2)[bad_s] <= slack[bad_s]), (amax[bad_s], slack[bad_s])
    # elements of the blocks whose scales agree (-0 and +0 are the same value)
    same = np.repeat(~bad_s, 32, axis=1)
    bad_e = (OF.e4m3fn_value(hq) != OF.e4m3fn_value(we)) & same
    rate = bad_e.sum() / max(1, same.sum())
    assert rate <= HQ_RATE, rate
    # the oracle's exact h must lie within dh of the interval of values that round to the GPU's
    # element (between the midpoints to its neighbours; e4m3 saturates beyond +-448)
    grid = _e4m3_grid()
    sc = np.exp2(np.repeat(wsc.astype(np.float64) - 127.0, 32, axis=1))[bad_e]
    gi = np.searchsorted(grid, OF.e4m3fn_value(hq[bad_e]))
    lo = np.where(gi > 0, (grid[np.maximum(gi - 1, 0)] + grid[gi]) / 2, -np.inf) * sc
    hi = np.where(gi < grid.size - 1, (grid[np.minimum(gi + 1, grid.size - 1)] + grid[gi]) / 2, np.inf) * sc
    v = h[bad_e]
    dist = np.maximum(lo - v, 0) + np.maximum(v - hi, 0)
    assert np.all(dist <= dh[bad_e]), (dist / dh[bad_e]).max()
    return rate, int(bad_e.sum()), int(bad_s.sum())


@pytest.mark.parametrize("name,T,override,n_rows", [("mixed", 300, MIXED_SMALL, None), ("mixed", 64, {}, None),
                                                    ("mixed", 4096, {}, 1024)])
def test_hq_matches_oracle(L, name, T, override, n_rows):
    sp, dw = device_layer(name, **override)
    lay = oracle_layer(name, **override)
    _, arrays = layer_arrays(name, **override)
    hot = arrays["hot_ids"]
    k, I = sp["k"], sp["I"]
    b = moegen.batch(sp, T)
    ids, _ = OM.route(b["logits"], k)
    ws, counts, offsets, perm = _run_stages(L, dw, to_dev(b["x"]), k, to_dev(ids), 7)
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in hot])
    if n_rows is not None and rows.size > n_rows:
        rows = np.sort(np.random.default_rng(T).choice(rows, n_rows, replace=False))
    hq = _region(L, dw, T, k, ws, L.MOE_WS_HQ).reshape(T * k, I)[rows]
    hqs = _region(L, dw, T, k, ws, L.MOE_WS_HQ_SCALES).reshape(T * k, I // 32)[rows]
    h, dh = _hq_oracle(lay, b["x"], k, I, rows, perm, offsets)
    rate, n_e, n_s = _check_hq(h, dh, hq, hqs)
    print(f"{name} T={T}: {rows.size} hot rows, h_q elements differing {n_e} ({rate:.2e}), scales {n_s}",
          flush=True)
