"""GPU parity of the quantisers (moe_quantize_w2, moe_quantize_mxfp4) against the oracle's
(oracle/quant.py): codes and scales bit for bit, on seeded weights with ragged row counts,
several kernel blocks, and the special values (zero groups, -0, subnormals, huge values,
exactly representable groups, e2m1 rounding ties)."""
import numpy as np
import pytest
import torch

import moegen
from oracle import formats as OF
from oracle import quant as OQ

from _helpers import host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_moe_expert_top_amd import _lib

    return _lib


def special_rows(K: int) -> np.ndarray:
    """Rows of edge cases, K a multiple of 64."""
    rows = []
    rows.append(np.zeros(K, np.float32))                         # all-zero groups
    rows.append(-np.zeros(K, np.float32))                        # -0
    r = np.full(K, 0.01, np.float32); r[::7] = -0.0; rows.append(r)
    rows.append(np.full(K, 1e-40, np.float32) * np.where(np.arange(K) % 3 == 0, -1, 1).astype(np.float32))
    r = (np.arange(K, dtype=np.float32) - K / 2) * np.float32(1e30); rows.append(r)   # huge
    lev = np.array([-4.0, -1.0, 1.0, 4.0], np.float32)
    c = np.arange(K) % 4
    rows.append(lev[c] * np.float32(0.0078125))                  # exactly representable groups
    # e2m1 ties inside a block whose amax (6 * 2^-3) fixes the shared exponent at -3
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32) * np.float32(0.125)
    r = np.resize(np.concatenate([t, -t]), K).astype(np.float32); rows.append(r)
    return np.stack(rows).astype(np.float32)


CASES = [(1, 32, 0), (3, 96, 1), (257, 512, 2), (64, 4096, 3)]


@pytest.mark.parametrize("rows,K,seed", CASES)
def test_quantize_w2_bit_exact(L, rows, K, seed):
    w = moegen.float_weights(rows, K, seed)
    if K % 64 == 0:
        w = np.concatenate([w, special_rows(K)])
    codes, scales = L.moe_quantize_w2(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    wc, ws = OQ.quantize_w2(w)
    got_c, got_s = host(codes).view(np.uint32), host(scales).view(np.uint16)
    assert np.array_equal(got_s, ws), np.argwhere(got_s != ws)[:5]
    assert np.array_equal(got_c, wc), np.argwhere(got_c != wc)[:5]


@pytest.mark.parametrize("rows,K,seed", CASES)
def test_quantize_mxfp4_bit_exact(L, rows, K, seed):
    w = moegen.float_weights(rows, K, seed)
    if K % 64 == 0:
        w = np.concatenate([w, special_rows(K)])
    codes, scales = L.moe_quantize_mxfp4(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    wc, ws = OQ.quantize_mxfp4(w)
    got_c, got_s = host(codes), host(scales)
    assert np.array_equal(got_s, ws), np.argwhere(got_s != ws)[:5]
    assert np.array_equal(got_c, wc), np.argwhere(got_c != wc)[:5]


def test_quantize_expert_shape_sampled(L):
    """One expert's W1 at the decode/prefill shape (2I x H = 4096 x 4096): every row on the
    GPU, sampled rows against the oracle, the whole matrix against the quality bound."""
    w = moegen.float_weights(4096, 4096, 11)
    dw = torch.from_numpy(w).cuda()
    codes, scales = L.moe_quantize_w2(dw)
    c4, s4 = L.moe_quantize_mxfp4(dw)
    torch.cuda.synchronize()
    rows = [0, 1, 2047, 4095]
    wc, ws = OQ.quantize_w2(w[rows])
    assert np.array_equal(host(codes).view(np.uint32)[rows], wc)
    assert np.array_equal(host(scales).view(np.uint16)[rows], ws)
    mc, ms = OQ.quantize_mxfp4(w[rows])
    assert np.array_equal(host(c4)[rows], mc) and np.array_equal(host(s4)[rows], ms)
    d = OF.dequant_w2(host(codes).view(np.uint32)[::64], host(scales).view(np.uint16)[::64])
    ref = w[::64].astype(np.float64)
    assert np.sum(d * ref) / np.linalg.norm(d) / np.linalg.norm(ref) > 0.92


def test_quantize_empty(L):
    for f in (L.moe_quantize_w2, L.moe_quantize_mxfp4):
        c, s = f(torch.empty((0, 64), dtype=torch.float32, device="cuda"))
        assert c.numel() == 0 and s.numel() == 0


def test_quantised_layer_end_to_end(L):
    """Float experts -> GPU quantiser -> the four calls, against the oracle on the same seeded
    float weights: the quantised codes and scales equal the oracle's bit for bit, and the layer
    on them is within the bf16 tolerance of the oracle layer on the oracle's codes."""
    from oracle import moe as OM
    from _helpers import TOL_BF16, max_err_over_rms

    E, k, H, I, T = 8, 2, 256, 512, 40
    w1 = np.stack([moegen.float_weights(2 * I, H, 100 + e) for e in range(E)])
    w2 = np.stack([moegen.float_weights(H, I, 200 + e) for e in range(E)])
    c1, s1 = L.moe_quantize_w2(torch.from_numpy(w1.reshape(E * 2 * I, H)).cuda())
    c2, s2 = L.moe_quantize_w2(torch.from_numpy(w2.reshape(E * H, I)).cuda())
    torch.cuda.synchronize()
    arrays = {"w1_codes": host(c1).view(np.uint32).reshape(E, 2 * I, H // 16),
              "w1_scales": host(s1).view(np.uint16).reshape(E, 2 * I, H // 32),
              "w2_codes": host(c2).view(np.uint32).reshape(E, H, I // 16),
              "w2_scales": host(s2).view(np.uint16).reshape(E, H, I // 32)}
    oc1, os1 = OQ.quantize_w2(w1.reshape(E * 2 * I, H))
    oc2, os2 = OQ.quantize_w2(w2.reshape(E * H, I))
    assert np.array_equal(arrays["w1_codes"].reshape(oc1.shape), oc1)
    assert np.array_equal(arrays["w1_scales"].reshape(os1.shape), os1)
    assert np.array_equal(arrays["w2_codes"].reshape(oc2.shape), oc2)
    assert np.array_equal(arrays["w2_scales"].reshape(os2.shape), os2)
    dw = L.DeviceWeights(1, E, H, I, arrays)
    sp = moegen.spec("tiny")
    b = moegen.batch(sp, T)
    res = L.layer_forward(dw, torch.from_numpy(b["logits"]).cuda(),
                          torch.from_numpy(b["x"].view(np.int16)).cuda(), k, out_fp32=True)
    want = OM.layer_forward(OM.Layer("w2", arrays), b["logits"], b["x"], k)
    assert max_err_over_rms(host(res["out"]), want["out"]) <= TOL_BF16
