"""CPU checks of the FP8 rounding-flip allowance the layer parity tests use: whatever h' within
dh of h a computation produces, its MXFP8 values lie within the allowance of the oracle's."""
import numpy as np

from oracle import formats as OF

from _helpers import mxfp8_flip_allowance


def _mx(v):
    return OF.mxfp8_dequant(*OF.mxfp8_quantize(v))


def test_allowance_covers_every_perturbation():
    r = np.random.default_rng(0)
    h = r.standard_normal((64, 256)) * np.exp2(r.integers(-6, 6, (64, 1)))
    dh = 1e-3 * np.abs(h).max(axis=1, keepdims=True) * np.ones_like(h)
    q, a = mxfp8_flip_allowance(h, dh)
    np.testing.assert_array_equal(q, _mx(h))
    assert 0 < (a > 0).mean() < 0.5
    for _ in range(20):
        hp = h + r.uniform(-1, 1, h.shape) * dh
        assert np.all(np.abs(_mx(hp) - q) <= a)
    for sgn in (-1.0, 1.0):  # the extremes of the interval
        assert np.all(np.abs(_mx(h + sgn * dh) - q) <= a)


def test_allowance_covers_a_block_scale_flip():
    r = np.random.default_rng(1)
    h = r.uniform(-1, 1, (2, 64))
    h[0, 5] = 2.0 - 1e-4             # the block's amax just below a power of two
    dh = np.full_like(h, 1e-3)
    q, a = mxfp8_flip_allowance(h, dh)
    hp = h.copy()
    hp[0, 5] = 2.0 + 1e-4            # ... and just above: the shared exponent moves up by one
    assert OF.mxfp8_quantize(hp)[1][0, 0] == OF.mxfp8_quantize(h)[1][0, 0] + 1
    assert np.all(np.abs(_mx(hp) - q) <= a)
    assert np.all(a[1] < a[0].max())  # the other rows are not widened


def test_zero_bound_gives_zero_allowance():
    h = np.random.default_rng(2).standard_normal((4, 64))
    q, a = mxfp8_flip_allowance(h, np.zeros_like(h))
    assert np.all(a == 0)
