"""Pins of the oracle's quantisers (oracle/quant.py) against brute force, closed forms and
invariants that do not reuse its own formulas."""
import numpy as np

from oracle import formats as F
from oracle import quant as Q


def _bf16(v):
    """exact bf16 values as fp32 (v must already be bf16-representable)"""
    return np.asarray(v, dtype=np.float32)


def _codes_of(words):
    """2-bit codes of u32 words, written as a bit loop (not the oracle's unpacking)."""
    words = np.asarray(words, dtype=np.uint32)
    out = np.zeros(words.shape[:-1] + (words.shape[-1] * 16,), dtype=np.int64)
    for j in range(words.shape[-1]):
        for i in range(16):
            out[..., 16 * j + i] = (words[..., j] >> np.uint32(2 * i)) & 3
    return out


def test_w2_exactly_representable_groups_come_back_exactly():
    rng = np.random.default_rng(1)
    lev = np.array([-4.0, -1.0, 1.0, 4.0])
    for _ in range(20):
        s = float(np.float32(rng.uniform(0.004, 0.03)))
        s = float((np.array([s], np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)[0])  # bf16
        c = rng.integers(0, 4, size=(3, 64))
        c[:, 0], c[:, 1], c[:, 32], c[:, 33] = 0, 2, 3, 1   # every group has a +-4 and a +-1
        w = (lev[c] * s).astype(np.float32)
        codes, scales = Q.quantize_w2(w)
        assert np.array_equal(_codes_of(codes), c)
        assert np.all(F.bf16_value(scales) == s)
        assert np.array_equal(F.dequant_w2(codes, scales), w.astype(np.float64))


def test_w2_nearest_level_matches_brute_force():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((500, 32)).astype(np.float32)
    s = np.abs(rng.standard_normal(500)).astype(np.float32) + np.float32(0.1)
    c = Q.w2_assign(w, s)
    lev = np.array([-4.0, -1.0, 1.0, 4.0])
    d = np.abs(w.astype(np.float64)[..., None] - lev * s.astype(np.float64)[:, None, None])
    # no exact ties in random data: the nearest level is unique
    assert np.array_equal(c, np.argmin(d, axis=-1))


def test_w2_tie_and_zero_rules():
    s = np.array([1.0], np.float32)
    w = np.array([[2.5, -2.5, 0.0, -0.0, 2.5000002, -2.5000002, 1e-30, -1e-30] + [0.5] * 24], np.float32)
    c = Q.w2_assign(w, s)[0, :8]
    assert list(c) == [2, 1, 2, 2, 3, 0, 2, 1]


def test_w2_refit_is_the_least_squares_scale():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((50, 32)).astype(np.float32)
    c = rng.integers(0, 4, size=(50, 32))
    s = Q.w2_refit(w, c).astype(np.float64)
    lev = np.array([-4.0, -1.0, 1.0, 4.0])[c]
    # the derivative of sum (w - lev s)^2 vanishes at the optimum: compare with lstsq
    for g in range(50):
        opt = np.linalg.lstsq(lev[g][:, None], w[g].astype(np.float64), rcond=None)[0][0]
        assert abs(s[g] - opt) <= 1e-6 * abs(opt)


def test_w2_each_round_does_not_increase_the_error():
    rng = np.random.default_rng(4)
    g = (rng.standard_normal((300, 32)) * rng.uniform(0.01, 3, (300, 1))).astype(np.float32)
    lev = np.array([-4.0, -1.0, 1.0, 4.0])
    s = (np.max(np.abs(g), axis=1) / 4).astype(np.float32)
    prev = None
    for _ in range(Q.W2_ROUNDS):
        c = Q.w2_assign(g, s)
        err_assign = np.sum((g - lev[c] * s[:, None].astype(np.float64)) ** 2, axis=1)
        if prev is not None:
            assert np.all(err_assign <= prev * (1 + 1e-6) + 1e-30)
        s = Q.w2_refit(g, c)
        prev = np.sum((g - lev[c] * s[:, None].astype(np.float64)) ** 2, axis=1)
        assert np.all(prev <= err_assign * (1 + 1e-6) + 1e-30)


def test_w2_power_of_two_equivariance_and_sign_mirror():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    c0, s0 = Q.quantize_w2(w)
    c1, s1 = Q.quantize_w2(w * np.float32(8.0))
    assert np.array_equal(c0, c1)
    assert np.array_equal(F.bf16_value(s1), 8.0 * F.bf16_value(s0))
    c2, s2 = Q.quantize_w2(-w)
    assert np.array_equal(s2, s0)
    assert np.array_equal(_codes_of(c2), 3 - _codes_of(c0))


def test_w2_zero_group():
    w = np.zeros((2, 64), np.float32)
    w[1, 32:] = np.float32(0.5)
    codes, scales = Q.quantize_w2(w)
    assert np.all(_codes_of(codes)[0] == 2) and np.all(_codes_of(codes)[1, :32] == 2)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 0] == 0
    # a constant group is represented exactly (+4 at scale 1/8 or +1 at scale 1/2)
    assert np.all(F.dequant_w2(codes, scales)[1, 32:] == 0.5)


def test_w2_quality_on_gaussian_weights():
    # the optimal symmetric 4-level quantiser of N(0,1) has an SQNR near 9.3 dB; the
    # {-4,-1,1,4} codebook with a per-32 scale lands close to it
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    d = F.dequant_w2(*Q.quantize_w2(w))
    cos = float(np.sum(d * w) / np.linalg.norm(d) / np.linalg.norm(w))
    assert 0.92 < cos < 0.96


def test_bf16_rne():
    v = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -3.0e-3], np.float32)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81]   # tie to even (down), tie to even (up), above tie
    got = Q.bf16_rne_bits(v)
    assert list(got[:4]) == want
    assert abs(F.bf16_value(got[4:])[0] + 3.0e-3) <= 2**-17   # half an ulp in [2^-9, 2^-8)


def test_e2m1_round_brute_force_and_ties():
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    # every tie between neighbours goes to the even mantissa field (nibble bit 0 == 0)
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, want in ties.items():
        for sg in (1.0, -1.0):
            n = int(Q.e2m1_round(np.array([sg * x]))[0])
            assert F.e2m1_value(n) == sg * want
    x = np.random.default_rng(7).uniform(-8, 8, 5000)
    n = Q.e2m1_round(x)
    v = F.e2m1_value(n)
    near = np.sign(x) * mags[np.argmin(np.abs(np.minimum(np.abs(x), 6.0)[:, None] - mags), axis=1)]
    assert np.array_equal(v, near)
    assert F.e2m1_value(Q.e2m1_round(np.array([-0.0, 7.0, -100.0]))).tolist() == [-0.0, 6.0, -6.0]


def test_mxfp4_worked_blocks():
    w = np.zeros((1, 64), np.float32)
    w[0, :32] = 1.0                 # amax 1 -> shared -2, 1 / 0.25 = 4
    w[0, 32] = 6.0                  # amax 6 -> shared 0
    w[0, 33] = -0.25                # tie between 0 and 0.5 -> -0
    w[0, 34] = 0.75                 # tie -> 1.0
    codes, scales = Q.quantize_mxfp4(w)
    assert scales.tolist() == [[125, 127]]
    assert codes[0, 0] == 0x66 and codes[0, 16] == (0x07 | (0x08 << 4)) and (codes[0, 17] & 0xF) == 0x2


def test_mxfp4_round_trip_and_quality():
    rng = np.random.default_rng(8)
    n = rng.integers(0, 16, (4, 64)).astype(np.uint8)
    codes = (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(118, 124, (4, 2)).astype(np.uint8)
    w = F.dequant_mxfp4(codes, scales).astype(np.float32)
    d = F.dequant_mxfp4(*Q.quantize_mxfp4(w))
    assert np.array_equal(d, w.astype(np.float64))   # representable tensors come back exactly
    w = (rng.standard_normal((32, 512)) * 0.02).astype(np.float32)
    d = F.dequant_mxfp4(*Q.quantize_mxfp4(w))
    assert float(np.sum(d * w) / np.linalg.norm(d) / np.linalg.norm(w)) > 0.98


def _bf16_rne_fp64(v):
    """fp64 -> nearest bf16 value (8 significant bits, ties to even), computed from the
    exponent and np.round (half to even) rather than from bit patterns."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    e = np.floor(np.log2(np.abs(v[nz])))
    ulp = np.exp2(e - 7)
    out[nz] = np.round(v[nz] / ulp) * ulp
    return out


def _w2_chain_fp64(g, rounds):
    """The fit written independently of the oracle: brute-force nearest level (argmin over the
    four levels) and a least-squares scale from numpy's lstsq, in fp64, `rounds` times from
    s = max|w| / 4.  Returns the last scale, the last codes and the smallest relative distance
    of any weight to a decision threshold over the rounds (to set aside near-ties)."""
    lev = np.array([-4.0, -1.0, 1.0, 4.0])
    gd = g.astype(np.float64)
    s = np.max(np.abs(gd), axis=1) / 4.0
    c = None
    margin = np.full(len(g), np.inf)
    for _ in range(rounds):
        d = np.abs(gd[..., None] - lev * s[:, None, None])
        c = np.argmin(d, axis=-1)
        ds = np.sort(d, axis=-1)
        margin = np.minimum(margin, np.min((ds[..., 1] - ds[..., 0]) / np.abs(s)[:, None], axis=1))
        s = np.array([np.linalg.lstsq(lev[c[i]][:, None], gd[i], rcond=None)[0][0] for i in range(len(g))])
    return s, c, margin


def test_w2_stored_scale_and_final_codes_against_an_independent_fit():
    """quantize_w2 returns (a) the bf16 (nearest even) of the least-squares scale refitted on the
    codes of round 3, and (b) codes that are the nearest levels of w against that *stored* bf16
    scale.  Both are checked against a fit written here from brute force and lstsq, and the data
    is chosen so that two or four rounds, or keeping round 3's codes, would give other results."""
    rng = np.random.default_rng(9)
    G = 3000
    base = rng.standard_normal((G, 32))
    heavy = rng.standard_t(2.0, size=(G, 32))            # heavy tails: rounds keep moving codes
    g = np.where(rng.uniform(size=(G, 1)) < 0.5, base, heavy) * rng.uniform(0.005, 0.05, (G, 1))
    g = g.astype(np.float32)
    codes, scales = Q.quantize_w2(g)
    got_s = F.bf16_value(scales.reshape(-1))
    got_c = _codes_of(codes.reshape(G, 2))
    lev = np.array([-4.0, -1.0, 1.0, 4.0])
    s3, c3, margin = _w2_chain_fp64(g, 3)
    want_s = _bf16_rne_fp64(s3)
    # set aside groups where fp32 and fp64 arithmetic could round a decision differently: a weight
    # within 1e-5 (relative to s) of a threshold in some round, or s3 near a bf16 rounding midpoint
    e = np.floor(np.log2(np.abs(s3)))
    frac = np.abs(s3) / np.exp2(e - 7)
    near_mid = np.abs(frac - np.floor(frac) - 0.5) < 1e-4
    keep = (margin > 1e-5) & ~near_mid
    assert keep.mean() > 0.99
    assert np.array_equal(got_s[keep], want_s[keep])
    # (b) final codes: brute-force nearest level against the stored scale
    d = np.abs(g.astype(np.float64)[..., None] - lev * got_s[:, None, None])
    ds = np.sort(d, axis=-1)
    clear = np.min(ds[..., 1] - ds[..., 0], axis=1) > 0   # no exact tie in the group
    assert clear.mean() > 0.99
    assert np.array_equal(got_c[clear], np.argmin(d, axis=-1)[clear])
    # the pin's power: on this data the round count and the final reassignment both matter
    s2, _, _ = _w2_chain_fp64(g, 2)
    s4, _, _ = _w2_chain_fp64(g, 4)
    assert np.sum(_bf16_rne_fp64(s2)[keep] != want_s[keep]) > 10
    assert np.sum(_bf16_rne_fp64(s4)[keep] != want_s[keep]) > 10
    assert np.sum(np.any(c3 != got_c, axis=1)) > 10
