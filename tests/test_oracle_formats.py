"""Pins of the oracle's format decoders/encoders against worked examples, exhaustive
tables, brute force and an independent library (torch's fp8/bf16 dtypes)."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "formats.txt")


def _golden():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        kind, words = lhs.split()
        vals = [float(v) for v in rhs.split(",")]
        out.append((kind, [int(w, 16) for w in words.split(",")], vals))
    return out


@pytest.mark.parametrize("kind,words,vals", _golden())
def test_golden(kind, words, vals):
    if kind == "w2":
        got = F.dequant_w2(np.array([words * 2], np.uint32), np.array([[0x3F80]], np.uint16))
        np.testing.assert_array_equal(got[0, :16], vals)
        np.testing.assert_array_equal(got[0, 16:], vals)
    elif kind == "w3":
        # scale byte 0x38 = 1.0 and the /64 divisor: decoded value = level / 64
        got = F.dequant_w3(np.array([words * 2], np.uint32), np.array([[0x38]], np.uint8))
        np.testing.assert_array_equal(got[0, :32] * 64, vals)
        np.testing.assert_array_equal(got[0, 32:] * 64, vals)
    elif kind == "e4m3":
        assert F.e4m3fn_value(words[0]) == vals[0]
    elif kind == "e8m0":
        assert F.e8m0_value(words[0]) == vals[0]
    elif kind == "e2m1":
        assert F.e2m1_value(words[0]) == vals[0]
    else:
        raise AssertionError(kind)


def _pack_w2_python(codes):
    """Independent packer: Python ints, code i of a word at bits 2i."""
    words = []
    for w in range(len(codes) // 16):
        v = 0
        for i in range(16):
            v |= int(codes[16 * w + i]) << (2 * i)
        words.append(v)
    return words


def _pack_w3_python(codes):
    words = []
    for g in range(len(codes) // 32):
        v = 0
        for i in range(32):
            v |= int(codes[32 * g + i]) << (3 * i)
        words += [(v >> (32 * j)) & 0xFFFFFFFF for j in range(3)]
    return words


def test_w2_random_roundtrip_against_python_packer():
    r = np.random.default_rng(1)
    rows, K = 3, 128
    codes = r.integers(0, 4, size=(rows, K))
    scales_f = r.uniform(-2, 2, size=(rows, K // 32)).astype(np.float32)
    sbits = torch.from_numpy(scales_f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    packed = np.array([_pack_w2_python(c) for c in codes], np.uint32)
    got = F.dequant_w2(packed, sbits)
    s = torch.from_numpy(sbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    want = np.array([-4.0, -1.0, 1.0, 4.0])[codes] * np.repeat(s, 32, axis=1)
    np.testing.assert_array_equal(got, want)


def test_w3_random_roundtrip_against_python_packer():
    r = np.random.default_rng(2)
    rows, K = 4, 192
    codes = r.integers(0, 8, size=(rows, K))
    packed = np.array([_pack_w3_python(c) for c in codes], np.uint32)
    np.testing.assert_array_equal(F.unpack_w3_codes(packed), codes)
    sb = r.integers(0, 0x7F, size=(rows, K // 64)).astype(np.uint8)
    got = F.dequant_w3(packed, sb)
    s = torch.from_numpy(sb).view(torch.float8_e4m3fn).double().numpy() / 64
    want = np.array([-8.0, -5, -3, -1, 1, 3, 5, 8])[codes] * np.repeat(s, 64, axis=1)
    np.testing.assert_array_equal(got, want)


def test_e4m3_all_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    mine = F.e4m3fn_value(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_e8m0_and_e2m1_tables():
    b = np.arange(255, dtype=np.uint8)
    np.testing.assert_array_equal(F.e8m0_value(b), [2.0 ** (i - 127) for i in range(255)])
    assert np.isnan(F.e8m0_value(255))
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for n in range(16):
        v = F.e2m1_value(n)
        assert abs(v) == mags[n & 7] and bool(np.signbit(v)) == bool(n & 8)


def test_e4m3_encode_roundtrip_all_finite():
    b = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(F.e4m3fn_encode(F.e4m3fn_value(b)), b)


def _finite_e4m3_grid():
    b = np.array([i for i in range(128) if i != 0x7F], np.uint8)
    return F.e4m3fn_value(b), b


def test_e4m3_encode_brute_force_nearest_even():
    """Brute force: the encoded value is the nearest grid value; at an exact tie the
    one with the even mantissa field wins; beyond 448 it saturates."""
    vals, bytes_ = _finite_e4m3_grid()
    r = np.random.default_rng(3)
    # random values, exact midpoints and saturating values
    mids = (vals[1:] + vals[:-1]) / 2
    xs = np.concatenate([r.uniform(-500, 500, 400), r.uniform(-1, 1, 400) * 2.0 ** r.integers(-12, 9, 400),
                         mids, -mids, [449.0, 464.0, 465.0, 1e6, -1e6, 0.0, -0.0]])
    enc = F.e4m3fn_encode(xs)
    for x, e in zip(xs, enc):
        a = min(abs(x), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        if len(best) == 2:
            best = [i for i in best if bytes_[i] % 2 == 0]
        want = bytes_[best[0]] | (0x80 if np.signbit(x) else 0)
        assert e == want, (x, hex(e), hex(want))


def test_e4m3_encode_matches_torch_in_range():
    r = np.random.default_rng(4)
    xs = (r.standard_normal(20000) * 2.0 ** r.integers(-10, 8, 20000)).astype(np.float32)
    xs = np.clip(xs, -448, 448)
    mine = F.e4m3fn_encode(xs.astype(np.float64))
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_bf16_value_matches_torch():
    b = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    mine = F.bf16_value(b)
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])


# ------------------------------------------------------------ exactness invariants
def test_w2_dequant_exact_in_bf16_for_all_scales():
    """{+-1, +-4} x every finite bf16 scale below 2^125 is a bf16 value: the dequantised
    2-bit weights have no rounding, so GPU and oracle must agree bit for bit."""
    s = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    sv = F.bf16_value(s)
    ok = np.isfinite(sv) & (np.abs(sv) < 2.0**125)
    prod = np.outer(sv[ok], [-4.0, -1.0, 1.0, 4.0]).reshape(-1)
    back = torch.from_numpy(prod).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(back, prod)


def test_w3_dequant_exact_in_bf16_for_all_scales():
    b = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], np.uint8)
    prod = np.outer(F.e4m3fn_value(b) / 64, [-8.0, -5, -3, -1, 1, 3, 5, 8]).reshape(-1)
    back = torch.from_numpy(prod).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(back, prod)


def test_mxfp4_to_fp8_is_lossless_and_keeps_scales():
    codes = np.arange(256, dtype=np.uint8).reshape(4, 64)
    scales = np.array([[120, 121, 5, 250], [127, 0, 127, 127], [254, 3, 100, 130], [121, 120, 121, 120]], np.uint8)
    elems, sc = F.mxfp4_to_fp8(codes, scales)
    assert elems.shape == (4, 128) and elems.dtype == np.uint8
    np.testing.assert_array_equal(sc, scales)
    np.testing.assert_array_equal(F.dequant_fp8(elems, sc), F.dequant_mxfp4(codes, scales))
    # the element map, nibble by nibble, including -0 -> 0x80
    nib = np.arange(16, dtype=np.uint8)
    packed = np.tile(nib[0::2] | (nib[1::2] << 4), 2).reshape(1, 16)
    e, _ = F.mxfp4_to_fp8(packed, np.array([[127]], np.uint8))
    # hand-derived e4m3fn bytes of 0, .5, 1, 1.5, 2, 3, 4, 6 and their negatives
    want = [0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C,
            0x80, 0xB0, 0xB8, 0xBC, 0xC0, 0xC4, 0xC8, 0xCC]
    np.testing.assert_array_equal(e[0], want * 2)


def test_mxfp4_nibble_order():
    codes = np.array([[0x21] * 16], np.uint8)  # low nibble 1 (0.5), high nibble 2 (1.0)
    v = F.dequant_mxfp4(codes, np.array([[127]], np.uint8))
    np.testing.assert_array_equal(v[0, 0::2], 0.5)
    np.testing.assert_array_equal(v[0, 1::2], 1.0)


# ------------------------------------------------------------------------ MXFP8
def test_mxfp8_scale_rule_closed_cases():
    def q(block):
        e, s = F.mxfp8_quantize(np.array([block], np.float64))
        return e[0], int(s[0, 0])
    blk = np.zeros(32)
    blk[5] = 1.0
    e, s = q(blk)           # amax 1 = 2^0 -> shared exponent -8
    assert s == 127 - 8 and e[5] == F.e4m3fn_encode(256.0)
    blk[5] = 448.0          # floor(log2 448) = 8 -> shared 0, element 448 exactly
    e, s = q(blk)
    assert s == 127 and e[5] == 0x7E
    blk[5] = 511.0          # floor(log2 511) = 8 -> 511 saturates to 448
    e, s = q(blk)
    assert s == 127 and e[5] == 0x7E
    e, s = q(np.zeros(32))  # all-zero block
    assert s == 0 and np.all(e == 0)


def test_mxfp8_brute_force_blocks():
    vals, bytes_ = _finite_e4m3_grid()
    r = np.random.default_rng(5)
    x = r.standard_normal((3, 64)) * np.array([[1e-3], [1.0], [40.0]])
    e, s = F.mxfp8_quantize(x)
    for row in range(3):
        for b in range(2):
            blk = x[row, 32 * b: 32 * b + 32]
            amax = np.max(np.abs(blk))
            shared = int(np.floor(np.log2(amax))) - 8
            assert int(s[row, b]) == shared + 127
            for i in range(32):
                a = min(abs(blk[i]) / 2.0**shared, 448.0)
                d = np.abs(vals - a)
                best = np.flatnonzero(d == d.min())
                if len(best) == 2:
                    best = [j for j in best if bytes_[j] % 2 == 0]
                want = bytes_[best[0]] | (0x80 if blk[i] < 0 else 0)
                assert e[row, 32 * b + i] == want
    back = F.mxfp8_dequant(e, s)
    scale = np.repeat(np.exp2(s.astype(float) - 127), 32, axis=1)
    sat = np.abs(x) / scale > 448
    # saturated elements become +-448 * 2^shared
    np.testing.assert_array_equal(back[sat], np.sign(x[sat]) * 448 * scale[sat])
    # others: half an ulp of 3 mantissa bits (2^-4 relative) or, in the subnormal
    # range, half the subnormal step 2^-9 (absolute, times the block scale)
    bound = np.maximum(np.abs(x) * 2.0**-4, 2.0**-10 * scale)
    assert np.all(np.abs(back - x)[~sat] <= bound[~sat])
