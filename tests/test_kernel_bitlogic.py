"""Host emulation of the bit tricks the HIP kernels use, checked against the oracle's
decoders.  This is not the oracle: it re-expresses, in Python integers, the exact integer
operations of the device code (v_perm_b32 byte selection, shifts, masks), so a wrong
constant or shift is caught on the CPU."""
import numpy as np

import moegen
from oracle import formats as OF


def v_perm_b32(s0: int, s1: int, sel: int) -> int:
    """Byte j of the result = byte sel.byte[j] of the 64-bit value s0:s1 (s1 = bytes 0..3);
    selector 12 gives 0x00, 13..15 give 0xFF (the forms the kernels use are 0..7)."""
    data = ((s0 & 0xFFFFFFFF) << 32) | (s1 & 0xFFFFFFFF)
    out = 0
    for j in range(4):
        s = (sel >> (8 * j)) & 0xFF
        if s < 8:
            b = (data >> (8 * s)) & 0xFF
        elif s == 12:
            b = 0
        elif s >= 13:
            b = 0xFF
        else:
            raise AssertionError("sign-replicating selectors are not used")
        out |= b << (8 * j)
    return out


# --- 2-bit: the per-group byte tables and the decode of one word (lowbit_fmt.h) ---
def w2_table(sw):
    """Scale word sw (bf16 of group 0 low, group 1 high) -> the two groups' high-byte tables."""
    x = sw ^ 0x80008000
    return [(v_perm_b32(x, sw, sel) + 0x01000001) & 0xFFFFFFFF for sel in (0x01010505, 0x03030707)]


def w2_decode_word(w, lut, sw, g):
    """Eight dwords (two MFMA operands) from one word of group g: for s = 0..3 the high bytes
    of codes s, 4+s, 8+s, 12+s, then two interleaves with the group's low byte (byte 2g of sw)."""
    sel = (0x01040004, 0x03040204) if g == 0 else (0x01060006, 0x03060206)
    out = []
    for s in range(4):
        hb = v_perm_b32(0, lut, (w >> (2 * s)) & 0x03030303)
        out += [v_perm_b32(sw, hb, sel[0]), v_perm_b32(sw, hb, sel[1])]
    return out  # dword 2s: (codes s, 4+s); dword 2s+1: (codes 8+s, 12+s)


def emulate_w2_row(codes_row, scales_row):
    K = len(codes_row) * 16
    out = np.empty(K, dtype=np.uint16)
    for wc, w in enumerate(codes_row.tolist()):
        st, g = wc // 4, (wc // 2) % 2  # 64-k step of the word, scale group within the step
        sw = int(scales_row[2 * st]) | (int(scales_row[2 * st + 1]) << 16)
        d = w2_decode_word(w, w2_table(sw)[g], sw, g)
        for s in range(4):
            out[16 * wc + s], out[16 * wc + 4 + s] = d[2 * s] & 0xFFFF, d[2 * s] >> 16
            out[16 * wc + 8 + s], out[16 * wc + 12 + s] = d[2 * s + 1] & 0xFFFF, d[2 * s + 1] >> 16
    return OF.bf16_value(out)


def test_w2_decode_trick_matches_oracle():
    sp = moegen.spec("tiny")
    ex = moegen.expert(sp, 2)
    want = OF.dequant_w2(ex["w1_codes"][:6], ex["w1_scales"][:6])
    for r in range(6):
        got = emulate_w2_row(ex["w1_codes"][r], ex["w1_scales"][r])
        np.testing.assert_array_equal(got, want[r])


def test_w2_decode_trick_golden_words_and_scale_signs():
    # one 64-k step: words 0, 1 in scale group 0, words 2, 3 in group 1 (its own scale)
    scales = (0x3F80, 0xBF80, 0x3BC8, 0xBC78, 0x0080, 0x7E00)
    words = (0x00000000, 0x55555555, 0xAAAAAAAA, 0xFFFFFFFF, 0xE4E4E4E4, 0x1B1B1B1B, 0x9C3A71E5)
    for i, s16 in enumerate(scales):
        s16b = scales[(i + 1) % len(scales)]
        for j, w in enumerate(words):
            w2 = words[(j + 3) % len(words)]
            codes = np.array([w, w, w2, w], np.uint32)
            sc = np.array([s16, s16b], np.uint16)
            got = emulate_w2_row(codes, sc)
            want = OF.dequant_w2(codes[None, :], sc[None, :])[0]
            np.testing.assert_array_equal(got, want)


# --- the k-slot order of the token operand (prepare kernel) and FC1's h store ---
# Within 16 consecutive k the MFMA slots hold k = 0,4,8,12, 1,5,9,13, 2,6,10,14, 3,7,11,15.
SLOT_K = [4 * (p % 4) + p // 4 for p in range(16)]


def kpos16(f):
    q, i = f >> 2, f & 3
    return 4 * i + q


def test_slot_order_is_consistent():
    assert SLOT_K == [0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15]
    # FC1's store position of feature f is the slot that holds k = f
    assert [SLOT_K[kpos16(f)] for f in range(16)] == list(range(16))
    # the decode: operand 0 = dwords (0,4),(8,12),(1,5),(9,13); operand 1 = the same for s = 2, 3
    pairs = [p for s in range(4) for p in ((s, 4 + s), (8 + s, 12 + s))]
    assert [k for p in pairs for k in p] == SLOT_K


def test_prepare_x_byte_selectors():
    x = list(range(0x1000, 0x1010))  # 16 distinct bf16 bit patterns
    d = [x[2 * j] | (x[2 * j + 1] << 16) for j in range(8)]
    LO, HI = 0x05040100, 0x07060302
    o = [v_perm_b32(d[2], d[0], LO), v_perm_b32(d[6], d[4], LO), v_perm_b32(d[2], d[0], HI),
         v_perm_b32(d[6], d[4], HI), v_perm_b32(d[3], d[1], LO), v_perm_b32(d[7], d[5], LO),
         v_perm_b32(d[3], d[1], HI), v_perm_b32(d[7], d[5], HI)]
    got = [v for dw in o for v in (dw & 0xFFFF, dw >> 16)]
    assert got == [x[k] for k in SLOT_K]


# --- 3-bit: the per-group byte tables and the decode of one 96-bit field (ffn_w3.hip) ---
# A group's table holds the bf16 bytes of LEVEL[c] * e4m3(s) / 64 for c = 0..7: LB0/HB0 the
# low/high bytes of c = 0..3 (levels -8,-5,-3,-1), LB1/HB1 those of c = 4..7 (1,3,5,8).
def e4m3_over_64_f32_bits(b):
    """fp32 bits of e4m3fn(b) / 64 by the kernels' integer path (finite bytes)."""
    mag = b & 0x7F
    if mag >> 3:
        bits = (mag << 20) + (114 << 23)
    else:
        bits = int(np.float32(mag).view(np.uint32)) if mag == 0 else \
            int((np.float32(mag) * np.float32(2.0 ** -15)).view(np.uint32))
    return bits | ((b & 0x80) << 24)


def f32_bits_mul(bits, m):
    return int((np.uint32(bits).view(np.float32) * np.float32(m)).view(np.uint32))


def w3_table(b):
    f1 = e4m3_over_64_f32_bits(b)
    f3, f5, f8 = f32_bits_mul(f1, 3), f32_bits_mul(f1, 5), f32_bits_mul(f1, 8)
    p13 = v_perm_b32(f3, f1, 0x07030602)   # [lo1, lo3, hi1, hi3]
    p58 = v_perm_b32(f8, f5, 0x07030602)   # [lo5, lo8, hi5, hi8]
    lb1 = v_perm_b32(p58, p13, 0x05040100)
    hb1 = v_perm_b32(p58, p13, 0x07060302)
    lb0 = v_perm_b32(0, lb1, 0x00010203)
    hb0 = v_perm_b32(0, hb1, 0x00010203) ^ 0x80808080
    return hb1, hb0, lb1, lb0


def pk_lshr16(v, a, b):
    lo, hi = v & 0xFFFF, v >> 16
    return (lo >> a) | ((hi >> b) << 16)


def alignbit(hi, lo, s):
    return (((hi << 32) | lo) >> s) & 0xFFFFFFFF


def w3_lookup(sel, tab):
    hb1, hb0, lb1, lb0 = tab
    hb = v_perm_b32(hb1, hb0, sel)
    lb = v_perm_b32(lb1, lb0, sel)
    return [v_perm_b32(hb, lb, 0x05010400), v_perm_b32(hb, lb, 0x07030602)]


M7 = 0x07070707


def w3_decode_field(w0, w1, w2, tab):
    """Four MFMA operands (16 dwords) from the three words of one 32-code field."""
    z = v_perm_b32(w2, w0, 0x04020500)        # [B0, B9, B2, B8]
    x = v_perm_b32(w1, w0, 0x04010603)        # [B3, B6, B1, B4]
    y = v_perm_b32(w2, w1, 0x07010603)        # [B7, B10, B5, B11]
    s0, s1, s2 = alignbit(w1, w0, 2), alignbit(w2, w1, 2), w2 >> 2
    u = v_perm_b32(s1, s0, 0x04010300)        # stream>>2 bytes [S0, S3, S1, S4]
    v = v_perm_b32(s2, s1, 0x06030502)        # [S6, S9, S7, S10]
    sels = [pk_lshr16(z, 0, 2) & M7, pk_lshr16(z, 3, 5) & M7,
            pk_lshr16(x, 0, 1) & M7, pk_lshr16(x, 3, 4) & M7,
            pk_lshr16(y, 1, 2) & M7, pk_lshr16(y, 4, 5) & M7,
            pk_lshr16(u, 4, 5) & M7, pk_lshr16(v, 4, 5) & M7]
    return [d for s in sels for d in w3_lookup(s, tab)]


# code index held by each of the 32 slots of a field (operand o = slots 8o .. 8o+7)
SLOT3 = [0, 24, 6, 22, 1, 25, 7, 23, 8, 16, 3, 11, 9, 17, 4, 12,
         19, 27, 14, 30, 20, 28, 15, 31, 2, 10, 5, 13, 18, 26, 21, 29]


def emulate_w3_row(codes_row, scales_row):
    K = len(codes_row) // 3 * 32
    out = np.empty(K, dtype=np.uint16)
    for f in range(K // 32):
        tab = w3_table(int(scales_row[f // 2]))
        d = w3_decode_field(*[int(c) for c in codes_row[3 * f:3 * f + 3]], tab)
        halves = [h for dw in d for h in (dw & 0xFFFF, dw >> 16)]
        for slot, c in enumerate(SLOT3):
            out[32 * f + c] = halves[slot]
    return OF.bf16_value(out)


def test_slot3_is_a_permutation():
    assert sorted(SLOT3) == list(range(32))


def test_w3_decode_trick_matches_oracle():
    sp = moegen.spec("w3")
    ex = moegen.expert(sp, 5)
    want = OF.dequant_w3(ex["w1_codes"][:4, :48], ex["w1_scales"][:4, :8])
    for r in range(4):
        got = emulate_w3_row(ex["w1_codes"][r, :48], ex["w1_scales"][r, :8])
        np.testing.assert_array_equal(got, want[r])


def test_w3_decode_every_finite_scale_byte_and_golden_fields():
    fields = [(0x88FAC688, 0xC688FAC6, 0xFAC688FA), (0x77053977, 0x39770539, 0x05397705),
              (0, 0, 0), (0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0x9C3A71E5, 0x0F1E2D3C, 0xA5A55A5A)]
    for b in range(256):
        if b & 0x7F == 0x7F:
            continue  # NaN encodings are not valid scales
        for f in fields:
            codes = np.array(f + f, np.uint32)
            got = emulate_w3_row(codes, np.array([b], np.uint8))
            want = OF.dequant_w3(codes[None, :], np.array([[b]], np.uint8))[0]
            np.testing.assert_array_equal(got, want, err_msg=f"scale byte {b:#x}")


def _header_table(name):
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "bit_moe_expert_top_amd", "csrc", "lowbit_fmt.h")).read()
    m = re.search(name + r"\[32\]\s*=\s*\{([^}]*)\}", src)
    return [int(v) for v in m.group(1).replace("\n", " ").split(",")]


def test_device_slot_tables_match_the_emulated_decode():
    slot_k, pos = _header_table("kW3SlotK"), _header_table("kW3Pos")
    assert slot_k == SLOT3
    assert [pos[c] for c in slot_k] == list(range(32))


# --- MX formats (mx_fmt.h): the e2m1 -> e4m3 byte table and the integer e4m3 encoder ---
E2M1_TO_E4M3_LO, E2M1_TO_E4M3_HI = 0x3C383000, 0x4C484440


def e2m1x8_to_e4m3(w):
    lo, hi = w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F
    elo = v_perm_b32(E2M1_TO_E4M3_HI, E2M1_TO_E4M3_LO, lo & 0x07070707) | ((lo & 0x08080808) << 4)
    ehi = v_perm_b32(E2M1_TO_E4M3_HI, E2M1_TO_E4M3_LO, hi & 0x07070707) | ((hi & 0x08080808) << 4)
    return v_perm_b32(ehi, elo, 0x05010400), v_perm_b32(ehi, elo, 0x07030602)


def test_e2m1_conversion_table_matches_oracle():
    r = np.random.default_rng(5)
    codes = r.integers(0, 256, size=(3, 64), dtype=np.uint8)
    codes[0, :16] = np.arange(0, 256, 16, dtype=np.uint8) | np.arange(16, dtype=np.uint8)  # every nibble
    want, _ = OF.mxfp4_to_fp8(codes, np.zeros((3, 4), np.uint8))
    for row in range(3):
        words = codes[row].view(np.uint32)
        got = []
        for w in words.tolist():
            o0, o1 = e2m1x8_to_e4m3(w)
            got += [(o0 >> (8 * i)) & 0xFF for i in range(4)] + [(o1 >> (8 * i)) & 0xFF for i in range(4)]
        assert got == want[row].tolist()


def e4m3_mag_rne(M, F):
    m = M.bit_length() - 1
    fl = m + F
    if fl > 8:
        return 0x7E
    if fl >= -6:
        sh, ebase = m - 3, fl + 7
    else:
        sh, ebase = -(F + 9), 0
    if sh <= 0:
        q = M << (-sh)
    elif sh > 25:
        q = 0
    else:
        q, rem, half = M >> sh, M & ((1 << sh) - 1), 1 << (sh - 1)
        q += 1 if (rem > half or (rem == half and q & 1)) else 0
    if ebase == 0:
        byte = q
    else:
        byte = (ebase + 1) << 3 if q == 16 else (ebase << 3) | (q - 8)
    return min(byte, 0x7E)


def bf16_to_e4m3_scaled(b, shared):
    sgn, mag = (b >> 8) & 0x80, b & 0x7FFF
    if mag == 0:
        return sgn
    eb, mb = mag >> 7, mag & 0x7F
    M = (mb | 0x80) if eb else mb
    E0 = eb - 134 if eb else -133
    return sgn | e4m3_mag_rne(M, E0 - shared)


def test_integer_e4m3_encoder_matches_oracle_rne():
    r = np.random.default_rng(6)
    # bf16 patterns over the whole range (normals, subnormals, zeros), with shared exponents
    bits = r.integers(0, 1 << 16, size=4000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    shared = r.integers(-127, 128, size=bits.size)
    vals = OF.bf16_value(bits) / np.exp2(shared.astype(np.float64))
    want = OF.e4m3fn_encode(vals)
    got = np.array([bf16_to_e4m3_scaled(int(b), int(s)) for b, s in zip(bits, shared)], np.uint8)
    np.testing.assert_array_equal(got, want)
