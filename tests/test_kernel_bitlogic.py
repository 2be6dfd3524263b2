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


# --- 2-bit: the per-group byte table and the decode of one word (ffn_lowbit.hip) ---
def w2_table(s16):
    hb = (s16 >> 8) & 0xFF
    lut = (((hb * 0x01010101) ^ 0x00008080) + 0x01000001) & 0xFFFFFFFF
    return lut, s16 & 0xFF


def w2_decode_word(w, lut, lb):
    """Eight dwords (two MFMA operands) from one word: for s = 0..3 the high bytes of codes
    s, 4+s, 8+s, 12+s, then two interleaves with the scale's low byte."""
    out = []
    for s in range(4):
        hb = v_perm_b32(0, lut, (w >> (2 * s)) & 0x03030303)
        out += [v_perm_b32(lb, hb, 0x01040004), v_perm_b32(lb, hb, 0x03040204)]
    return out  # dword 2s: (codes s, 4+s); dword 2s+1: (codes 8+s, 12+s)


def emulate_w2_row(codes_row, scales_row):
    K = len(codes_row) * 16
    out = np.empty(K, dtype=np.uint16)
    for wc, w in enumerate(codes_row.tolist()):
        lut, lb = w2_table(int(scales_row[wc // 2]))
        d = w2_decode_word(w, lut, lb)
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
    for s16 in (0x3F80, 0xBF80, 0x3BC8, 0xBC78, 0x0080, 0x7E00):
        for w in (0x00000000, 0x55555555, 0xAAAAAAAA, 0xFFFFFFFF, 0xE4E4E4E4, 0x1B1B1B1B, 0x9C3A71E5):
            codes = np.array([w, w], np.uint32)
            got = emulate_w2_row(codes, np.array([s16], np.uint16))
            want = OF.dequant_w2(codes[None, :], np.array([[s16]], np.uint16))[0]
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
