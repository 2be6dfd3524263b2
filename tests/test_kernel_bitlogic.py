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


# --- 2-bit: the per-group byte table and the two pair extractions (ffn_lowbit.hip) ---
def w2_table(s16):
    hb = (s16 >> 8) & 0xFF
    lo = (((hb * 0x01010101) ^ 0x00008080) + 0x01000001) & 0xFFFFFFFF
    hi = s16 & 0xFF
    return lo, hi


def w2_decode(w, half, lo, hi):
    M, C = 0x03000300, 0x00040004
    if half == 0:
        sels = [((w >> (2 * m)) & M) | C for m in range(4)]
    else:
        sels = [(((w << (8 - 2 * m)) & 0xFFFFFFFF) & M) | C for m in range(4)]
    return [v_perm_b32(hi, lo, s) for s in sels]


def emulate_w2_row(codes_row, scales_row):
    K = len(codes_row) * 16
    out = np.empty(K, dtype=np.uint16)
    for wc, w in enumerate(codes_row.tolist()):
        lo, hi = w2_table(int(scales_row[wc // 2]))
        p0, p1 = w2_decode(w, 0, lo, hi), w2_decode(w, 1, lo, hi)
        for m in range(4):
            out[16 * wc + 4 + m] = p0[m] & 0xFFFF
            out[16 * wc + 12 + m] = p0[m] >> 16
            out[16 * wc + m] = p1[m] & 0xFFFF
            out[16 * wc + 8 + m] = p1[m] >> 16
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
SLOT_K = [4, 12, 5, 13, 6, 14, 7, 15, 0, 8, 1, 9, 2, 10, 3, 11]


def kpos16(f):
    q, i = f >> 2, f & 3
    return 2 * i + ((q & 1) ^ 1) * 8 + (q >> 1)


def test_slot_order_is_consistent():
    # FC1's store position of feature f is the slot that holds k = f
    assert [SLOT_K[kpos16(f)] for f in range(16)] == list(range(16))
    # the decode pairs: dword m of half 0 holds (4+m, 12+m), of half 1 holds (m, 8+m)
    pairs = [(4 + m, 12 + m) for m in range(4)] + [(m, 8 + m) for m in range(4)]
    assert [k for p in pairs for k in p] == SLOT_K


def test_prepare_x_byte_selectors():
    x = list(range(0x1000, 0x1010))  # 16 distinct bf16 bit patterns
    d = [x[2 * j] | (x[2 * j + 1] << 16) for j in range(8)]
    a, b = d[:4], d[4:]
    sel_lo, sel_hi = 0x05040100, 0x07060302
    o = [v_perm_b32(b[2], a[2], sel_lo), v_perm_b32(b[2], a[2], sel_hi),
         v_perm_b32(b[3], a[3], sel_lo), v_perm_b32(b[3], a[3], sel_hi),
         v_perm_b32(b[0], a[0], sel_lo), v_perm_b32(b[0], a[0], sel_hi),
         v_perm_b32(b[1], a[1], sel_lo), v_perm_b32(b[1], a[1], sel_hi)]
    got = [v for dw in o for v in (dw & 0xFFFF, dw >> 16)]
    assert got == [x[k] for k in SLOT_K]
