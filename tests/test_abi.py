"""The C ABI library loads and exports every function include/bitmoe.h declares (no GPU
calls), and the host-side argument checks reject bad input without touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitmoe.h")
LIB = os.path.join(ROOT, "bit_moe_expert_top_amd", "libbitmoe.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine"):
        assert n in names
    assert len(names) >= 10


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libbitmoe.so not built")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    lib.moe_status_str.restype = ctypes.c_char_p
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(-3) == b"MOE_ERR_WORKSPACE"


def test_host_argument_checks_need_no_gpu(lib):
    """Every check below fails on the host before anything is enqueued."""
    p = ctypes.c_void_p(16)  # never dereferenced: the calls must reject the arguments first
    lib.moe_route.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.moe_route(p, 4, 8, 0, p, p, None) == -1       # k < 1
    assert lib.moe_route(p, 4, 8, 9, p, p, None) == -1       # k > E
    assert lib.moe_route(p, 4, 2000, 2, p, p, None) == -1    # E too large
    assert lib.moe_route(None, 4, 8, 2, p, p, None) == -1    # null input
    assert lib.moe_route(None, 0, 8, 2, None, None, None) == 0  # T = 0 is a no-op
    lib.moe_permute.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.moe_permute_ws_bytes.restype = ctypes.c_size_t
    need = lib.moe_permute_ws_bytes(100000, 8, 384)
    assert need > 0
    assert lib.moe_permute(p, 100000, 8, 384, p, p, p, p, p, need - 1, None) == -3  # workspace
    assert lib.moe_permute(p, 4, 8, 4, p, p, p, p, None, 0, None) == -1  # k > E
    lib.moe_combine.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                ctypes.c_void_p]
    assert lib.moe_combine(p, p, p, 4, 2, 6, p, 1, None) == -1  # H % 4
    assert lib.moe_combine(None, p, p, 4, 2, 8, p, 1, None) == -1


def test_ffn_argument_checks(lib):
    import sys
    sys.path.insert(0, ROOT)
    from bit_moe_expert_top_amd import _lib as L

    p = 16
    w = L.MoeWeights(8, 256, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None)
    assert L.lib.moe_expert_ffn_ws_bytes(ctypes.byref(w), 16, 2, 0) > 0
    bad = L.MoeWeights(8, 200, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None)
    assert L.lib.moe_expert_ffn(ctypes.byref(bad), p, 16, 2, p, p, p, p, p, 1 << 30, None) == -1  # H % 32
    # whole scale groups (32 weights, 64 for 3-bit) but not whole 256-k steps: valid, not built
    for fmt, H, want in ((L.MOE_FMT_W2, 288, -2), (L.MOE_FMT_W3, 288, -1), (L.MOE_FMT_W3, 320, -2),
                         (L.MOE_FMT_W2, 20480, -2)):
        wh = L.MoeWeights(8, H, 512, fmt, p, p, p, p, 0, None, None, None, None, None)
        assert L.lib.moe_expert_ffn(ctypes.byref(wh), p, 16, 2, p, p, p, p, p, 1 << 30, None) == want, (fmt, H)
        wi = L.MoeWeights(8, 512, H, fmt, p, p, p, p, 0, None, None, None, None, None)
        assert L.lib.moe_expert_ffn(ctypes.byref(wi), p, 16, 2, p, p, p, p, p, 1 << 30, None) == want, (fmt, H)
        assert L.lib.moe_expert_ffn_ws_bytes(ctypes.byref(wh), 16, 2, 0) == 0
    assert L.lib.moe_expert_ffn(ctypes.byref(w), p, 16, 2, p, p, p, p, p, 10, None) == -3  # workspace
    nofmt = L.MoeWeights(8, 256, 512, 7, p, p, p, p, 0, None, None, None, None, None)
    assert L.lib.moe_expert_ffn(ctypes.byref(nofmt), p, 16, 2, p, p, p, p, p, 1 << 30, None) == -1
    hot_missing = L.MoeWeights(8, 256, 512, L.MOE_FMT_W2, p, p, p, p, 2, None, None, None, None, None)
    assert L.lib.moe_expert_ffn(ctypes.byref(hot_missing), p, 16, 2, p, p, p, p, p, 1 << 30, None) == -1
    assert L.lib.moe_debug_dequant(ctypes.byref(w), 8, 1, p, None) == -1  # expert out of range


def test_ffn_flags(lib):
    import sys
    sys.path.insert(0, ROOT)
    from bit_moe_expert_top_amd import _lib as L

    p = 16
    base = (8, 256, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None)
    unknown = L.MoeWeights(*base, 4)
    assert L.lib.moe_expert_ffn_ws_bytes(ctypes.byref(unknown), 256, 2, 0) == 0
    assert L.lib.moe_expert_ffn(ctypes.byref(unknown), p, 16, 2, p, p, p, p, p, 1 << 30, None) == -1
    plain = L.MoeWeights(*base, 0)
    inv = L.MoeWeights(*base, L.MOE_FLAG_BATCH_INVARIANT)
    # batch-invariant mode streams every group (no grouped-GEMM work list from 128 tokens on):
    # the same workspace below that, at most a little less above
    for T in (16, 100, 256, 4096):
        a = L.lib.moe_expert_ffn_ws_bytes(ctypes.byref(plain), T, 2, 0)
        b = L.lib.moe_expert_ffn_ws_bytes(ctypes.byref(inv), T, 2, 0)
        assert 0 < b and (b == a if T < 128 else a - 16 * 1024 < b <= a)
    assert L.lib.moe_expert_ffn_num_stages(ctypes.byref(inv), 256, 2, 1 << 30) == 5
    dw = L.MoeWeights(*base)
    assert dw.flags == 0
    # FP4 residual hot set: no FP8 stages; only on 2-bit experts
    hot = (8, 256, 512, L.MOE_FMT_W2, p, p, p, p, 2, p, p, p, p, p)
    res = L.MoeWeights(*hot, L.MOE_FLAG_HOT_RESIDUAL)
    fp8 = L.MoeWeights(*hot, 0)
    assert L.lib.moe_expert_ffn_num_stages(ctypes.byref(res), 256, 2, 1 << 30) == 5
    assert L.lib.moe_expert_ffn_num_stages(ctypes.byref(fp8), 256, 2, 1 << 30) > 5
    assert L.lib.moe_expert_ffn_ws_bytes(ctypes.byref(res), 256, 2, 0) < L.lib.moe_expert_ffn_ws_bytes(
        ctypes.byref(fp8), 256, 2, 0)
    w3res = L.MoeWeights(8, 256, 512, L.MOE_FMT_W3, p, p, p, p, 2, p, p, p, p, p, L.MOE_FLAG_HOT_RESIDUAL)
    assert L.lib.moe_expert_ffn(ctypes.byref(w3res), p, 16, 2, p, p, p, p, p, 1 << 30, None) == -2
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.lib.moe_expert_ffn_ws_region(ctypes.byref(res), 16, 2, 1 << 30, L.MOE_WS_HQ, ctypes.byref(off),
                                          ctypes.byref(n)) == -2
    header = open(os.path.join(ROOT, "include", "bitmoe.h")).read()
    assert "int32_t flags;" in header.split("} moe_weights;")[0].split("const void* hot_w2_scales;")[1]


def test_ffn_rejects_batches_beyond_32bit_offsets(lib):
    import sys
    sys.path.insert(0, ROOT)
    from bit_moe_expert_top_amd import _lib as L

    p = 16
    w = L.MoeWeights(8, 4096, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None)
    T = (1 << 32) // (4096 * 2)  # T * H * 2 == 2^32
    assert L.lib.moe_expert_ffn(ctypes.byref(w), p, T, 1, p, p, p, p, p, 1 << 40, None) == -2
    assert L.lib.moe_expert_ffn(ctypes.byref(w), p, T - 1, 1, p, p, p, p, p, 10, None) == -3  # ws check next


def test_quantizer_argument_checks(lib):
    p = ctypes.c_void_p(16)
    for name in ("moe_quantize_w2", "moe_quantize_mxfp4"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_void_p]
        assert f(p, 4, 48, p, p, None) == -1      # K not a multiple of 32
        assert f(p, 4, 0, p, p, None) == -1       # K <= 0
        assert f(p, -1, 64, p, p, None) == -1     # rows < 0
        assert f(None, 4, 64, p, p, None) == -1   # null input
        assert f(p, 4, 64, p, None, None) == -1   # null output
        assert f(None, 0, 64, None, None, None) == 0  # rows = 0 is a no-op


def test_front_argument_checks(lib):
    """moe_route_permute_prepare rejects bad arguments on the host; batches above 4096 routed
    rows (T*k) are UNSUPPORTED (the caller runs the three calls instead)."""
    import sys
    sys.path.insert(0, ROOT)
    from bit_moe_expert_top_amd import _lib as L

    p = 16
    w = L.MoeWeights(8, 256, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None)
    f = L.lib.moe_route_permute_prepare
    args = lambda T, k, ws_bytes=1 << 30, counts=p: (ctypes.byref(w), p, p, T, k, p, p, counts, p, p, p, p,
                                                      ws_bytes, None)
    assert f(*args(2049, 2)) == -2               # more than 4096 rows: not this call
    assert f(*args(2048, 2, ws_bytes=10)) == -3  # 4096 rows pass; the workspace is checked next
    assert f(*args(4, 0)) == -1                  # k < 1
    assert f(*args(4, 9)) == -1                  # k > E
    assert f(*args(-1, 2)) == -1                 # T < 0
    assert f(*args(4, 2, counts=None)) == -1     # null output
    assert f(*args(4, 2, ws_bytes=10)) == -3     # workspace too small
    bad = L.MoeWeights(8, 200, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None)
    assert f(ctypes.byref(bad), p, p, 4, 2, p, p, p, p, p, p, p, 1 << 30, None) == -1
