"""ctypes binding of ``libbitmoe.so`` (the C ABI in ``include/bitmoe.h``).

Argument marshalling only: torch tensors supply device memory and the current HIP stream;
every step of the layer runs in the library's kernels.  There is no fallback: if the
library is not built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitmoe.so")

MOE_FMT_W2, MOE_FMT_W3, MOE_FMT_MXFP4 = 1, 2, 3

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_moe_expert_top_amd.build`")
lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class MoeWeights(ctypes.Structure):
    _fields_ = [
        ("E", _i32), ("H", _i32), ("I", _i32), ("fmt", _i32),
        ("w1_codes", _p), ("w1_scales", _p), ("w2_codes", _p), ("w2_scales", _p),
        ("n_hot", _i32), ("hot_ids", _p),
        ("hot_w1_codes", _p), ("hot_w1_scales", _p), ("hot_w2_codes", _p), ("hot_w2_scales", _p),
        ("flags", _i32),
    ]


MOE_FLAG_BATCH_INVARIANT = 1
MOE_FLAG_HOT_RESIDUAL = 2


class MoeTierState(ctypes.Structure):
    _fields_ = [("E", _i32), ("n_slots", _i32), ("slot_of_expert", _p), ("expert_of_slot", _p),
                ("last_use", _p), ("tick", _i64)]


_SIGS = {
    "moe_route": (_i32, [_p, _i32, _i32, _i32, _p, _p, _p]),
    "moe_permute_ws_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_permute": (_i32, [_p, _i32, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_expert_ffn_ws_bytes": (_sz, [ctypes.POINTER(MoeWeights), _i32, _i32, _i32]),
    "moe_expert_ffn": (_i32, [ctypes.POINTER(MoeWeights), _p, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_expert_ffn_num_stages": (_i32, [ctypes.POINTER(MoeWeights), _i32, _i32, _sz]),
    "moe_expert_ffn_noalloc": (_i32, [ctypes.POINTER(MoeWeights), _p, _i32, _i32, _p, _p, _p, _p, _p]),
    "moe_expert_ffn_stage": (_i32, [ctypes.POINTER(MoeWeights), _p, _i32, _i32, _p, _p, _p, _p, _p, _sz, _i32,
                                    _p]),
    "moe_route_permute_prepare": (_i32, [ctypes.POINTER(MoeWeights), _p, _p, _i32, _i32] + [_p] * 7 + [_sz, _p]),
    "moe_combine": (_i32, [_p, _p, _p, _i32, _i32, _i32, _p, _i32, _p]),
    "moe_mxfp4_to_fp8": (_i32, [_p, _p, _i64, _i32, _p, _p, _p]),
    "moe_mxfp8_quantize": (_i32, [_p, _i64, _i32, _p, _p, _p]),
    "moe_quantize_w2": (_i32, [_p, _i64, _i32, _p, _p, _p]),
    "moe_quantize_mxfp4": (_i32, [_p, _i64, _i32, _p, _p, _p]),
    "moe_debug_dequant": (_i32, [ctypes.POINTER(MoeWeights), _i32, _i32, _p, _p]),
    "moe_expert_ffn_ws_region": (_i32, [ctypes.POINTER(MoeWeights), _i32, _i32, _sz, _i32,
                                        ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "moe_fp8_slot_layout": (_i32, [_i32, _i32] + [ctypes.POINTER(_sz)] * 5),
    "moe_status_str": (ctypes.c_char_p, [_i32]),
    "moe_tier_plan": (_i32, [ctypes.POINTER(MoeTierState), _p, _i64, _p, _p, _p]),
    "moe_tier_load": (_i32, [ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeights), _p, _p, _i32, _p]),
    "moe_tier_remap": (_i32, [_p, _i64, _p, _p, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {lib.moe_status_str(status).decode()} ({status})")
        self.status = status


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor on the GPU")


# --------------------------------------------------------------------- weights
class DeviceWeights:
    """Device copies of one layer's packed experts and the ``moe_weights`` struct that points
    at them (the tensors are kept alive by this object)."""

    def __init__(self, fmt: int, E: int, H: int, I: int, arrays: dict, device="cuda", flags: int = 0):
        def t(a):
            return torch.from_numpy(a.view(_np_uint_as_int(a.dtype))).to(device) if a is not None else None

        self.fmt, self.E, self.H, self.I = fmt, E, H, I
        self.t = {key: t(a) for key, a in arrays.items() if a is not None and a.size > 0}
        hot = self.t.get("hot_ids")
        self.n_hot = 0 if hot is None else int(hot.numel())
        g = lambda key: _ptr(self.t.get(key))
        self.c = MoeWeights(E, H, I, fmt, g("w1_codes"), g("w1_scales"), g("w2_codes"), g("w2_scales"),
                            self.n_hot, g("hot_ids"), g("hot_w1_codes"), g("hot_w1_scales"),
                            g("hot_w2_codes"), g("hot_w2_scales"), flags)

    def set_batch_invariant(self, on: bool = True):
        """Switch the layer's batch-invariant mode (MOE_FLAG_BATCH_INVARIANT) on or off."""
        self.c.flags = (self.c.flags | MOE_FLAG_BATCH_INVARIANT) if on else (self.c.flags & ~MOE_FLAG_BATCH_INVARIANT)
        return self


def _np_uint_as_int(dt):
    import numpy as np

    return {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16, np.dtype(np.uint8): np.uint8,
            np.dtype(np.int32): np.int32}[np.dtype(dt)]


# --------------------------------------------------------------------- the four calls
def moe_route(logits: torch.Tensor, k: int, topk_ids=None, topk_w=None):
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device) if topk_w is None else topk_w
    _check("moe_route", lib.moe_route(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _stream()))
    return topk_ids, topk_w


def moe_permute_ws_bytes(T: int, k: int, E: int) -> int:
    return lib.moe_permute_ws_bytes(T, k, E)


def moe_permute(topk_ids: torch.Tensor, E: int, ws=None, out=None):
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev))
    counts, offsets, perm, inv = out
    need = moe_permute_ws_bytes(T, k, E)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    nbytes = 0 if ws is None else ws.numel()
    _check("moe_permute", lib.moe_permute(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm),
                                          _ptr(inv), _ptr(ws), nbytes, _stream()))
    return counts, offsets, perm, inv


def moe_expert_ffn_ws_bytes(w: DeviceWeights, T: int, k: int, fp8_slots: int = 0) -> int:
    return lib.moe_expert_ffn_ws_bytes(ctypes.byref(w.c), T, k, fp8_slots)


def moe_expert_ffn(w: DeviceWeights, x: torch.Tensor, k: int, counts, offsets, perm, y_perm=None, ws=None,
                   fp8_slots: int | None = None):
    _dev(x, torch.int16, "x (bf16 bits as int16)")
    T = x.shape[0]
    if y_perm is None:
        y_perm = torch.empty((T * k, w.H), dtype=torch.float32, device=x.device)
    if ws is None:
        slots = w.n_hot if fp8_slots is None else fp8_slots
        ws = torch.empty(max(1, moe_expert_ffn_ws_bytes(w, T, k, slots)), dtype=torch.uint8, device=x.device)
    _check("moe_expert_ffn", lib.moe_expert_ffn(ctypes.byref(w.c), _ptr(x), T, k, _ptr(counts), _ptr(offsets),
                                                _ptr(perm), _ptr(y_perm), _ptr(ws), ws.numel(), _stream()))
    return y_perm


NOALLOC_SCRATCH_BYTES = 16 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_expert_ffn_noalloc(w: DeviceWeights, x: torch.Tensor, k: int, counts, offsets, perm, y_perm):
    """moe_expert_ffn with the library's static workspace (no allocation by the library; y_perm is
    the caller's)."""
    _dev(x, torch.int16, "x (bf16 bits as int16)")
    T = x.shape[0]
    _check("moe_expert_ffn_noalloc", lib.moe_expert_ffn_noalloc(ctypes.byref(w.c), _ptr(x), T, k, _ptr(counts),
                                                                _ptr(offsets), _ptr(perm), _ptr(y_perm), _stream()))
    return y_perm


def moe_expert_ffn_num_stages(w: DeviceWeights, T: int, k: int, ws_bytes: int) -> int:
    return lib.moe_expert_ffn_num_stages(ctypes.byref(w.c), T, k, ws_bytes)


def moe_expert_ffn_stage(w: DeviceWeights, x: torch.Tensor, k: int, counts, offsets, perm, y_perm, ws,
                         stage: int):
    T = x.shape[0]
    _check("moe_expert_ffn_stage", lib.moe_expert_ffn_stage(ctypes.byref(w.c), _ptr(x), T, k, _ptr(counts),
                                                            _ptr(offsets), _ptr(perm), _ptr(y_perm), _ptr(ws),
                                                            ws.numel(), stage, _stream()))


LOWBIT_STAGES = 5  # stages 0..4: prepare, FC1 (stream, GEMM), FC2 (stream, GEMM); 5: hot prepare


def moe_expert_ffn_two_streams(w: DeviceWeights, x: torch.Tensor, k: int, counts, offsets, perm, y_perm, ws,
                               side: torch.cuda.Stream, stage_events=None):
    """moe_expert_ffn with the hot experts' preparation and first MXFP4 -> FP8 conversion on a
    second stream, concurrent with the low-bit stages (they touch disjoint workspace regions
    and rows); the FP8 matmuls start once both are done.  Same kernels and inputs as the
    one-stream call, so the same output bits.  stage_events: optional {stage: (start, end)} HIP
    events recorded around each stage on the stream that runs it."""
    T = x.shape[0]
    n = moe_expert_ffn_num_stages(w, T, k, ws.numel())
    main = torch.cuda.current_stream()

    def run(st):
        ev = stage_events.get(st) if stage_events else None
        if ev:
            ev[0].record(torch.cuda.current_stream())
        moe_expert_ffn_stage(w, x, k, counts, offsets, perm, y_perm, ws, st)
        if ev:
            ev[1].record(torch.cuda.current_stream())

    if n <= LOWBIT_STAGES + 1:  # no hot set (or nothing to convert): one stream
        for st in range(n):
            run(st)
        return y_perm
    fork = torch.cuda.Event()
    fork.record(main)
    side.wait_event(fork)
    with torch.cuda.stream(side):
        run(LOWBIT_STAGES)        # hot work list, MXFP8 of x
        run(LOWBIT_STAGES + 1)    # first batch of hot experts: MXFP4 -> FP8 into the slots
        join = torch.cuda.Event()
        join.record(side)
    for st in range(LOWBIT_STAGES):
        run(st)
    main.wait_event(join)
    for st in range(LOWBIT_STAGES + 2, n):
        run(st)
    for t in (x, counts, offsets, perm, y_perm, ws):
        t.record_stream(side)
    return y_perm


FRONT_MAX_ROWS = 4096  # moe_route_permute_prepare takes batches of at most this many routed rows (T*k)


def moe_route_permute_prepare(w: DeviceWeights, logits: torch.Tensor, x: torch.Tensor, k: int, ws: torch.Tensor,
                              out=None):
    """moe_route + moe_permute + stage 0 of the FFN (T*k <= FRONT_MAX_ROWS); returns
    (topk_ids, topk_w, counts, offsets, perm, inv).  ``ws`` is the FFN workspace."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev))
    ids, gw, counts, offsets, perm, inv = out
    _check("moe_route_permute_prepare",
           lib.moe_route_permute_prepare(ctypes.byref(w.c), _ptr(logits), _ptr(x), T, k, _ptr(ids), _ptr(gw),
                                         _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(ws), ws.numel(),
                                         _stream()))
    return ids, gw, counts, offsets, perm, inv


def moe_combine(y_perm: torch.Tensor, inv: torch.Tensor, topk_w: torch.Tensor, out_fp32: bool = False,
                out=None):
    T, k = topk_w.shape
    H = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32 if out_fp32 else torch.int16, device=y_perm.device)
    _check("moe_combine", lib.moe_combine(_ptr(y_perm), _ptr(inv), _ptr(topk_w), T, k, H, _ptr(out),
                                          1 if out_fp32 else 0, _stream()))
    return out


def moe_mxfp4_to_fp8(codes: torch.Tensor, scales: torch.Tensor):
    rows, half = codes.shape
    K = 2 * half
    elems = torch.empty((rows, K), dtype=torch.uint8, device=codes.device)
    sc = torch.empty((rows, K // 32), dtype=torch.uint8, device=codes.device)
    _check("moe_mxfp4_to_fp8", lib.moe_mxfp4_to_fp8(_ptr(codes), _ptr(scales), rows, K, _ptr(elems), _ptr(sc),
                                                    _stream()))
    return elems, sc


def moe_mxfp8_quantize(x: torch.Tensor):
    rows, K = x.shape
    elems = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    sc = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check("moe_mxfp8_quantize", lib.moe_mxfp8_quantize(_ptr(x), rows, K, _ptr(elems), _ptr(sc), _stream()))
    return elems, sc


def moe_quantize_w2(w: torch.Tensor):
    """fp32 [rows][K] (device) -> (codes int32 [rows][K/16], bf16 scale bits int16 [rows][K/32])."""
    rows, K = w.shape
    codes = torch.empty((rows, K // 16), dtype=torch.int32, device=w.device)
    sc = torch.empty((rows, K // 32), dtype=torch.int16, device=w.device)
    _check("moe_quantize_w2", lib.moe_quantize_w2(_ptr(w), rows, K, _ptr(codes), _ptr(sc), _stream()))
    return codes, sc


def moe_quantize_mxfp4(w: torch.Tensor):
    """fp32 [rows][K] (device) -> (codes uint8 [rows][K/2], e8m0 scales uint8 [rows][K/32])."""
    rows, K = w.shape
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=w.device)
    sc = torch.empty((rows, K // 32), dtype=torch.uint8, device=w.device)
    _check("moe_quantize_mxfp4", lib.moe_quantize_mxfp4(_ptr(w), rows, K, _ptr(codes), _ptr(sc), _stream()))
    return codes, sc


MOE_WS_XQ, MOE_WS_XQ_SCALES, MOE_WS_HQ, MOE_WS_HQ_SCALES, MOE_WS_SLOTS = 1, 2, 3, 4, 5


def moe_expert_ffn_ws_region(w: DeviceWeights, T: int, k: int, ws_bytes: int, region: int):
    """(byte offset, bytes) of an intermediate of moe_expert_ffn inside its workspace."""
    off, n = _sz(0), _sz(0)
    _check("moe_expert_ffn_ws_region", lib.moe_expert_ffn_ws_region(ctypes.byref(w.c), T, k, ws_bytes, region,
                                                                    ctypes.byref(off), ctypes.byref(n)))
    return off.value, n.value


def moe_fp8_slot_layout(H: int, I: int) -> dict:
    """Byte offsets of W1, W1 scales, W2, W2 scales inside one FP8 slot, and the slot size."""
    v = [_sz(0) for _ in range(5)]
    _check("moe_fp8_slot_layout", lib.moe_fp8_slot_layout(H, I, *(ctypes.byref(x) for x in v)))
    return dict(zip(("w1", "w1_scales", "w2", "w2_scales", "slot_bytes"), (x.value for x in v)))


def moe_debug_dequant(w: DeviceWeights, e: int, which: int):
    """which: 1 / 2 = W1 / W2 through the streaming kernels' decoder, 3 / 4 through the grouped
    GEMM's decoder, 5 / 6 the FP4 residual of hot slot e (layers with MOE_FLAG_HOT_RESIDUAL)."""
    rows, K = (2 * w.I, w.H) if which in (1, 3, 5) else (w.H, w.I)
    out = torch.empty((rows, K), dtype=torch.float32, device="cuda")
    _check("moe_debug_dequant", lib.moe_debug_dequant(ctypes.byref(w.c), e, which, _ptr(out), _stream()))
    return out


def layer_forward(w: DeviceWeights, logits: torch.Tensor, x: torch.Tensor, k: int, out_fp32: bool = True,
                  fp8_slots: int | None = None):
    """The four calls in order; returns every intermediate (for tests and the bench)."""
    ids, gw = moe_route(logits, k)
    counts, offsets, perm, inv = moe_permute(ids, w.E)
    y = moe_expert_ffn(w, x, k, counts, offsets, perm, fp8_slots=fp8_slots)
    out = moe_combine(y, inv, gw, out_fp32=out_fp32)
    return dict(ids=ids, gates=gw, counts=counts, offsets=offsets, perm=perm, inv=inv, y_perm=y, out=out)


# --------------------------------------------------------------------- host-RAM expert tier
class TierState:
    """Host-side LRU slot state of a tiered layer (the ``moe_tier_state`` struct and the numpy
    arrays it points at)."""

    def __init__(self, E: int, n_slots: int, slot_of_expert=None):
        import numpy as np

        if slot_of_expert is None:
            slot_of_expert = np.full(E, -1, dtype=np.int32)
        assert slot_of_expert.dtype == np.int32 and slot_of_expert.shape == (E,) and slot_of_expert.flags.c_contiguous
        slot_of_expert[:] = -1
        self.slot_of_expert = slot_of_expert
        self.expert_of_slot = np.full(n_slots, -1, dtype=np.int32)
        self.last_use = np.zeros(n_slots, dtype=np.int64)
        self.c = MoeTierState(E, n_slots, self.slot_of_expert.ctypes.data, self.expert_of_slot.ctypes.data,
                              self.last_use.ctypes.data, 0)

    @property
    def tick(self) -> int:
        return self.c.tick


def moe_tier_plan(st: TierState, ids_host):
    """ids_host: int32 numpy array of routed expert ids.  Returns (load_expert, load_slot)."""
    import numpy as np

    ids = np.ascontiguousarray(ids_host, dtype=np.int32).reshape(-1)
    S = st.c.n_slots
    le, ls = np.zeros(S, dtype=np.int32), np.zeros(S, dtype=np.int32)
    n = ctypes.c_int32(0)
    _check("moe_tier_plan", lib.moe_tier_plan(ctypes.byref(st.c), ids.ctypes.data, ids.size, le.ctypes.data,
                                              ls.ctypes.data, ctypes.byref(n)))
    return le[:n.value].copy(), ls[:n.value].copy()


def moe_tier_load(host_w: MoeWeights, slot_w: MoeWeights, load_expert, load_slot):
    import numpy as np

    le = np.ascontiguousarray(load_expert, dtype=np.int32)
    ls = np.ascontiguousarray(load_slot, dtype=np.int32)
    _check("moe_tier_load", lib.moe_tier_load(ctypes.byref(host_w), ctypes.byref(slot_w), le.ctypes.data,
                                              ls.ctypes.data, le.size, _stream()))


def moe_tier_remap(ids: torch.Tensor, slot_of_expert: torch.Tensor, out=None):
    _dev(ids, torch.int32, "topk_ids")
    _dev(slot_of_expert, torch.int32, "slot_of_expert")
    out = torch.empty_like(ids) if out is None else out
    _check("moe_tier_remap", lib.moe_tier_remap(_ptr(ids), ids.numel(), _ptr(slot_of_expert), _ptr(out),
                                                _stream()))
    return out


class TieredLayer:
    """One low-bit layer whose E experts live in pinned host memory, with n_slots of them held on
    the GPU as an LRU cache.  ``forward`` routes the batch, makes its experts resident, and runs
    the layer on the slots."""

    def __init__(self, fmt: int, E: int, H: int, I: int, arrays: dict, n_slots: int, device="cuda"):
        if not 1 <= n_slots <= E:
            raise ValueError("n_slots must be in [1, E]")
        if fmt not in (MOE_FMT_W2, MOE_FMT_W3):
            raise ValueError("the tier holds 2-bit or 3-bit experts")
        for key in ("w1_codes", "w1_scales", "w2_codes", "w2_scales"):
            if arrays.get(key) is None or arrays[key].shape[0] != E:
                raise ValueError(f"{key}: expected an array with a leading axis of {E} experts")
        self.fmt, self.E, self.H, self.I, self.n_slots = fmt, E, H, I, n_slots
        keys = ("w1_codes", "w1_scales", "w2_codes", "w2_scales")
        self.host = {}
        self.slot = {}
        for key in keys:
            a = arrays[key]
            t = torch.from_numpy(a.view(_np_uint_as_int(a.dtype)))
            self.host[key] = t.pin_memory()
            self.slot[key] = torch.zeros((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=device)
        self.host_c = MoeWeights(E, H, I, fmt, *(self.host[k_].data_ptr() for k_ in keys), 0, None, None, None,
                                 None, None, 0)
        self.slot_dw = DeviceWeights.__new__(DeviceWeights)
        self.slot_dw.fmt, self.slot_dw.E, self.slot_dw.H, self.slot_dw.I = fmt, n_slots, H, I
        self.slot_dw.n_hot, self.slot_dw.t = 0, self.slot
        self.slot_dw.c = MoeWeights(n_slots, H, I, fmt, *(self.slot[k_].data_ptr() for k_ in keys), 0, None, None,
                                    None, None, None, 0)
        # the slot table lives in pinned host memory (the plan writes it in place) and is copied
        # to the device asynchronously; the next plan runs only after the next batch's ids have
        # been read back, i.e. after that copy has completed
        self.table_h = torch.full((E,), -1, dtype=torch.int32).pin_memory()
        self.state = TierState(E, n_slots, self.table_h.numpy())
        self.table = torch.full((E,), -1, dtype=torch.int32, device=device)
        self.ids_h = torch.empty(0, dtype=torch.int32).pin_memory()
        self.loaded = 0  # experts copied host -> device so far
        self._table2 = None
        self._side = None

    def forward(self, logits: torch.Tensor, x: torch.Tensor, k: int, out_fp32: bool = True):
        ids, gw = moe_route(logits, k)
        R = ids.numel()
        if self.ids_h.numel() < R:
            self.ids_h = torch.empty(R, dtype=torch.int32).pin_memory()
        self.ids_h[:R].copy_(ids.view(-1), non_blocking=True)
        torch.cuda.current_stream().synchronize()  # the plan needs this batch's experts
        le, ls = moe_tier_plan(self.state, self.ids_h[:R].numpy())
        moe_tier_load(self.host_c, self.slot_dw.c, le, ls)
        self.loaded += len(le)
        self.table.copy_(self.table_h, non_blocking=True)
        sids = moe_tier_remap(ids, self.table)
        counts, offsets, perm, inv = moe_permute(sids, self.n_slots)
        y = moe_expert_ffn(self.slot_dw, x, k, counts, offsets, perm)
        out = moe_combine(y, inv, gw, out_fp32=out_fp32)
        return dict(ids=ids, slot_ids=sids, gates=gw, counts=counts, offsets=offsets, perm=perm, inv=inv,
                    y_perm=y, out=out, n_load=len(le))

    def forward_pipelined(self, batches, k: int, out_fp32: bool = True):
        """A sequence of independent batches [(logits, x), ...] with the copies of batch i+1
        overlapping the FFN of batch i: batch i+1 is routed, planned and loaded on a second
        stream while the main stream computes batch i.  Its plan counts batch i's experts as
        used too, so none of the slots batch i reads is evicted (the slot budget must hold the
        experts of two consecutive batches); its loads wait until batch i-1 is done.  Returns
        the outputs in order; each is bit-equal to `forward` on that batch alone."""
        import numpy as np

        if self._side is None:
            self._side = torch.cuda.Stream()
            self._table2 = torch.full_like(self.table, -1)
        main, side = torch.cuda.current_stream(), self._side
        tables = (self.table, self._table2)

        def stage_in(i, prev_ids, wait_done):
            lg = batches[i][0]
            with torch.cuda.stream(side):
                ids, gw = moe_route(lg, k)
                ids_h = torch.empty(ids.numel(), dtype=torch.int32).pin_memory()
                ids_h.copy_(ids.view(-1), non_blocking=True)
                got = torch.cuda.Event()
                got.record(side)
            got.synchronize()
            ids_np = ids_h.numpy()
            need = ids_np if prev_ids is None else np.concatenate([ids_np, prev_ids])
            le, ls = moe_tier_plan(self.state, need)
            with torch.cuda.stream(side):
                if wait_done is not None:
                    side.wait_event(wait_done)  # batch i-2 has left its slots and its slot table
                moe_tier_load(self.host_c, self.slot_dw.c, le, ls)
                tables[i % 2].copy_(self.table_h, non_blocking=True)
                ready = torch.cuda.Event()
                ready.record(side)
            self.loaded += len(le)
            return ids, gw, ids_np, ready, len(le)

        side.wait_stream(main)  # the inputs were written on the main stream before this call
        outs, done = [], []
        nxt = stage_in(0, None, None) if batches else None
        for i in range(len(batches)):
            ids, gw, ids_np, ready, nl = nxt
            main.wait_event(ready)
            ids.record_stream(main)
            gw.record_stream(main)
            x = batches[i][1]
            sids = moe_tier_remap(ids, tables[i % 2])
            counts, offsets, perm, inv = moe_permute(sids, self.n_slots)
            y = moe_expert_ffn(self.slot_dw, x, k, counts, offsets, perm)
            out = moe_combine(y, inv, gw, out_fp32=out_fp32)
            ev = torch.cuda.Event()
            ev.record(main)
            done.append(ev)
            outs.append(dict(ids=ids, out=out, n_load=nl))
            if i + 1 < len(batches):
                nxt = stage_in(i + 1, ids_np, done[i - 1] if i >= 1 else None)
        return outs
