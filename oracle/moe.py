"""The routed-expert MoE FFN, step by step, in fp64 -- test infrastructure only.

route -> permute -> (dequant) FC1 + SwiGLU -> FC2 -> combine.  Every step is the plain
definition; matmuls are numpy's (a library primitive used as one step).
"""
from __future__ import annotations

import numpy as np

from . import formats as F


# ------------------------------------------------------------------------ routing
def route(logits, k: int):
    """Top-k routing over router logits.

    [Moet-README] (hybrid section): every token is served by a few routed experts out
    of the layer's 384.  The pages do not state the score function; reading taken:
    * the k experts with the largest logits, ordered by (logit descending, expert id
      ascending) -- ties go to the lower id, and -0.0 equals +0.0;
    * gates = softmax over the k selected logits (so they sum to one).

    Returns ``topk_ids int32[T][k]`` (descending logit order) and ``gates f64[T][k]``."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    assert 1 <= k <= E
    assert not np.any(np.isnan(lg)), "NaN router logits are the caller's error"
    # a stable ascending sort of -logit keeps equal logits in expert-id order
    order = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    gates = z / z.sum(axis=1, keepdims=True)
    return ids, gates


# ---------------------------------------------------------------------- grouping
def permute(topk_ids, E: int):
    """Group the T*k routed rows by expert (stable).

    Row ``r' = t*k + j`` is the j-th expert choice of token t.  Reading (the pages do
    not describe grouping): counts[e] = rows routed to e, offsets = exclusive prefix sum
    (offsets[E] = T*k), rows ordered by (expert, token, slot); ``perm[r] = t*k + j``
    of the r-th grouped row and ``inv[t*k + j] = r``."""
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    R = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    assert counts.size == E
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty(R, dtype=np.int32)
    inv[perm] = np.arange(R, dtype=np.int32)
    return counts, offsets, perm, inv


# ------------------------------------------------------------------- the experts
def silu(a):
    """silu(a) = a * sigmoid(a) = a / (1 + e^-a)."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def fc1(x, W1):
    """a = x W1^T: ``f64[n][H] x f64[2I][H] -> f64[n][2I]``."""
    return x @ W1.T


def swiglu(a):
    """SwiGLU of the FC1 output: columns [0, I) are the gate, [I, 2I) the up projection
    (reading: gate rows first in W1).  h = silu(gate) * up."""
    I = a.shape[1] // 2
    return silu(a[:, :I]) * a[:, I:]


def fc2(h, W2):
    """y = h W2^T: ``f64[n][I] x f64[H][I] -> f64[n][H]``."""
    return h @ W2.T


def mxfp8_round_trip(v):
    return F.mxfp8_dequant(*F.mxfp8_quantize(v))


def swiglu_ffn(x, W1, W2, fp8: bool = False):
    """One expert on its rows.  [Moet-README] release notes of -r23: the MoE is FC1,
    SwiGLU (and, for FP8 compute, MXFP8 quantisation), then FC2.

    x ``f64[n][H]``; W1 ``f64[2I][H]``; W2 ``f64[H][I]``; everything in fp64.  With
    ``fp8`` the FC1 and FC2 inputs are MXFP8-quantised first (reading: FP8 matrix cores
    need both operands in FP8, so x is quantised like h)."""
    if fp8:
        x = mxfp8_round_trip(x)
    h = swiglu(fc1(x, W1))
    if fp8:
        h = mxfp8_round_trip(h)
    return fc2(h, W2)


class Layer:
    """Packed weights of one layer and the fp64 expert matrices they decode to.

    ``arrays`` holds the low-bit stacks (``w1_codes`` ... ``w2_scales`` with a leading
    [E] axis) and optionally ``hot_ids`` plus the MXFP4 stacks (``hot_w1_codes`` ...).
    ``fmt`` is "w2" or "w3".  ``hot_mode`` says what the MXFP4 stacks of the hot set are:

    * "replace": a hot expert is held in MXFP4 and computed in FP8 after the conversion of
      [Day0-MXFP4] section 4; its low-bit copy is not used (reading: the hot set *replaces*
      the low-bit copy of those experts);
    * "residual": [Moet-QA] (the FP4 delta cache: the hottest experts get an FP4-precision
      correction layer above their 2-bit weights) and [Moet-README] README line "2-bit
      experts on vLLM v0.24.0" (a 2-bit codebook plus an FP4 delta cache).  Reading: a hot
      expert's weight is its 2-bit weight plus the MXFP4 residual, summed element by element
      before the matmuls (so before SwiGLU), and computed like the 2-bit experts (bf16
      operands; the sum is formed exactly here in fp64)."""

    def __init__(self, fmt: str, arrays: dict, hot_mode: str = "replace"):
        assert hot_mode in ("replace", "residual")
        assert hot_mode == "replace" or fmt == "w2", "the FP4 residual sits on 2-bit experts"
        self.fmt = fmt
        self.a = arrays
        self.hot_mode = hot_mode
        hid = arrays.get("hot_ids", np.zeros(0, np.int32))
        self.hot = {int(e): s for s, e in enumerate(np.asarray(hid).tolist())}

    def is_fp8(self, e: int) -> bool:
        return e in self.hot and self.hot_mode == "replace"

    def fp8_image(self, e: int, which: int):
        """The converted FP8 workspace image of hot expert e's W{which}."""
        s = self.hot[e]
        return F.mxfp4_to_fp8(self.a[f"hot_w{which}_codes"][s], self.a[f"hot_w{which}_scales"][s])

    def low_bit(self, e: int, which: int) -> np.ndarray:
        """The low-bit weights of expert e's W{which}, decoded."""
        c, s = self.a[f"w{which}_codes"][e], self.a[f"w{which}_scales"][e]
        return F.dequant_w2(c, s) if self.fmt == "w2" else F.dequant_w3(c, s)

    def residual(self, e: int, which: int) -> np.ndarray:
        """The MXFP4 residual of hot expert e's W{which} (residual mode), decoded."""
        s = self.hot[e]
        return F.dequant_mxfp4(self.a[f"hot_w{which}_codes"][s], self.a[f"hot_w{which}_scales"][s])

    def dense(self, e: int, which: int) -> np.ndarray:
        if e in self.hot:
            if self.hot_mode == "replace":
                return F.dequant_fp8(*self.fp8_image(e, which))
            return self.low_bit(e, which) + self.residual(e, which)
        return self.low_bit(e, which)


def expert_ffn(layer: Layer, x_bits, k: int, offsets, perm, experts=None):
    """y_perm ``f64[T*k][H]``: row r is the FFN output of grouped row r, computed by the
    expert the row belongs to.  ``experts`` restricts the work to a subset (other rows
    stay NaN), for sampled checks at large sizes."""
    X = F.bf16_value(x_bits)
    off = np.asarray(offsets, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    E = off.size - 1
    R = perm.size
    H = X.shape[1]
    y = np.full((R, H), np.nan)
    for e in range(E) if experts is None else sorted(set(int(v) for v in experts)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        tok = perm[lo:hi] // k
        y[lo:hi] = swiglu_ffn(X[tok], layer.dense(e, 1), layer.dense(e, 2), layer.is_fp8(e))
    return y


# ------------------------------------------------------------------------ combine
def combine(y_perm, inv, gates, T: int, k: int):
    """out[t] = sum over j = 0..k-1 of gates[t, j] * y_perm[inv[t*k + j]] (fp64).
    Reading (not described on the pages): the gate-weighted sum of a token's expert
    outputs, in slot order."""
    y = np.asarray(y_perm, dtype=np.float64)
    inv = np.asarray(inv, dtype=np.int64).reshape(T, k)
    g = np.asarray(gates, dtype=np.float64).reshape(T, k)
    out = np.zeros((T, y.shape[1]))
    for j in range(k):
        out += g[:, j : j + 1] * y[inv[:, j]]
    return out


def layer_forward(layer: Layer, logits, x_bits, k: int):
    """The whole layer: returns a dict with every intermediate."""
    ids, gates = route(logits, k)
    E = np.asarray(logits).shape[1]
    counts, offsets, perm, inv = permute(ids, E)
    y = expert_ffn(layer, x_bits, k, offsets, perm)
    T = ids.shape[0]
    out = combine(y, inv, gates, T, k)
    return dict(ids=ids, gates=gates, counts=counts, offsets=offsets, perm=perm, inv=inv,
                y_perm=y, out=out)
