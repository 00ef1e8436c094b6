"""Number formats used by the oracle: bf16 rounding and weight dequantisation.

bf16 here is round-to-nearest-even of a real number to 8 significant bits
(the storage format of the bf16 activations and checkpoints).  Dequantised
weights are ``float(scale) * code`` (mirror-sd README, "The Story": int8
codes with per-channel fp16 scales; "Results": 4-bit target weights, here one
fp16 scale per 64-wide group along K).
"""
from __future__ import annotations

import contextlib

import numpy as np

F64 = np.float64

# Accumulation of linear(): "f64" (the oracle) or "f32" (float32 products
# and sums).  The second mode exists only to measure the bf16 noise floor: how
# far two equally valid accumulation orders of the same bf16 model drift apart
# once their bf16 roundings start to differ.
_ACCUM = ["f64"]


@contextlib.contextmanager
def gemm_accumulation(kind: str):
    assert kind in ("f64", "f32")
    old = _ACCUM[0]
    _ACCUM[0] = kind
    try:
        yield
    finally:
        _ACCUM[0] = old


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float64.

    x = m * 2**e with 0.5 <= |m| < 1; keeping 8 significant bits means
    rounding m * 2**8 to an integer.  All steps are exact in float64 except
    the single rounding done by rint (half to even).  bf16 subnormals and
    overflow are not modelled (the step never produces them).
    """
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def identity(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


def rounder(act: str):
    """The materialisation rounding of a stack: bf16 or none (fp32 models,
    evaluated in float64)."""
    return round_bf16 if act == "bf16" else identity


def dequant(weight, rows=None) -> np.ndarray:
    """Dequantise a canonical weight (or a slice of its rows) to float64.

    ``weight`` has ``fmt``, ``values`` (float formats) or ``codes`` +
    ``scales`` (int8: one fp16 scale per row; int4: one per 64-wide group).
    """
    sl = slice(None) if rows is None else rows
    if weight.values is not None:
        return np.asarray(weight.values[sl], dtype=F64)
    codes = np.asarray(weight.codes[sl], dtype=F64)
    scales = np.asarray(weight.scales[sl], dtype=np.float16).astype(F64)
    if scales.ndim == 1:                      # per output channel
        return codes * scales[:, None]
    n, k = codes.shape                        # per 64-wide group along K
    g = scales.shape[1]
    return (codes.reshape(n, g, k // g) * scales[:, :, None]).reshape(n, k)


def linear(x: np.ndarray, weight, rows=None, chunk_rows: int = 16384) -> np.ndarray:
    """y = x @ deq(W[rows]).T in float64, dequantising ``chunk_rows`` rows at a
    time.  ``rows`` is an optional (start, stop) row range of W."""
    x = np.asarray(x, dtype=F64)
    lo, hi = (0, weight.n) if rows is None else rows
    out = np.empty((x.shape[0], hi - lo), dtype=F64)
    f32 = _ACCUM[0] == "f32"
    x32 = x.astype(np.float32) if f32 else None
    for r0 in range(lo, hi, chunk_rows):
        r1 = min(hi, r0 + chunk_rows)
        w = dequant(weight, slice(r0, r1))
        out[:, r0 - lo:r1 - lo] = (x32 @ w.astype(np.float32).T) if f32 else x @ w.T
    return out
