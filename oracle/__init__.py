"""CPU oracle for the gated temporal scan -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product path (the HIP library and its binding)
never touches it.

`forward` / `forward_enrich` / `backward` / `backward_inputs` / `cifg_update` /
`column_sums` widen every input exactly to float64 (float32 as is,
bfloat16 given as raw uint16 bits by zero-extending the low mantissa) and
call plain double-precision C loops (gscan_oracle.c).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_forward.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                       ctypes.c_double, dp]
        lib.oracle_forward.restype = None
        lib.oracle_backward.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                        ctypes.c_double, dp, dp, dp, dp]
        lib.oracle_backward.restype = None
        lib.oracle_backward_inputs.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                               ctypes.c_double, dp, dp, dp]
        lib.oracle_backward_inputs.restype = None
        lib.oracle_cifg_update.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, dp]
        lib.oracle_cifg_update.restype = None
        lib.oracle_column_sums.argtypes = [dp, i64, i64, dp]
        lib.oracle_column_sums.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def widen(x: np.ndarray) -> np.ndarray:
    """Exact widening to float64.  uint16 arrays are raw bfloat16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float64)


def _shapes(h_history, h_s2, W_A, K):
    SH2, D = W_A.shape
    B = h_s2.shape[0]
    if h_history.shape != (B * K, SH2) or h_s2.shape != (B, SH2):
        raise ValueError(f"shape mismatch: h_history {h_history.shape}, h_s2 {h_s2.shape}, "
                         f"W {W_A.shape}, K {K}")
    return B, SH2, D


def forward(h_history, h_s2, W_A, W_B, W_C, K: int, a_shift: float = 0.0) -> np.ndarray:
    """context[B, D] in float64."""
    h, hs, wa, wb, wc = (widen(a) for a in (h_history, h_s2, W_A, W_B, W_C))
    B, SH2, D = _shapes(h, hs, wa, K)
    ctx = np.empty((B, D), dtype=np.float64)
    _load().oracle_forward(h.ctypes.data, hs.ctypes.data, wa.ctypes.data, wb.ctypes.data,
                           wc.ctypes.data, B, K, SH2, D, float(a_shift), ctx.ctypes.data)
    return ctx


def forward_enrich(h_history, h_s2, W_A, W_B, W_C, K: int, h_enriched, col_offset: int,
                   a_shift: float = 0.0) -> np.ndarray:
    """h_enriched [B, ld] (float64) with the context added element-wise into
    columns col_offset .. col_offset + D - 1 of each row, other columns as
    given.  The design spec's Forward Step 2 ends by accumulating the context
    into h_enriched and its Step 3 applies it element-wise; the spec fixes
    neither the buffer's width nor where the context lands, so the caller
    names the row pitch and the column offset."""
    ctx = forward(h_history, h_s2, W_A, W_B, W_C, K, a_shift)
    out = widen(h_enriched).copy()
    D = ctx.shape[1]
    if out.ndim != 2 or out.shape[0] != ctx.shape[0] or not 0 <= col_offset <= out.shape[1] - D:
        raise ValueError(f"h_enriched {out.shape} cannot take [B, {D}] at column {col_offset}")
    out[:, col_offset:col_offset + D] += ctx
    return out


def backward(h_history, h_s2, W_A, W_B, W_C, K: int, d_context, a_shift: float = 0.0):
    """(dW_A, dW_B, dW_C), each [SH2, D] float64, for L = sum(d_context * context)."""
    h, hs, wa, wb, wc, dc = (widen(a) for a in (h_history, h_s2, W_A, W_B, W_C, d_context))
    B, SH2, D = _shapes(h, hs, wa, K)
    if dc.shape != (B, D):
        raise ValueError(f"d_context shape {dc.shape} != {(B, D)}")
    dwa = np.empty((SH2, D), dtype=np.float64)
    dwb = np.empty((SH2, D), dtype=np.float64)
    dwc = np.empty((SH2, D), dtype=np.float64)
    _load().oracle_backward(h.ctypes.data, hs.ctypes.data, wa.ctypes.data, wb.ctypes.data,
                            wc.ctypes.data, B, K, SH2, D, float(a_shift), dc.ctypes.data,
                            dwa.ctypes.data, dwb.ctypes.data, dwc.ctypes.data)
    return dwa, dwb, dwc


def backward_inputs(h_history, h_s2, W_A, W_B, W_C, K: int, d_context, a_shift: float = 0.0):
    """(d_h_history [B*K, SH2], d_h_s2 [B, SH2]) float64, for L = sum(d_context * context)."""
    h, hs, wa, wb, wc, dc = (widen(a) for a in (h_history, h_s2, W_A, W_B, W_C, d_context))
    B, SH2, D = _shapes(h, hs, wa, K)
    if dc.shape != (B, D):
        raise ValueError(f"d_context shape {dc.shape} != {(B, D)}")
    dh = np.empty((B * K, SH2), dtype=np.float64)
    dhs = np.empty((B, SH2), dtype=np.float64)
    _load().oracle_backward_inputs(h.ctypes.data, hs.ctypes.data, wa.ctypes.data,
                                   wb.ctypes.data, wc.ctypes.data, B, K, SH2, D, float(a_shift),
                                   dc.ctypes.data, dh.ctypes.data, dhs.ctypes.data)
    return dh, dhs


def cifg_update(C, H, X, W_f, b_f) -> np.ndarray:
    """The CIFG matrix-memory update of every sample, independent mode
    (BURT-IMMA API reference, batched_cifg_update with shared_memory_mode
    false; steps 1-4 of cifg_update): returns the updated C [B, d, d] in
    float64.  H [B, d], X [B, d_input], W_f [d, d + d_input], b_f [d]."""
    c, h, x, w, bf = (widen(a) for a in (C, H, X, W_f, b_f))
    B, d = h.shape
    d_input = x.shape[1] if x.ndim == 2 else 0
    if (c.shape != (B, d, d) or x.shape != (B, d_input) or w.shape != (d, d + d_input)
            or bf.shape != (d,)):
        raise ValueError(f"shape mismatch: C {c.shape}, H {h.shape}, X {x.shape}, "
                         f"W_f {w.shape}, b_f {bf.shape}")
    out = np.empty_like(c)
    _load().oracle_cifg_update(c.ctypes.data, h.ctypes.data, x.ctypes.data, w.ctypes.data,
                               bf.ctypes.data, B, d, d_input, out.ctypes.data)
    return out


def column_sums(grad) -> np.ndarray:
    """out[j] = sum_r grad[r, j] in float64 (the bias-gradient reduction)."""
    g = widen(grad)
    if g.ndim != 2:
        raise ValueError(f"grad must be 2-D, got shape {g.shape}")
    g = np.ascontiguousarray(g)
    rows, cols = g.shape
    out = np.empty(cols, dtype=np.float64)
    _load().oracle_column_sums(g.ctypes.data, rows, cols, out.ctypes.data)
    return out


def sample_rows(inputs: dict, K: int, samples) -> dict:
    """Inputs restricted to the given samples (forward is per-sample independent)."""
    samples = np.asarray(samples, dtype=np.int64)
    rows = (samples[:, None] * K + np.arange(K)[None, :]).reshape(-1)
    out = dict(inputs)
    out["h_history"] = inputs["h_history"][rows]
    out["h_s2"] = inputs["h_s2"][samples]
    if "d_context" in inputs:
        out["d_context"] = inputs["d_context"][samples]
    return out
