"""Seeded synthetic inputs (host side), shared by the HIP path's tests and
benchmark and by the CPU oracle.  Holds no arithmetic of the scan.

The generator itself is C (`csrc/synth.c`, built into `libgscan_synth.so`):
counter-based SplitMix64 + Box-Muller, thread-count independent.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import workloads as wl

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgscan_synth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it first (__graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.gscan_synth_normal_f32.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_void_p]
        lib.gscan_synth_normal_f32.restype = None
        lib.gscan_synth_round_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.gscan_synth_round_bf16.restype = None
        lib.gscan_synth_splitmix64_first.argtypes = [ctypes.c_uint64]
        lib.gscan_synth_splitmix64_first.restype = ctypes.c_uint64
        lib.gscan_synth_normal_one.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64]
        lib.gscan_synth_normal_one.restype = ctypes.c_double
        _lib = lib
    return _lib


def splitmix64_first(state: int) -> int:
    return int(_load().gscan_synth_splitmix64_first(ctypes.c_uint64(state & (2**64 - 1))))


def normal_one(seed: int, tid: int, n: int) -> float:
    return float(_load().gscan_synth_normal_one(seed, tid, n))


def normal_f32(seed: int, tid: int, shape, stddev: float = 1.0, first: int = 0) -> np.ndarray:
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    n = out.size
    if n:
        _load().gscan_synth_normal_f32(seed, tid, float(stddev), int(first), n,
                                       out.ctypes.data)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> raw bfloat16 bits (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        _load().gscan_synth_round_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bits to float32 (storage conversion only)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(w: wl.Workload, seed: int | None = None, B: int | None = None,
                with_grad: bool = True) -> dict:
    """Host arrays for workload `w`.

    h_history [B*K, SH2] and h_s2 [B, SH2] are float32, or raw bfloat16 bits
    (uint16) when w.in_dtype == "bf16"; W_A, W_B, W_C [SH2, D] and
    d_context [B, D] are float32.  `B` overrides the batch (the first B
    samples of the same streams, so a smaller batch is a prefix of the larger).
    """
    seed = w.seed if seed is None else seed
    B = w.B if B is None else B
    h = normal_f32(seed, wl.TID_H_HISTORY, (B * w.K, w.SH2))
    hs2 = normal_f32(seed, wl.TID_H_S2, (B, w.SH2))
    if w.in_dtype == "bf16":
        h = round_bf16(h)
        hs2 = round_bf16(hs2)
    out = {
        "h_history": h,
        "h_s2": hs2,
        "W_A": normal_f32(seed, wl.TID_W_A, (w.SH2, w.D), w.w_std),
        "W_B": normal_f32(seed, wl.TID_W_B, (w.SH2, w.D), w.w_std),
        "W_C": normal_f32(seed, wl.TID_W_C, (w.SH2, w.D), w.w_std),
    }
    if with_grad:
        out["d_context"] = normal_f32(seed, wl.TID_D_CONTEXT, (B, w.D))
    return out


def make_cifg_inputs(w: "wl.CifgWorkload", seed: int | None = None) -> dict:
    """Host arrays for the CIFG update: C [B, d, d] ~ N(0, 1/d) (a memory of
    modest norm), H [B, d] and X [B, d_input] ~ N(0, 1), W_f [d, d + d_input]
    ~ N(0, 1/(d + d_input)), b_f [d] ~ N(0, 1); all float32."""
    seed = w.seed if seed is None else seed
    d, di = w.d_model, w.d_input
    return {
        "C": normal_f32(seed, wl.TID_CIFG_C, (w.B, d, d), 1.0 / np.sqrt(d)),
        "H": normal_f32(seed, wl.TID_CIFG_H, (w.B, d)),
        "X": normal_f32(seed, wl.TID_CIFG_X, (w.B, di)),
        "W_f": normal_f32(seed, wl.TID_CIFG_W, (d, d + di), 1.0 / np.sqrt(d + di)),
        "b_f": normal_f32(seed, wl.TID_CIFG_B, (d,)),
    }
