"""Helpers for the GPU tests: host arrays -> device tensors, calls through the
C ABI (via the package binding), and the parity metrics."""
import numpy as np
import torch

import gated_linear_recurrence_history_amd as gs
from gated_linear_recurrence_history_amd import workloads as wl

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:  # raw bfloat16 bits
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def device_inputs(x: dict) -> dict:
    return {k: to_dev(v) for k, v in x.items()}


def gpu_forward(t: dict, K: int, a_shift: float) -> np.ndarray:
    ctx = gs.forward(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], K, a_shift)
    torch.cuda.synchronize()
    return ctx.cpu().numpy()


def gpu_backward(t: dict, K: int, a_shift: float, d_context=None):
    d = t["d_context"] if d_context is None else d_context
    dW = gs.backward(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], K, d, a_shift)
    torch.cuda.synchronize()
    return tuple(g.cpu().numpy() for g in dW)


def ctx_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / (1 + |ref|)  (the context tolerance metric)."""
    return float(np.max(np.abs(gpu.astype(np.float64) - ref) / (1.0 + np.abs(ref))))


def rel_l2(gpu: np.ndarray, ref: np.ndarray) -> float:
    """||gpu - ref||_2 / ||ref||_2, or ||gpu||_2 when ref is exactly zero."""
    nr = float(np.linalg.norm(ref))
    d = float(np.linalg.norm(gpu.astype(np.float64) - ref))
    return d / nr if nr > 0 else d


def workload(B, K, SH2, D, dtype="f32", a_shift=0.0, seed=777) -> wl.Workload:
    return wl.Workload(f"case_B{B}_K{K}_S{SH2}_D{D}_{dtype}", B, K, SH2, D, in_dtype=dtype,
                       a_shift=a_shift, seed=seed)
