"""The gated temporal scan as a torch.autograd.Function over the C ABI.

The pattern follows the BURT-IMMA CUDA Kernel API Reference page, section
6.3 "PyTorch Custom Op Integration" (a kernel library reached through
ctypes, section 6.2, wrapped in an autograd Function that saves what its
backward needs); here the forward calls ``gscan_forward_ex`` and the backward
``gscan_backward_full_ex`` (weight and input gradients from one call) or
``gscan_backward_ex`` (weight gradients only, when no input needs a
gradient).  The backward replays the forward from the saved inputs, as
Backward Step 1 of the design spec does, so nothing but the inputs is kept
between the passes.  Argument marshalling only: every step runs in the HIP
library.
"""
from __future__ import annotations

import torch

from . import binding


class GatedScanFunction(torch.autograd.Function):
    """context = gated_scan(h_history, h_s2, W_A, W_B, W_C, K, a_shift).

    h_history [B*K, SH2] and h_s2 [B, SH2] (float32 or bfloat16), W_* [SH2, D]
    float32, all contiguous on one GPU; context [B, D] float32.  Gradients:
    W_* in float32; h_history / h_s2 in their own dtype (the library forms
    them in float32; bfloat16 inputs receive them rounded to bfloat16).
    """

    @staticmethod
    def forward(ctx, h_history, h_s2, W_A, W_B, W_C, K: int, a_shift: float = 0.0):
        out = binding.forward(h_history, h_s2, W_A, W_B, W_C, int(K), float(a_shift))
        ctx.save_for_backward(h_history, h_s2, W_A, W_B, W_C)
        ctx.K = int(K)
        ctx.a_shift = float(a_shift)
        return out

    @staticmethod
    def backward(ctx, d_context):
        h_history, h_s2, W_A, W_B, W_C = ctx.saved_tensors
        d = d_context.to(torch.float32).contiguous()
        args = (h_history, h_s2, W_A, W_B, W_C, ctx.K)
        need_in = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        if need_in:
            dWA, dWB, dWC, dh, dhs2 = binding.backward_full(*args, d, ctx.a_shift)
            dh = dh.to(h_history.dtype) if ctx.needs_input_grad[0] else None
            dhs2 = dhs2.to(h_s2.dtype) if ctx.needs_input_grad[1] else None
        else:
            dWA, dWB, dWC = binding.backward(*args, d, ctx.a_shift)
            dh = dhs2 = None
        return (dh, dhs2,
                dWA if ctx.needs_input_grad[2] else None,
                dWB if ctx.needs_input_grad[3] else None,
                dWC if ctx.needs_input_grad[4] else None,
                None, None)


def gated_scan(h_history, h_s2, W_A, W_B, W_C, K: int, a_shift: float = 0.0):
    """Differentiable forward of the scan (see GatedScanFunction)."""
    return GatedScanFunction.apply(h_history, h_s2, W_A, W_B, W_C, K, a_shift)
