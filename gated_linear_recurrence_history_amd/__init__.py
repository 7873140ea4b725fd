"""MI355X-native gated temporal scan (Mamba2-style), forward and backward.

The compute path is the HIP library `libgscan.so` (hand-written gfx950
kernels behind a C ABI, declared in include/gscan.h); `forward` and
`backward` (and `backward_full`, which adds the input gradients) are thin
ctypes wrappers over it, and `gated_scan` is the same as a
torch.autograd.Function.  There is no CPU fallback.
"""
from .binding import (forward, forward_enrich, backward, backward_full,  # noqa: F401
                      backward_workspace_bytes, forward_workspace_bytes,
                      backward_full_workspace_bytes, backward_partials, backward_reduce,
                      batched_cifg_update, bias_grad_reduce, library_path, GScanError)
from . import workloads  # noqa: F401
from .autograd import GatedScanFunction, gated_scan  # noqa: F401

__all__ = ["forward", "forward_enrich", "backward", "backward_full", "backward_workspace_bytes",
           "forward_workspace_bytes", "backward_full_workspace_bytes", "backward_partials",
           "backward_reduce", "batched_cifg_update", "bias_grad_reduce", "library_path", "GScanError",
           "workloads", "GatedScanFunction", "gated_scan"]
