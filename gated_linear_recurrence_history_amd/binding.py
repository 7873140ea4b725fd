"""ctypes binding over libgscan.so (declared in include/gscan.h).

Argument marshalling only: shape/dtype/device checks, raw device pointers and
the current HIP stream go to the C ABI, every step of the computation runs in
the library's kernels.  PyTorch provides device memory and streams.  There is
no fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgscan.so")

GSCAN_F32 = 0
GSCAN_BF16 = 1

_lib = None


class GScanError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"gscan status {status}: {detail}")
        self.status = status


def library_path() -> str:
    return LIB_PATH


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build the HIP library first "
                               "(__graft_entry__.build()); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
        L.gscan_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]
        L.gscan_forward.restype = ctypes.c_int
        L.gscan_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp,
                                     vp]
        L.gscan_backward.restype = ctypes.c_int
        L.gscan_forward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp,
                                       ctypes.c_int, f32, vp, ctypes.c_size_t, vp]
        L.gscan_forward_ex.restype = ctypes.c_int
        L.gscan_backward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp,
                                        ctypes.c_int, f32, vp, ctypes.c_size_t, vp]
        L.gscan_backward_ex.restype = ctypes.c_int
        L.gscan_forward_enrich.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, i64,
                                           i64, ctypes.c_int, f32, vp, ctypes.c_size_t, vp]
        L.gscan_forward_enrich.restype = ctypes.c_int
        L.gscan_batched_cifg_update.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        L.gscan_batched_cifg_update.restype = ctypes.c_int
        L.gscan_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp,
                                             vp, ctypes.c_int, f32, vp]
        L.gscan_backward_noalloc.restype = ctypes.c_int
        L.gscan_backward_partials.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp,
                                              ctypes.c_int, f32, vp, ctypes.c_size_t, vp]
        L.gscan_backward_partials.restype = ctypes.c_int
        L.gscan_backward_reduce.argtypes = [vp, ctypes.c_size_t, i64, i64, i64, i64, ctypes.c_int,
                                            vp, vp, vp, vp]
        L.gscan_backward_reduce.restype = ctypes.c_int
        L.gscan_backward_full_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp,
                                             vp, vp, vp, ctypes.c_int, f32, vp, ctypes.c_size_t,
                                             vp]
        L.gscan_backward_full_ex.restype = ctypes.c_int
        L.gscan_backward_full_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        L.gscan_backward_full_workspace_bytes.restype = ctypes.c_size_t
        L.gscan_bias_grad_reduce.argtypes = [vp, i64, i64, vp, vp, ctypes.c_size_t, vp]
        L.gscan_bias_grad_reduce.restype = ctypes.c_int
        L.gscan_bias_grad_reduce_workspace_bytes.argtypes = [i64, i64]
        L.gscan_bias_grad_reduce_workspace_bytes.restype = ctypes.c_size_t
        L.gscan_backward_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        L.gscan_backward_workspace_bytes.restype = ctypes.c_size_t
        L.gscan_forward_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        L.gscan_forward_workspace_bytes.restype = ctypes.c_size_t
        L.gscan_status_string.argtypes = [ctypes.c_int]
        L.gscan_status_string.restype = ctypes.c_char_p
        L.gscan_last_error.argtypes = []
        L.gscan_last_error.restype = ctypes.c_char_p
        L.gscan_version.argtypes = []
        L.gscan_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        detail = lib().gscan_last_error().decode(errors="replace")
        raise GScanError(status, detail)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GSCAN_F32
    if t.dtype == torch.bfloat16:
        return GSCAN_BF16
    raise TypeError(f"h_history/h_s2 must be float32 or bfloat16, got {t.dtype}")


def _stream_handle(stream, device):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _prep(h_history, h_s2, W_A, W_B, W_C, K):
    import torch
    tensors = (h_history, h_s2, W_A, W_B, W_C)
    dev = h_history.device
    for t in tensors:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("all operands must be torch tensors on a GPU device")
        if t.device != dev:
            raise ValueError("all operands must be on the same device")
        if not t.is_contiguous():
            raise ValueError("all operands must be contiguous (row-major)")
    code = _dtype_code(h_history)
    if h_s2.dtype != h_history.dtype:
        raise TypeError("h_s2 must have the dtype of h_history")
    for w in (W_A, W_B, W_C):
        if w.dtype != torch.float32:
            raise TypeError("weights must be float32")
        if w.shape != W_A.shape or w.dim() != 2:
            raise ValueError("W_A, W_B, W_C must all be [SH2, D]")
    SH2, D = W_A.shape
    K = int(K)
    if K <= 0 or h_history.dim() != 2 or h_history.shape[1] != SH2 or h_history.shape[0] % K:
        raise ValueError(f"h_history must be [B*K, SH2]; got {tuple(h_history.shape)}, K={K}")
    B = h_history.shape[0] // K
    if tuple(h_s2.shape) != (B, SH2):
        raise ValueError(f"h_s2 must be [B, SH2] = {(B, SH2)}; got {tuple(h_s2.shape)}")
    return dev, code, B, K, SH2, D


def _check_f32(t, shape, dev, name):
    """A caller-supplied float32 tensor the library reads or writes: the exact
    shape, contiguous, on the inputs' device (the kernels index it by shape
    alone, so anything else would be read or written out of bounds)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device != dev:
        raise ValueError(f"{name} must be a tensor on {dev}")
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}; "
                         f"got {t.dtype} {tuple(t.shape)}")


def _check_outs(out, shapes, dev, name="out"):
    if not isinstance(out, (tuple, list)) or len(out) != len(shapes):
        raise ValueError(f"{name} must hold {len(shapes)} tensors")
    for i, (t, shp) in enumerate(zip(out, shapes)):
        _check_f32(t, shp, dev, f"{name}[{i}]")


def _check_workspace(ws, need, dev):
    """A caller workspace: a contiguous uint8 GPU tensor on `dev` of at least
    `need` bytes (the library also checks size and alignment)."""
    import torch
    if not isinstance(ws, torch.Tensor) or ws.device != dev:
        raise ValueError(f"workspace must be a tensor on {dev}")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, needs {need}")


def forward_workspace_bytes(B: int, K: int, SH2: int, D: int, bf16: bool = False) -> int:
    return int(lib().gscan_forward_workspace_bytes(B, K, SH2, D,
                                                   GSCAN_BF16 if bf16 else GSCAN_F32))


def _forward_workspace(workspace, B, K, SH2, D, code, dev):
    """(pointer, bytes, tensor to keep alive) of the forward's workspace: the
    caller's (checked), or one from torch's caching allocator where the shape
    needs one, or none."""
    import torch
    need = int(lib().gscan_forward_workspace_bytes(B, K, SH2, D, code))
    if workspace is not None:
        _check_workspace(workspace, need, dev)
        return workspace.data_ptr(), workspace.numel(), workspace
    if need == 0:
        return None, 0, None
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    return ws.data_ptr(), need, ws


def forward(h_history, h_s2, W_A, W_B, W_C, K: int, a_shift: float = 0.0, out=None,
            workspace=None, stream=None):
    """context[B, D] (float32) = C * x_K for every (sample, state).

    `workspace` may be a uint8 device tensor of at least forward_workspace_bytes()
    bytes (only shapes outside the fused kernels use one); otherwise one is
    taken from torch's caching allocator where needed.
    """
    import torch
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    if out is None:
        out = torch.empty((B, D), dtype=torch.float32, device=dev)
    else:
        _check_f32(out, (B, D), dev, "out")
    wp, wn, _keep = _forward_workspace(workspace, B, K, SH2, D, code, dev)
    _check(lib().gscan_forward_ex(
        h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
        W_C.data_ptr(), B, K, SH2, D, out.data_ptr(), code, float(a_shift), wp, wn,
        _stream_handle(stream, dev)))
    return out


def forward_enrich(h_history, h_s2, W_A, W_B, W_C, K: int, h_enriched, col_offset: int = 0,
                   a_shift: float = 0.0, context_out=None, workspace=None, stream=None):
    """Adds context[b, s] into h_enriched[b, col_offset + s] in place
    (h_enriched: contiguous float32 [B, ld] on the inputs' device) and, if
    `context_out` is given ([B, D] float32), writes the context there too.
    Returns h_enriched."""
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    if h_enriched.dim() != 2:
        raise ValueError("h_enriched must be [B, ld]")
    _check_f32(h_enriched, (B, h_enriched.shape[1]), dev, "h_enriched")
    ld = int(h_enriched.shape[1])
    if not 0 <= int(col_offset) <= ld - D:
        raise ValueError(f"col_offset {col_offset} outside 0..{ld - D} for h_enriched [B, {ld}]")
    cptr = None
    if context_out is not None:
        _check_f32(context_out, (B, D), dev, "context_out")
        cptr = context_out.data_ptr()
    wp, wn, _keep = _forward_workspace(workspace, B, K, SH2, D, code, dev)
    _check(lib().gscan_forward_enrich(
        h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
        W_C.data_ptr(), B, K, SH2, D, cptr, h_enriched.data_ptr(), ld, int(col_offset), code,
        float(a_shift), wp, wn, _stream_handle(stream, dev)))
    return h_enriched


def prepare_forward_enrich(h_history, h_s2, W_A, W_B, W_C, K, h_enriched, col_offset=0,
                           a_shift=0.0, stream=None):
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(h_enriched, (B, h_enriched.shape[1]), dev, "h_enriched")
    ld = int(h_enriched.shape[1])
    if not 0 <= int(col_offset) <= ld - D:
        raise ValueError("col_offset out of range")
    wp, wn, ws = _forward_workspace(None, B, K, SH2, D, code, dev)
    args = (h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
            W_C.data_ptr(), B, K, SH2, D, None, h_enriched.data_ptr(), ld, int(col_offset), code,
            ctypes.c_float(a_shift), wp, wn, _stream_handle(stream, dev))
    return Prepared(lib().gscan_forward_enrich, args,
                    (h_history, h_s2, W_A, W_B, W_C, h_enriched, ws))


def batched_cifg_update(C_batch, H, X, W_f, b_f, stream=None):
    """In-place CIFG matrix-memory update of every sample (independent mode):
    C_batch [B, d, d] <- f * C_batch + (1 - f) * h h^T with
    f = sigmoid(W_f [h; x] + b_f) per row.  All float32 contiguous GPU
    tensors on one device; X is [B, d_input] (d_input may be 0).  Returns
    C_batch."""
    import torch
    if not isinstance(C_batch, torch.Tensor) or not C_batch.is_cuda or C_batch.dim() != 3:
        raise ValueError("C_batch must be a [B, d, d] GPU tensor")
    dev = C_batch.device
    B, d = int(C_batch.shape[0]), int(C_batch.shape[1])
    _check_f32(C_batch, (B, d, d), dev, "C_batch")
    _check_f32(H, (B, d), dev, "H")
    if X.dim() != 2:
        raise ValueError("X must be [B, d_input]")
    din = int(X.shape[1])
    _check_f32(X, (B, din), dev, "X")
    _check_f32(W_f, (d, d + din), dev, "W_f")
    _check_f32(b_f, (d,), dev, "b_f")
    _check(lib().gscan_batched_cifg_update(
        C_batch.data_ptr(), H.data_ptr(), X.data_ptr() if din else None, W_f.data_ptr(),
        b_f.data_ptr(), B, d, din, _stream_handle(stream, dev)))
    return C_batch


def prepare_batched_cifg_update(C_batch, H, X, W_f, b_f, stream=None):
    B, d, din = int(C_batch.shape[0]), int(C_batch.shape[1]), int(X.shape[1])
    dev = C_batch.device
    for t, shp, nm in ((C_batch, (B, d, d), "C_batch"), (H, (B, d), "H"), (X, (B, din), "X"),
                       (W_f, (d, d + din), "W_f"), (b_f, (d,), "b_f")):
        _check_f32(t, shp, dev, nm)
    args = (C_batch.data_ptr(), H.data_ptr(), X.data_ptr() if din else None, W_f.data_ptr(),
            b_f.data_ptr(), B, d, din, _stream_handle(stream, dev))
    return Prepared(lib().gscan_batched_cifg_update, args, (C_batch, H, X, W_f, b_f))


def backward_workspace_bytes(B: int, K: int, SH2: int, D: int, bf16: bool = False) -> int:
    return int(lib().gscan_backward_workspace_bytes(B, K, SH2, D,
                                                    GSCAN_BF16 if bf16 else GSCAN_F32))


def backward(h_history, h_s2, W_A, W_B, W_C, K: int, d_context, a_shift: float = 0.0,
             out=None, workspace=None, stream=None):
    """(dW_A, dW_B, dW_C), each float32 [SH2, D], for L = sum(d_context * context).

    `workspace` may be a uint8 device tensor of at least backward_workspace_bytes()
    bytes; otherwise one is taken from torch's caching allocator.
    """
    import torch
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(d_context, (B, D), dev, "d_context")
    if out is None:
        out = tuple(torch.empty((SH2, D), dtype=torch.float32, device=dev) for _ in range(3))
    else:
        _check_outs(out, [(SH2, D)] * 3, dev)
    ws_bytes = int(lib().gscan_backward_workspace_bytes(B, K, SH2, D, code))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, ws_bytes, dev)
    _check(lib().gscan_backward_ex(
        h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
        W_C.data_ptr(), B, K, SH2, D, d_context.data_ptr(), out[0].data_ptr(),
        out[1].data_ptr(), out[2].data_ptr(), code, float(a_shift), workspace.data_ptr(),
        workspace.numel(), _stream_handle(stream, dev)))
    return out


def backward_full_workspace_bytes(B: int, K: int, SH2: int, D: int, bf16: bool = False) -> int:
    return int(lib().gscan_backward_full_workspace_bytes(B, K, SH2, D,
                                                         GSCAN_BF16 if bf16 else GSCAN_F32))


def backward_full(h_history, h_s2, W_A, W_B, W_C, K: int, d_context, a_shift: float = 0.0,
                  out=None, workspace=None, stream=None):
    """(dW_A, dW_B, dW_C, d_h_history, d_h_s2) for L = sum(d_context * context):
    the weight gradients of `backward` and the input gradients, float32
    [SH2, D] x 3, [B*K, SH2] and [B, SH2].  `out` may hold those five tensors."""
    import torch
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(d_context, (B, D), dev, "d_context")
    if out is None:
        out = tuple(torch.empty((SH2, D), dtype=torch.float32, device=dev) for _ in range(3)) + (
            torch.empty((B * K, SH2), dtype=torch.float32, device=dev),
            torch.empty((B, SH2), dtype=torch.float32, device=dev))
    else:
        _check_outs(out, [(SH2, D)] * 3 + [(B * K, SH2), (B, SH2)], dev)
    ws_bytes = int(lib().gscan_backward_full_workspace_bytes(B, K, SH2, D, code))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, ws_bytes, dev)
    _check(lib().gscan_backward_full_ex(
        h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
        W_C.data_ptr(), B, K, SH2, D, d_context.data_ptr(), out[0].data_ptr(),
        out[1].data_ptr(), out[2].data_ptr(), out[3].data_ptr(), out[4].data_ptr(), code,
        float(a_shift), workspace.data_ptr(), workspace.numel(), _stream_handle(stream, dev)))
    return out


def prepare_backward_full(h_history, h_s2, W_A, W_B, W_C, K, d_context, out, workspace,
                          a_shift=0.0, stream=None):
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(d_context, (B, D), dev, "d_context")
    _check_outs(out, [(SH2, D)] * 3 + [(B * K, SH2), (B, SH2)], dev)
    _check_workspace(workspace, int(lib().gscan_backward_full_workspace_bytes(B, K, SH2, D, code)),
                     dev)
    args = (h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
            W_C.data_ptr(), B, K, SH2, D, d_context.data_ptr(), out[0].data_ptr(),
            out[1].data_ptr(), out[2].data_ptr(), out[3].data_ptr(), out[4].data_ptr(), code,
            ctypes.c_float(a_shift), workspace.data_ptr(), workspace.numel(),
            _stream_handle(stream, dev))
    return Prepared(lib().gscan_backward_full_ex, args,
                    (h_history, h_s2, W_A, W_B, W_C, d_context, out, workspace))


def bias_grad_reduce(grad, out=None, workspace=None, stream=None):
    """out[j] = sum_r grad[r, j] (float32 [cols]) for a contiguous float32
    [rows, cols] GPU tensor: the batch-parallel bias-gradient reduction."""
    import torch
    if (not grad.is_cuda or grad.dtype != torch.float32 or grad.dim() != 2
            or not grad.is_contiguous()):
        raise ValueError("grad must be a contiguous float32 [rows, cols] GPU tensor")
    rows, cols = grad.shape
    if out is None:
        out = torch.empty(cols, dtype=torch.float32, device=grad.device)
    else:
        _check_f32(out, (cols,), grad.device, "out")
    n = int(lib().gscan_bias_grad_reduce_workspace_bytes(rows, cols))
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=grad.device)
    else:
        _check_workspace(workspace, n, grad.device)
    _check(lib().gscan_bias_grad_reduce(grad.data_ptr() if rows else None, rows, cols,
                                        out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                        _stream_handle(stream, grad.device)))
    return out


def prepare_bias_grad_reduce(grad, out, workspace, stream=None):
    _check_f32(grad, tuple(grad.shape), grad.device, "grad")
    if grad.dim() != 2:
        raise ValueError("grad must be [rows, cols]")
    rows, cols = grad.shape
    _check_f32(out, (cols,), grad.device, "out")
    _check_workspace(workspace, int(lib().gscan_bias_grad_reduce_workspace_bytes(rows, cols)),
                     grad.device)
    args = (grad.data_ptr(), rows, cols, out.data_ptr(), workspace.data_ptr(), workspace.numel(),
            _stream_handle(stream, grad.device))
    return Prepared(lib().gscan_bias_grad_reduce, args, (grad, out, workspace))


def backward_partials(h_history, h_s2, W_A, W_B, W_C, K: int, d_context, workspace,
                      a_shift: float = 0.0, stream=None):
    """Phase 1 of the backward: per-workgroup weight-gradient partials into
    `workspace` (a uint8 device tensor of at least backward_workspace_bytes())."""
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(d_context, (B, D), dev, "d_context")
    _check_workspace(workspace, int(lib().gscan_backward_workspace_bytes(B, K, SH2, D, code)), dev)
    _check(lib().gscan_backward_partials(
        h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(), W_C.data_ptr(),
        B, K, SH2, D, d_context.data_ptr(), code, float(a_shift), workspace.data_ptr(),
        workspace.numel(), _stream_handle(stream, dev)))


def backward_reduce(workspace, B: int, K: int, SH2: int, D: int, out, bf16: bool = False,
                    stream=None):
    """Phase 2 of the backward: fixed-order sum of the partials into out = (dW_A, dW_B, dW_C)."""
    code = GSCAN_BF16 if bf16 else GSCAN_F32
    _check_workspace(workspace, int(lib().gscan_backward_workspace_bytes(B, K, SH2, D, code)),
                     workspace.device)
    _check_outs(out, [(SH2, D)] * 3, workspace.device)
    _check(lib().gscan_backward_reduce(
        workspace.data_ptr(), workspace.numel(), B, K, SH2, D,
        GSCAN_BF16 if bf16 else GSCAN_F32, out[0].data_ptr(), out[1].data_ptr(),
        out[2].data_ptr(), _stream_handle(stream, workspace.device)))


class Prepared:
    """A C-ABI call with its arguments marshalled once (for tight loops: one
    ctypes call per invocation, no per-call Python checks).  The tensors
    passed to prepare_* must stay alive while the object is used."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            _check(st)


def prepare_forward(h_history, h_s2, W_A, W_B, W_C, K, out, a_shift=0.0, stream=None):
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(out, (B, D), dev, "out")
    wp, wn, ws = _forward_workspace(None, B, K, SH2, D, code, dev)
    args = (h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
            W_C.data_ptr(), B, K, SH2, D, out.data_ptr(), code, ctypes.c_float(a_shift), wp, wn,
            _stream_handle(stream, dev))
    return Prepared(lib().gscan_forward_ex, args, (h_history, h_s2, W_A, W_B, W_C, out, ws))


def prepare_backward(h_history, h_s2, W_A, W_B, W_C, K, d_context, out, workspace,
                     a_shift=0.0, stream=None):
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(d_context, (B, D), dev, "d_context")
    _check_outs(out, [(SH2, D)] * 3, dev)
    _check_workspace(workspace, int(lib().gscan_backward_workspace_bytes(B, K, SH2, D, code)), dev)
    args = (h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
            W_C.data_ptr(), B, K, SH2, D, d_context.data_ptr(), out[0].data_ptr(),
            out[1].data_ptr(), out[2].data_ptr(), code, ctypes.c_float(a_shift),
            workspace.data_ptr(), workspace.numel(), _stream_handle(stream, dev))
    return Prepared(lib().gscan_backward_ex, args,
                    (h_history, h_s2, W_A, W_B, W_C, d_context, out, workspace))


def prepare_backward_partials(h_history, h_s2, W_A, W_B, W_C, K, d_context, workspace,
                              a_shift=0.0, stream=None):
    dev, code, B, K, SH2, D = _prep(h_history, h_s2, W_A, W_B, W_C, K)
    _check_f32(d_context, (B, D), dev, "d_context")
    _check_workspace(workspace, int(lib().gscan_backward_workspace_bytes(B, K, SH2, D, code)), dev)
    args = (h_history.data_ptr(), h_s2.data_ptr(), W_A.data_ptr(), W_B.data_ptr(),
            W_C.data_ptr(), B, K, SH2, D, d_context.data_ptr(), code, ctypes.c_float(a_shift),
            workspace.data_ptr(), workspace.numel(), _stream_handle(stream, dev))
    return Prepared(lib().gscan_backward_partials, args,
                    (h_history, h_s2, W_A, W_B, W_C, d_context, workspace))


def prepare_backward_reduce(workspace, B, K, SH2, D, out, bf16=False, stream=None):
    code = GSCAN_BF16 if bf16 else GSCAN_F32
    _check_workspace(workspace, int(lib().gscan_backward_workspace_bytes(B, K, SH2, D, code)),
                     workspace.device)
    _check_outs(out, [(SH2, D)] * 3, workspace.device)
    args = (workspace.data_ptr(), workspace.numel(), B, K, SH2, D,
            GSCAN_BF16 if bf16 else GSCAN_F32, out[0].data_ptr(), out[1].data_ptr(),
            out[2].data_ptr(), _stream_handle(stream, workspace.device))
    return Prepared(lib().gscan_backward_reduce, args, (workspace, out))
