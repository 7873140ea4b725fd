"""gscan_backward_noalloc (the backward whose partials live in the library's
static scratch array, for callers that cannot allocate) against
gscan_backward_ex, through the C ABI: two calls in a row, the second on a
smaller input, each bitwise equal to the workspace entry point's result
(same kernels, same order) and within the oracle's weight-gradient bar."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_linear_recurrence_history_amd import binding, synth

pytestmark = pytest.mark.gpu

from tests.gpu_util import DEV, device_inputs, rel_l2, workload  # noqa: E402

CASES = [
    (8192, 8, 256, 16, "f32", 0.0),    # the headline shape (12 MiB of partials)
    (777, 5, 192, 32, "f32", 0.5),     # smaller, general backward kernel
    (301, 4, 80, 16, "f32", -1.0),     # materialised-projection path
]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(L, t, B, K, SH2, D, code, a, out, stream):
    return L.gscan_backward_noalloc(
        _ptr(t["h_history"]), _ptr(t["h_s2"]), _ptr(t["W_A"]), _ptr(t["W_B"]), _ptr(t["W_C"]),
        B, K, SH2, D, _ptr(t["d_context"]), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), code,
        ctypes.c_float(a), stream)


def _with_workspace(L, t, B, K, SH2, D, code, a, out, stream):
    ws = torch.empty(L.gscan_backward_workspace_bytes(B, K, SH2, D, code), dtype=torch.uint8,
                     device=DEV)
    st = L.gscan_backward_ex(
        _ptr(t["h_history"]), _ptr(t["h_s2"]), _ptr(t["W_A"]), _ptr(t["W_B"]), _ptr(t["W_C"]),
        B, K, SH2, D, _ptr(t["d_context"]), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), code,
        ctypes.c_float(a), _ptr(ws), ws.numel(), stream)
    torch.cuda.synchronize()
    return st


def test_noalloc_matches_workspace_entry_twice():
    L = binding.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    for B, K, SH2, D, dt, a in CASES:  # second call: a smaller input
        print(f"case noalloc B={B} K={K} SH2={SH2} D={D} {dt} a={a}", flush=True)
        code = binding.GSCAN_BF16 if dt == "bf16" else binding.GSCAN_F32
        assert L.gscan_backward_workspace_bytes(B, K, SH2, D, code) <= (16 << 20)
        w = workload(B, K, SH2, D, dt, a, seed=41)
        x = synth.make_inputs(w)
        t = device_inputs(x)
        got = tuple(torch.full((SH2, D), float("nan"), device=DEV) for _ in range(3))
        st = _noalloc(L, t, B, K, SH2, D, code, a, got, stream)
        assert st == 0, L.gscan_last_error()
        torch.cuda.synchronize()
        ref = tuple(torch.empty((SH2, D), device=DEV) for _ in range(3))
        assert _with_workspace(L, t, B, K, SH2, D, code, a, ref, stream) == 0
        g = [o.cpu().numpy() for o in got]
        r = [o.cpu().numpy() for o in ref]
        for p, q in zip(g, r):
            assert np.array_equal(p, q)
        ref_dW = oracle.backward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K,
                                 x["d_context"], a)
        ge = [rel_l2(p, q) for p, q in zip(g, ref_dW)]
        print(f"  dW rel-L2 vs oracle {['%.2e' % e for e in ge]}", flush=True)
        assert max(ge) <= 1e-4
