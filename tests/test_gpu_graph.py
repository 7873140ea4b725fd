"""The library's calls under HIP graph capture: a training step (forward and
the two-phase backward with a caller workspace, and the allocation-free
backward) captured once through torch's graph API and replayed with new
input values copied into the captured buffers, eager work and
synchronisations between the replays; every replay is compared bitwise
with the same calls made eagerly on the same inputs.  Nothing in these
calls allocates or clears memory from the host, so the captured graph
holds kernel nodes only (SH2 = 208 runs the materialised-projection path,
whose forward also takes a caller workspace here)."""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_history_amd as gs
from gated_linear_recurrence_history_amd import binding, synth

pytestmark = pytest.mark.gpu

from tests.gpu_util import DEV, device_inputs, workload  # noqa: E402


@pytest.mark.parametrize("shape", [(512, 8, 256, 16), (300, 5, 192, 32), (300, 5, 208, 32)],
                         ids=lambda s: "B%d_K%d_S%d_D%d" % s)
def test_graph_replay_matches_eager(shape):
    B, K, SH2, D = shape
    print(f"case graph B={B} K={K} SH2={SH2} D={D}", flush=True)
    w = workload(B, K, SH2, D, seed=61)
    t = device_inputs(synth.make_inputs(w))
    ctx = torch.empty((B, D), device=DEV)
    dW = tuple(torch.empty((SH2, D), device=DEV) for _ in range(3))
    dW_na = tuple(torch.empty((SH2, D), device=DEV) for _ in range(3))
    ws = torch.empty(gs.backward_workspace_bytes(B, K, SH2, D), dtype=torch.uint8, device=DEV)
    nf = gs.forward_workspace_bytes(B, K, SH2, D)
    wsf = torch.empty(nf, dtype=torch.uint8, device=DEV) if nf else None
    args = (t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], K)
    L = binding.lib()

    def step():
        gs.forward(*args, 0.5, out=ctx, workspace=wsf)
        gs.backward(*args, t["d_context"], 0.5, out=dW, workspace=ws)
        stream = torch.cuda.current_stream(DEV).cuda_stream
        ptr = [a.data_ptr() for a in args[:5]]
        st = L.gscan_backward_noalloc(*ptr, B, K, SH2, D, t["d_context"].data_ptr(),
                                      dW_na[0].data_ptr(), dW_na[1].data_ptr(),
                                      dW_na[2].data_ptr(), 0, 0.5, stream)
        assert st == 0, L.gscan_last_error()

    # warm up on a side stream (as torch's graph API asks), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    for rep in range(4):
        # new inputs in the captured buffers, then eager work on other memory
        for k in ("h_history", "h_s2", "d_context"):
            t[k].copy_(torch.from_numpy(
                rng.standard_normal(tuple(t[k].shape)).astype(np.float32)).to(DEV))
        scratch = torch.randn(1 << 20, device=DEV)
        scratch.mul_(2.0).add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [ctx.cpu().numpy()] + [o.cpu().numpy() for o in dW + dW_na]
        step()  # the same calls, eagerly
        torch.cuda.synchronize()
        ref = [ctx.cpu().numpy()] + [o.cpu().numpy() for o in dW + dW_na]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {rep}"
        assert np.all(np.isfinite(got[0]))
