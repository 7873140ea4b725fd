"""GPU behaviour beyond parity: bitwise reproducibility, isolation of
non-finite values between samples, stream and workspace variants, and error
reporting through the binding."""
import ctypes

import numpy as np
import pytest
import torch

import gated_linear_recurrence_history_amd as gs
from gated_linear_recurrence_history_amd import binding, synth, workloads as wl

pytestmark = pytest.mark.gpu

from tests.gpu_util import DEV, device_inputs, gpu_backward, gpu_forward, workload  # noqa: E402


def test_bitwise_reproducible():
    w = wl.HEADLINE
    print(f"case reproducible {w.name}", flush=True)
    t = device_inputs(synth.make_inputs(w))
    c1 = gpu_forward(t, w.K, 0.0)
    c2 = gpu_forward(t, w.K, 0.0)
    assert np.array_equal(c1, c2)
    g1 = gpu_backward(t, w.K, 0.0)
    g2 = gpu_backward(t, w.K, 0.0)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("K,SH2", [(8, 128), (5, 128), (70, 128), (8, 80), (6, 1008)])
def test_non_finite_stays_in_its_sample(K, SH2):
    w = workload(40, K, SH2, 32, seed=5)
    print(f"case nonfinite K={K} SH2={SH2}", flush=True)
    x = synth.make_inputs(w)
    clean = gpu_forward(device_inputs(x), K, 0.0)
    y = {k: v.copy() for k, v in x.items()}
    y["h_history"][5 * K + K // 2, 3] = np.nan        # sample 5
    y["h_history"][17 * K, 0] = np.inf                # sample 17, first step
    y["h_s2"][30, 7] = -np.inf                        # sample 30
    dirty = gpu_forward(device_inputs(y), K, 0.0)
    bad = {5, 17, 30}
    for b in range(w.B):
        if b in bad:
            assert not np.all(np.isfinite(dirty[b])), b
        else:
            assert np.array_equal(dirty[b], clean[b]), b
    dW = gpu_backward(device_inputs(y), K, 0.0)
    assert all(not np.all(np.isfinite(g)) for g in dW[:2])


def test_plain_entry_points_and_streams():
    w = workload(300, 8, 256, 32, seed=9)
    print("case plain/ex/stream", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    ref_ctx = gpu_forward(t, w.K, 0.0)
    ref_dW = gpu_backward(t, w.K, 0.0)
    L = binding.lib()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ctx = torch.full((w.B, w.D), 7.0, device=DEV)
        dW = [torch.full((w.SH2, w.D), 7.0, device=DEV) for _ in range(3)]
        h = ctypes.c_void_p(s.cuda_stream)
        assert L.gscan_forward(t["h_history"].data_ptr(), t["h_s2"].data_ptr(),
                               t["W_A"].data_ptr(), t["W_B"].data_ptr(), t["W_C"].data_ptr(),
                               w.B, w.K, w.SH2, w.D, ctx.data_ptr(), h) == 0
        assert L.gscan_backward(t["h_history"].data_ptr(), t["h_s2"].data_ptr(),
                                t["W_A"].data_ptr(), t["W_B"].data_ptr(), t["W_C"].data_ptr(),
                                w.B, w.K, w.SH2, w.D, t["d_context"].data_ptr(),
                                dW[0].data_ptr(), dW[1].data_ptr(), dW[2].data_ptr(), h) == 0
    s.synchronize()
    assert np.array_equal(ctx.cpu().numpy(), ref_ctx)
    for a, b in zip(dW, ref_dW):
        assert np.array_equal(a.cpu().numpy(), b)


def test_errors_leave_outputs_untouched():
    w = workload(32, 8, 256, 16, seed=3)
    t = device_inputs(synth.make_inputs(w))
    out = torch.full((w.B, w.D), 3.0, device=DEV)
    bad_W = torch.zeros((w.SH2, 24), device=DEV)  # D = 24 is not a multiple of 16
    bad_h = torch.zeros((w.B * w.K, 24), device=DEV)
    with pytest.raises(gs.GScanError) as ei:
        L = binding.lib()
        st = L.gscan_forward_ex(t["h_history"].data_ptr(), t["h_s2"].data_ptr(),
                                bad_W.data_ptr(), bad_W.data_ptr(), bad_W.data_ptr(), w.B, w.K,
                                w.SH2, 24, out.data_ptr(), 0, 0.0, None, 0, None)
        binding._check(st)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    with pytest.raises(ValueError):
        gs.forward(bad_h, t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K)


def test_graph_replays():
    """Forward and backward captured once in a HIP graph and replayed with
    new inputs copied in between (eager work and synchronisation between
    replays): every replay equals an eager call on its inputs."""
    w = workload(2048, 8, 256, 16, seed=21)
    print("case graph replays", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    h = t["h_history"].clone()
    d = t["d_context"].clone()
    n = binding.backward_workspace_bytes(w.B, w.K, w.SH2, w.D)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    ctx = torch.empty((w.B, w.D), device=DEV)
    out = tuple(torch.empty((w.SH2, w.D), device=DEV) for _ in range(3))

    def step():
        gs.forward(h, t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K, 0.0, out=ctx)
        gs.backward(h, t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K, d, 0.0, out=out,
                    workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        h.copy_(t["h_history"] * (1.0 - 0.25 * i))
        d.copy_(t["d_context"] * (1.0 + 0.5 * i) - 0.25 * i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_ctx = ctx.cpu().numpy()
        got = tuple(o.cpu().numpy() for o in out)
        ref_ctx = gpu_forward({**t, "h_history": h}, w.K, 0.0)
        ref = gpu_backward({**t, "h_history": h}, w.K, 0.0, d_context=d)
        assert np.array_equal(got_ctx, ref_ctx), i
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), i


def test_graph_replays_input_grads_and_bias_grad():
    """gscan_backward_full_ex and gscan_bias_grad_reduce captured in one HIP
    graph (caller workspaces, the general backward kernel's shape so the
    adjoint kernel is in it too) and replayed with new inputs in between:
    every replay equals eager calls on its inputs."""
    w = workload(300, 5, 192, 32, seed=23)  # K = 5: the general kernel + adjoint pass
    print("case graph replays (input grads, bias grad)", flush=True)
    t = device_inputs(synth.make_inputs(w))
    h = t["h_history"].clone()
    d = t["d_context"].clone()
    g = torch.empty((4099, 24), device=DEV)
    nf = binding.backward_full_workspace_bytes(w.B, w.K, w.SH2, w.D)
    wsf = torch.empty(nf, dtype=torch.uint8, device=DEV)
    nb = binding.lib().gscan_bias_grad_reduce_workspace_bytes(4099, 24)
    wsb = torch.empty(nb, dtype=torch.uint8, device=DEV)
    out = (tuple(torch.empty((w.SH2, w.D), device=DEV) for _ in range(3))
           + (torch.empty((w.B * w.K, w.SH2), device=DEV), torch.empty((w.B, w.SH2), device=DEV)))
    gsum = torch.empty(24, device=DEV)

    def step():
        gs.backward_full(h, t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K, d, 0.25, out=out,
                         workspace=wsf)
        gs.bias_grad_reduce(g, out=gsum, workspace=wsb)

    g.normal_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        h.copy_(t["h_history"] * (1.0 + 0.5 * i))
        d.copy_(t["d_context"] * (0.5 - 0.25 * i))
        g.copy_(torch.randn((4099, 24), device=DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy() for o in out] + [gsum.cpu().numpy()]
        ref = gs.backward_full(h, t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K, d, 0.25)
        refg = gs.bias_grad_reduce(g)
        torch.cuda.synchronize()
        for a, b in zip(got, [r.cpu().numpy() for r in ref] + [refg.cpu().numpy()]):
            assert np.array_equal(a, b), i


def test_forward_caller_workspace():
    """A shape outside the fused kernels: the forward with a caller's
    workspace gives bitwise the result of the call's own stream-ordered
    allocation, for the plain and the enrich entry points; a workspace that
    is too small is refused before anything runs."""
    w = workload(333, 6, 208, 32, seed=13)
    print("case forward workspace", flush=True)
    t = device_inputs(synth.make_inputs(w))
    L = binding.lib()
    need = L.gscan_forward_workspace_bytes(w.B, w.K, w.SH2, w.D, 0)
    assert need >= 4 * (w.B * w.K * 2 * w.D + w.B * w.D)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    ins = [t[k].data_ptr() for k in ("h_history", "h_s2", "W_A", "W_B", "W_C")]
    own = torch.full((w.B, w.D), 7.0, device=DEV)
    mine = torch.full((w.B, w.D), 7.0, device=DEV)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    assert L.gscan_forward_ex(*ins, w.B, w.K, w.SH2, w.D, own.data_ptr(), 0, 0.0, None, 0,
                              stream) == 0
    assert L.gscan_forward_ex(*ins, w.B, w.K, w.SH2, w.D, mine.data_ptr(), 0, 0.0,
                              ws.data_ptr(), need, stream) == 0
    small = torch.full((w.B, w.D), 7.0, device=DEV)
    assert L.gscan_forward_ex(*ins, w.B, w.K, w.SH2, w.D, small.data_ptr(), 0, 0.0,
                              ws.data_ptr(), need - 4, stream) == 4
    torch.cuda.synchronize()
    assert torch.equal(own, mine)
    assert torch.all(small == 7.0)
    he1 = torch.zeros((w.B, 50), device=DEV)
    he2 = torch.zeros((w.B, 50), device=DEV)
    gs.forward_enrich(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K, he1,
                      col_offset=3)
    assert L.gscan_forward_enrich(*ins, w.B, w.K, w.SH2, w.D, None, he2.data_ptr(), 50, 3, 0, 0.0,
                                  ws.data_ptr(), need, stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(he1, he2)
    assert torch.equal(he1[:, 3:3 + w.D], own)
