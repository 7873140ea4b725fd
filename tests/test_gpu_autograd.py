"""gated_scan (the autograd Function over the C ABI): the context and every
gradient torch's autograd produces are bitwise the direct calls' results,
and match the oracle; inputs that need no gradient get none; bfloat16
inputs receive their gradients in bfloat16."""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_history_amd as gs
import oracle
from gated_linear_recurrence_history_amd import synth

pytestmark = pytest.mark.gpu

from tests.gpu_util import ctx_err, device_inputs, rel_l2, workload  # noqa: E402


@pytest.mark.parametrize("case", [(300, 8, 256, 16, "f32", 0.5), (37, 5, 96, 32, "f32", -1.0),
                                  (50, 16, 128, 32, "bf16", 1.0)],
                         ids=lambda c: "B%d_K%d_S%d_D%d_%s_a%g" % c)
def test_autograd_matches_direct_calls_and_oracle(case):
    B, K, SH2, D, dt, a = case
    print(f"case autograd B={B} K={K} SH2={SH2} D={D} {dt}", flush=True)
    w = workload(B, K, SH2, D, dt, a, seed=71)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    leaves = [t[k].clone().requires_grad_(t[k].dtype == torch.float32 or k.startswith("h"))
              for k in ("h_history", "h_s2", "W_A", "W_B", "W_C")]
    ctx = gs.gated_scan(*leaves, K, a)
    (ctx * t["d_context"]).sum().backward()
    torch.cuda.synchronize()
    direct = gs.backward_full(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], K,
                              t["d_context"], a)
    torch.cuda.synchronize()
    assert torch.equal(ctx.detach(), gs.forward(t["h_history"], t["h_s2"], t["W_A"], t["W_B"],
                                                t["W_C"], K, a))
    for leaf, ref in zip(leaves[2:], direct[:3]):
        assert torch.equal(leaf.grad, ref)
    for leaf, ref in zip(leaves[:2], direct[3:]):
        assert leaf.grad.dtype == leaf.dtype
        assert torch.equal(leaf.grad, ref.to(leaf.dtype))
    args = (x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K)
    ref_dW = oracle.backward(*args, x["d_context"], a)
    assert ctx_err(ctx.detach().cpu().numpy(), oracle.forward(*args, a)) <= 1e-4
    assert max(rel_l2(l.grad.cpu().numpy(), r) for l, r in zip(leaves[2:], ref_dW)) <= 1e-4


def test_autograd_weights_only():
    """With constant inputs only the weight gradients are formed (the
    backward without input gradients), equal to the direct backward."""
    w = workload(64, 8, 256, 16, seed=72)
    t = device_inputs(synth.make_inputs(w))
    Ws = [t[k].clone().requires_grad_(True) for k in ("W_A", "W_B", "W_C")]
    ctx = gs.gated_scan(t["h_history"], t["h_s2"], *Ws, w.K, 0.0)
    (ctx * t["d_context"]).sum().backward()
    ref = gs.backward(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K,
                      t["d_context"], 0.0)
    torch.cuda.synchronize()
    for W, r in zip(Ws, ref):
        assert torch.equal(W.grad, r)
    assert t["h_history"].grad is None
