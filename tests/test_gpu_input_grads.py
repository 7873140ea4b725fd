"""Parity of the input gradients (gscan_backward_full_ex, through the C ABI)
with the CPU oracle.

d_h_history [B*K, SH2] and d_h_s2 [B, SH2] are held element-wise to
|gpu - ref| <= tol*(1 + |ref|), tol = 1e-4 for fp32 inputs and 2e-2 for bf16:
the method states no tolerance for these outputs, and they are per-element
results like the context, from the same split-bf16 products with fp32
accumulation (over 2D, resp. D, terms after a backward whose dL/dA, dL/dB
and dL/dC already meet the context's bound).  The weight gradients returned
alongside must be bitwise those of gscan_backward_ex.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_history_amd as gs
import oracle
from gated_linear_recurrence_history_amd import synth, workloads as wl

pytestmark = pytest.mark.gpu

from tests.gpu_util import ctx_err, device_inputs, gpu_backward, gpu_forward, workload  # noqa: E402

SHAPES = [
    # B, K, SH2, D, dtype, a_shift
    (64, 8, 256, 16, "f32", 0.0),     # the tiny workload's shape
    (37, 5, 192, 32, "f32", 0.5),     # K not dividing 16 (general backward kernel)
    (1, 1, 64, 16, "f32", 0.0),       # one sample, one step
    (20, 24, 256, 16, "f32", 0.0),    # samples straddle 64-row chunks
    (33, 8, 512, 16, "f32", 0.0),     # widest SH2
    (50, 8, 256, 16, "bf16", 0.0),
    (17, 64, 256, 64, "f32", 2.0),
    (3, 2, 448, 256, "f32", 0.25),    # widest D: 16 k-chunks of 32
    (37, 16, 256, 48, "f32", 1.0),    # three state slices
    (45, 2, 192, 16, "bf16", 0.5),
    (70, 2, 256, 16, "f32", 0.0),
    (21, 32, 128, 32, "f32", -1.0),   # samples of 2 blocks (per-block kernel)
    (9, 64, 64, 16, "bf16", 0.5),     # samples of 4 blocks
    # D = 16 with the per-block kernel: the input gradients come out of the
    # backward pass itself (ragged groups, every SH2 it takes, K folded in or not)
    (37, 16, 256, 16, "f32", 1.0),
    (13, 32, 128, 16, "f32", -2.0),
    (29, 4, 128, 16, "f32", -1.0),
    (1000, 8, 192, 16, "bf16", 0.25),
    (19, 8, 64, 16, "f32", 3.0),
    (8, 64, 512, 64, "f32", 1.0),     # split backward: adjoints straight from the scan pass
    (2, 256, 512, 128, "bf16", -0.5),
    (37, 5, 96, 32, "f32", 0.5),      # materialised-projection path: SH2 % 64 != 0
    (6, 9, 1024, 64, "bf16", -1.0),   # and SH2 above 512
    (300, 4, 16, 16, "f32", 2.0),
]


def _nan_outs(t, K):
    """NaN-filled output tensors, so an element a call leaves unwritten fails
    the comparison."""
    SH2, D = t["W_A"].shape
    B = t["h_s2"].shape[0]
    dev = t["W_A"].device
    return tuple(torch.full(sh, float("nan"), dtype=torch.float32, device=dev)
                 for sh in [(SH2, D)] * 3 + [(B * K, SH2), (B, SH2)])


def _full(t, K, a, d=None):
    d = t["d_context"] if d is None else d
    out = _nan_outs(t, K)
    gs.backward_full(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], K, d, a, out=out)
    torch.cuda.synchronize()
    return tuple(o.cpu().numpy() for o in out)


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B%d_K%d_S%d_D%d_%s_a%g" % c)
def test_input_grad_parity(case):
    B, K, SH2, D, dt, a = case
    w = workload(B, K, SH2, D, dt, a)
    print(f"case input grads {w.name} a_shift={a}", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    got = _full(t, K, a)
    ref_dh, ref_dhs = oracle.backward_inputs(x["h_history"], x["h_s2"], x["W_A"], x["W_B"],
                                             x["W_C"], K, x["d_context"], a)
    tol = 2e-2 if dt == "bf16" else 1e-4
    e1, e2 = ctx_err(got[3], ref_dh), ctx_err(got[4], ref_dhs)
    print(f"  d_h_history {e1:.2e} d_h_s2 {e2:.2e}", flush=True)
    assert e1 <= tol and e2 <= tol
    if dt == "bf16":  # exact widening: the fp32 bar against the same rounded inputs
        assert e1 <= 1e-4 and e2 <= 1e-4
    for g, r in zip(got[:3], gpu_backward(t, K, a)):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS + wl.OUT_OF_ENVELOPE])
def test_input_grad_full_size(name):
    """Each named workload, and the headline shape at the two out-of-envelope
    widths, at full size in the benchmark's launch
    configuration: every element of d_h_history and d_h_s2 against the
    oracle, except for the wide workload (2^21 rows of 512: hours of host
    time for the fp64 oracle), where the rows of 64 sampled samples are
    compared (a sample's input gradients depend on that sample alone); and
    <h_s2, dL/dh_s2> = L over the whole batch (L is linear in h_s2)."""
    w = next(c for c in wl.WORKLOADS + wl.OUT_OF_ENVELOPE if c.name == name)
    tol = wl.tolerance(w)
    print(f"case input grads full {w.name} B={w.B} K={w.K} SH2={w.SH2} D={w.D}", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    out = _nan_outs(t, w.K)
    gs.backward_full(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K,
                     t["d_context"], w.a_shift, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out[3]).all()) and bool(torch.isfinite(out[4]).all())
    got_dhs = out[4].cpu().numpy()
    if w.name != "wide_fp32":
        got_dh = out[3].cpu().numpy()
        ref_dh, ref_dhs = oracle.backward_inputs(x["h_history"], x["h_s2"], x["W_A"], x["W_B"],
                                                 x["W_C"], w.K, x["d_context"], w.a_shift)
        e1, e2 = ctx_err(got_dh, ref_dh), ctx_err(got_dhs, ref_dhs)
        del got_dh, ref_dh
        print(f"  d_h_history {e1:.2e} d_h_s2 {e2:.2e} (all rows)", flush=True)
    else:
        rng = np.random.default_rng(4242)
        n_s = 64
        samples = np.sort(np.concatenate([[0, w.B - 1],
                                          rng.choice(np.arange(1, w.B - 1), n_s - 2,
                                                     replace=False)]))
        rows = (samples[:, None] * w.K + np.arange(w.K)[None, :]).reshape(-1)
        got_dh = out[3][torch.from_numpy(rows).to(out[3].device)].cpu().numpy()
        sub = oracle.sample_rows(x, w.K, samples)
        ref_dh, ref_dhs = oracle.backward_inputs(sub["h_history"], sub["h_s2"], sub["W_A"],
                                                 sub["W_B"], sub["W_C"], w.K, sub["d_context"],
                                                 w.a_shift)
        e1, e2 = ctx_err(got_dh, ref_dh), ctx_err(got_dhs[samples], ref_dhs)
        print(f"  sampled d_h_history {e1:.2e} d_h_s2 {e2:.2e} over {len(samples)} samples",
              flush=True)
    assert e1 <= min(tol, 1e-4) and e2 <= min(tol, 1e-4)
    del out
    ctx = gpu_forward(t, w.K, w.a_shift).astype(np.float64)
    L = float(np.sum(x["d_context"].astype(np.float64) * ctx))
    prod = oracle.widen(x["h_s2"]) * got_dhs.astype(np.float64)
    assert abs(prod.sum() - L) <= 1e-4 * np.abs(prod).sum()
