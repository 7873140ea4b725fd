"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Small and ragged shapes compare every output element; the five named
workloads run at full size in the same launch configuration the benchmark
times, checked element-wise where the oracle can afford it and otherwise on
sampled outputs (forward: a spread of samples; backward: an upstream
gradient supported on sampled samples, whose exact weight gradients are the
oracle's on those samples alone) plus properties that hold at any size.

Tolerances (from the method's stated targets): context max |err| <=
tol*(1+|ref|), each dW relative L2 <= tol, tol = 1e-4 (fp32 inputs) or
2e-2 (bf16 inputs).  The HIP path widens bf16 exactly and accumulates in
fp32, so bf16 cases are additionally held to 1e-4 against the oracle that
uses the same rounded values.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_recurrence_history_amd import synth, workloads as wl

pytestmark = pytest.mark.gpu

from tests.gpu_util import (ctx_err, device_inputs, gpu_backward, gpu_forward, rel_l2,  # noqa: E402
                            to_dev, workload)

SMALL = [
    # B, K, SH2, D, dtype, a_shift
    (64, 8, 256, 16, "f32", 0.0),     # the tiny workload's shape
    (37, 5, 192, 32, "f32", 0.5),     # ragged last group, K not dividing 16
    (1, 1, 64, 16, "f32", 0.0),       # one sample, one step
    (16, 1, 64, 16, "f32", -2.0),
    (19, 3, 128, 48, "f32", 1.0),
    (20, 24, 256, 16, "f32", 0.0),    # samples straddle 64-row chunks
    (9, 70, 64, 16, "f32", -0.5),     # a sample open at both ends of a chunk
    (5, 130, 128, 32, "f32", 2.0),
    (33, 8, 512, 16, "f32", 0.0),     # widest SH2
    (50, 8, 256, 16, "bf16", 0.0),
    (17, 64, 256, 64, "f32", 2.0),    # long-scan shape, small batch
    (4, 256, 512, 128, "f32", 0.0),   # wide shape, small batch
    (23, 7, 320, 80, "bf16", -1.0),
    (3, 2, 448, 256, "f32", 0.25),    # widest D
    # K dividing 16 with SH2 <= 256 (the backward's per-block kernel): a
    # sample spans 4, 2 or 1 lane groups, or a lane holds several samples
    (37, 16, 256, 16, "f32", 1.0),
    (29, 4, 128, 32, "f32", -1.0),
    (45, 2, 192, 16, "bf16", 0.5),
    (13, 16, 64, 48, "f32", 2.0),
    (70, 2, 256, 16, "f32", 0.0),
    # more than 512 groups of 16 samples: the forward walks several groups
    # per workgroup (ragged last group, two state slices)
    (9000, 2, 64, 16, "f32", 0.5),
    (8300, 4, 128, 32, "bf16", -1.0),
    # D > 16: several state slices per forward workgroup of two groups
    # (a missing second group, bf16 rows, samples straddling blocks, more
    # groups than grid slots in one pass)
    (40, 16, 256, 64, "bf16", 0.5),
    (33, 20, 384, 32, "f32", -0.5),
    (9000, 16, 64, 32, "f32", 1.0),
    # K = 32 or 64 with SH2 <= 256 (the per-block backward kernel): a sample
    # fills 2 or 4 blocks of a chunk
    (21, 32, 128, 16, "f32", 0.0),
    (9, 64, 64, 32, "bf16", -0.5),
    (13, 32, 256, 48, "f32", 2.0),
    (6, 64, 192, 16, "f32", 1.0),
    (35, 32, 256, 16, "f32", -3.0),
    # K = 8 and 64 run the per-block backward compiled for that K: every
    # SH2 it takes, ragged batches, several state slices, both input types
    (27, 8, 128, 32, "f32", -1.0),
    (45, 8, 64, 16, "f32", 0.5),
    (29, 8, 192, 48, "bf16", 2.0),
    (19, 64, 128, 16, "f32", 0.0),
]


def _check(x, w, ctx, dW, ref_ctx, ref_dW, tol=1e-4):
    ce = ctx_err(ctx, ref_ctx)
    ge = [rel_l2(g, r) for g, r in zip(dW, ref_dW)]
    print(f"  {w.name}: ctx {ce:.2e} dW {['%.2e' % e for e in ge]}", flush=True)
    assert ce <= tol
    assert max(ge) <= tol


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%d_K%d_S%d_D%d_%s_a%g" % c)
def test_parity_small(case):
    B, K, SH2, D, dt, a = case
    w = workload(B, K, SH2, D, dt, a)
    print(f"case {w.name} a_shift={a}", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    ctx = gpu_forward(t, K, a)
    dW = gpu_backward(t, K, a)
    ref_ctx = oracle.forward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K, a)
    ref_dW = oracle.backward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K,
                             x["d_context"], a)
    _check(x, w, ctx, dW, ref_ctx, ref_dW)


def _spread(n_total, n, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n_total, size=n - 2, replace=False).tolist())
    s.update({0, n_total - 1})
    return np.array(sorted(s), dtype=np.int64)


def _euler(x, dWB, dWC, ctx, tol):
    """L = sum d*ctx equals <W_B, dW_B> and <W_C, dW_C> (1-homogeneity), to the
    slack the parity tolerances allow."""
    d = x["d_context"].astype(np.float64)
    L = float(np.sum(d * ctx))
    slackL = tol * float(np.sum(np.abs(d) * (1.0 + np.abs(ctx))))
    for W, dW in ((x["W_B"], dWB), (x["W_C"], dWC)):
        ip = float(np.sum(W.astype(np.float64) * dW))
        slack = tol * float(np.linalg.norm(W) * np.linalg.norm(dW)) + slackL
        assert abs(ip - L) <= slack, (ip, L, slack)


@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS])
def test_parity_full_size(name):
    w = wl.BY_NAME[name]
    tol = wl.tolerance(w)
    print(f"case full {w.name} B={w.B} K={w.K} SH2={w.SH2} D={w.D} {w.in_dtype}", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    ctx = gpu_forward(t, w.K, w.a_shift)
    dW = gpu_backward(t, w.K, w.a_shift)
    assert np.all(np.isfinite(ctx)) and all(np.all(np.isfinite(g)) for g in dW)
    if w.B * w.K * w.SH2 <= 8192 * 8 * 256:
        # the oracle takes the whole workload
        ref_ctx = oracle.forward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], w.K,
                                 w.a_shift)
        ref_dW = oracle.backward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], w.K,
                                 x["d_context"], w.a_shift)
        _check(x, w, ctx, dW, ref_ctx, ref_dW, tol=min(tol, 1e-4))
    else:
        # forward on a spread of samples
        n_s = {"longK_fp32": 96, "bigbatch_bf16": 512, "wide_fp32": 24}.get(w.name, 64)
        sidx = _spread(w.B, n_s, 11)
        xs = oracle.sample_rows(x, w.K, sidx)
        ref_ctx = oracle.forward(xs["h_history"], xs["h_s2"], xs["W_A"], xs["W_B"], xs["W_C"],
                                 w.K, w.a_shift)
        ce = ctx_err(ctx[sidx], ref_ctx)
        print(f"  sampled ctx err {ce:.2e} over {len(sidx)} samples", flush=True)
        assert ce <= min(tol, 1e-4)
        # backward with the upstream gradient on sampled samples only
        bidx = _spread(w.B, max(8, n_s // 2), 12)
        dmask = np.zeros_like(x["d_context"])
        dmask[bidx] = x["d_context"][bidx]
        dWm = gpu_backward(t, w.K, w.a_shift, to_dev(dmask))
        xb = oracle.sample_rows(x, w.K, bidx)
        ref_dW = oracle.backward(xb["h_history"], xb["h_s2"], xb["W_A"], xb["W_B"], xb["W_C"],
                                 w.K, xb["d_context"], w.a_shift)
        ge = [rel_l2(g, r) for g, r in zip(dWm, ref_dW)]
        print(f"  sampled dW err {['%.2e' % e for e in ge]} over {len(bidx)} samples", flush=True)
        assert max(ge) <= min(tol, 1e-4)
    # properties on the dense run
    _euler(x, dW[1], dW[2], ctx.astype(np.float64), tol)


def test_linearity_in_upstream_gradient_full_size():
    w = wl.HEADLINE
    print(f"case linearity {w.name}", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    d1 = x["d_context"]
    d2 = synth.normal_f32(99, 5, d1.shape)
    g1 = gpu_backward(t, w.K, 0.0, to_dev(d1))
    g2 = gpu_backward(t, w.K, 0.0, to_dev(d2))
    g12 = gpu_backward(t, w.K, 0.0, to_dev((d1 + d2).astype(np.float32)))
    for a, b, c in zip(g1, g2, g12):
        assert rel_l2(c, a.astype(np.float64) + b) <= 1e-5
