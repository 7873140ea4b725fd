"""The forward with the context folded into h_enriched (gscan_forward_enrich,
through the C ABI) against the oracle: the D columns at the offset gain the
context (|err| <= tol * (1 + |ref|), the context's bar), every other column
is bitwise unchanged, and a context output written alongside is bitwise the
plain forward's."""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_history_amd as gs
import oracle
from gated_linear_recurrence_history_amd import synth, workloads as wl

pytestmark = pytest.mark.gpu

from tests.gpu_util import DEV, ctx_err, device_inputs, gpu_forward, workload  # noqa: E402

CASES = [
    # B, K, SH2, D, dtype, a_shift, ld, col_offset, with context_out
    (8192, 8, 256, 16, "f32", 0.0, 256, 0, False),     # the headline, h_enriched of width SH2
    (8192, 8, 256, 16, "f32", 0.0, 256, 240, True),    # last D columns
    (37, 5, 192, 32, "f32", 0.5, 50, 7, True),         # odd pitch and offset
    (50, 8, 256, 16, "bf16", -1.0, 16, 0, False),      # h_enriched exactly [B, D]
    (17, 64, 256, 64, "f32", 2.0, 300, 100, False),    # several state slices per workgroup
    (9000, 2, 64, 16, "f32", 0.5, 33, 17, True),       # persistent forward over many groups
    (8, 256, 512, 128, "f32", -0.5, 640, 512, True),   # the forward over 256-row tiles
    (12, 64, 512, 64, "bf16", 1.0, 70, 3, False),
    (41, 6, 112, 32, "f32", 0.5, 45, 13, True),        # materialised-projection forward
    (7, 3, 640, 16, "bf16", -1.0, 16, 0, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_K%d_S%d_D%d_%s_a%g_ld%d_off%d_%s" % c)
def test_forward_enrich(case):
    B, K, SH2, D, dt, a, ld, off, with_ctx = case
    w = workload(B, K, SH2, D, dt, a, seed=61)
    print(f"case enrich {w.name} ld={ld} off={off} ctx={with_ctx}", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    h0 = synth.normal_f32(62, 0, (B, ld))
    he = torch.from_numpy(h0).to(DEV)
    cout = torch.full((B, D), float("nan"), device=DEV) if with_ctx else None
    gs.forward_enrich(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], K, he, off, a,
                      context_out=cout)
    torch.cuda.synchronize()
    got = he.cpu().numpy()
    ref = oracle.forward_enrich(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K, h0,
                                off, a)
    keep = np.ones(ld, dtype=bool)
    keep[off:off + D] = False
    assert np.array_equal(got[:, keep], h0[:, keep])
    err = ctx_err(got[:, off:off + D], ref[:, off:off + D])
    print(f"  enriched slice err {err:.2e}", flush=True)
    assert err <= 1e-4
    if with_ctx:
        assert np.array_equal(cout.cpu().numpy(), gpu_forward(t, K, a))


def test_forward_enrich_headline_twice_accumulates():
    """Two calls add the context twice (a read-modify-write, not an overwrite)."""
    w = wl.HEADLINE
    print("case enrich twice", flush=True)
    x = synth.make_inputs(w)
    t = device_inputs(x)
    he = torch.zeros((w.B, w.SH2), device=DEV)
    for _ in range(2):
        gs.forward_enrich(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K, he, 64)
    torch.cuda.synchronize()
    ctx = gpu_forward(t, w.K, 0.0)
    got = he.cpu().numpy()
    assert np.array_equal(got[:, 64:80], ctx + ctx)
    assert not got[:, :64].any() and not got[:, 80:].any()
