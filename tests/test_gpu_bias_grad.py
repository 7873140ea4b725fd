"""Parity of the bias-gradient reduction (gscan_bias_grad_reduce, through
the C ABI) with the CPU oracle.

Both sides sum in fp64 (the GPU in a fixed blocked order, the oracle row by
row) and the GPU rounds once to fp32, so each output must lie within one
fp32 ulp-sized step of the oracle: |gpu - ref| <= 2^-23 |ref| + 1e-12 sum|x|.
Repeated calls are bitwise equal.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_history_amd as gs
import oracle

pytestmark = pytest.mark.gpu

from tests.gpu_util import DEV  # noqa: E402

SHAPES = [
    (524288, 3),    # IQN bias gradient: B*Q = 8192 * 64 rows, out_dim 3
    (8192, 24),     # Q-denoise hidden-layer bias (12 -> 24 -> 12 MLP, B = 8192)
    (8192, 12),
    (77777, 7),     # ragged row count
    (4096, 256),    # widest phase-1 row layout
    (1000, 257),    # columns owned per thread
    (300, 1000),
    (1, 1),
    (0, 5),         # empty batch: zeros
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%d" % s)
def test_bias_grad_reduce_parity(shape):
    rows, cols = shape
    print(f"case bias grad {rows}x{cols}", flush=True)
    rng = np.random.default_rng(1000 + rows + cols)
    g = (rng.standard_normal((rows, cols)) * 3.0 + 0.5).astype(np.float32)
    t = torch.from_numpy(g).to(DEV)
    out1 = gs.bias_grad_reduce(t)
    out2 = gs.bias_grad_reduce(t)
    torch.cuda.synchronize()
    a, b = out1.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(a, b)
    ref = oracle.column_sums(g)
    scale = np.abs(g.astype(np.float64)).sum(axis=0)
    err = np.abs(a.astype(np.float64) - ref)
    assert np.all(err <= 2.0 ** -23 * np.abs(ref) + 1e-12 * scale), (err.max(), ref[:4])
