"""Pins for the oracle's CIFG matrix-memory update (BURT-IMMA API reference,
batched_cifg_update in independent mode; cifg_update steps 1-4), each fixed
by the definition without re-deriving the oracle's loops: saturated gates
(C unchanged, or C = h h^T exactly), a constant gate, the row-wise
broadcast of the gate, the order of the concatenation [h ; x], linearity in
C and independence of the samples.  Inputs from numpy's generator."""
import math

import numpy as np
import pytest

import oracle


def _inputs(B, d, din, seed):
    rng = np.random.default_rng(seed)
    return dict(C=rng.standard_normal((B, d, d)) / math.sqrt(d),
                H=rng.standard_normal((B, d)), X=rng.standard_normal((B, din)),
                W_f=rng.standard_normal((d, d + din)) / math.sqrt(d + din),
                b_f=rng.standard_normal(d))


def _run(x):
    return oracle.cifg_update(x["C"], x["H"], x["X"], x["W_f"], x["b_f"])


@pytest.mark.parametrize("B,d,din", [(3, 8, 5), (2, 16, 16), (1, 4, 0)])
def test_gate_one_keeps_memory(B, d, din):
    x = _inputs(B, d, din, 1)
    x["W_f"][:] = 0.0
    x["b_f"][:] = 1.0e4          # sigmoid = 1 exactly in float64
    assert np.array_equal(_run(x), x["C"])


@pytest.mark.parametrize("B,d,din", [(3, 8, 5), (2, 16, 16)])
def test_gate_zero_gives_outer_product(B, d, din):
    x = _inputs(B, d, din, 2)
    x["W_f"][:] = 0.0
    x["b_f"][:] = -1.0e4         # sigmoid = 0 exactly: C = h h^T
    h = x["H"]
    assert np.array_equal(_run(x), h[:, :, None] * h[:, None, :])


@pytest.mark.parametrize("f0", [0.25, 0.9])
def test_constant_gate(f0):
    x = _inputs(4, 12, 7, 3)
    x["W_f"][:] = 0.0
    x["b_f"][:] = math.log(f0 / (1.0 - f0))
    h = x["H"]
    expect = f0 * x["C"] + (1.0 - f0) * h[:, :, None] * h[:, None, :]
    assert np.max(np.abs(_run(x) - expect)) < 1e-14


def test_gate_is_per_row():
    # C = 0 and h = 1: every entry of row i is 1 - f_i, so rows are constant
    # along j, and with W_f = 0 row values fall as b_f[i] rises
    B, d, din = 2, 10, 3
    x = _inputs(B, d, din, 4)
    x["C"][:] = 0.0
    x["H"][:] = 1.0
    x["W_f"][:] = 0.0
    out = _run(x)
    assert np.array_equal(out, np.repeat(out[:, :, :1], d, axis=2))
    order = np.argsort(x["b_f"])
    col = out[0, order, 0]
    assert np.all(np.diff(col) < 0)
    assert np.all((col > 0) & (col < 1))


def test_concat_order_h_then_x():
    # with the x columns of W_f zero the update ignores X and equals the
    # update of the same problem without x (W_f restricted to its first d
    # columns): the first d inputs of the gate are h
    B, d, din = 3, 9, 6
    x = _inputs(B, d, din, 5)
    x["W_f"][:, d:] = 0.0
    a = _run(x)
    y = dict(x)
    y["X"] = np.random.default_rng(6).standard_normal((B, din)) * 10.0
    assert np.array_equal(a, _run(y))
    z = dict(x)
    z["X"] = np.zeros((B, 0))
    z["W_f"] = x["W_f"][:, :d].copy()
    assert np.max(np.abs(a - _run(z))) < 1e-14
    # and the x columns do act when nonzero
    w = dict(x)
    w["W_f"] = x["W_f"].copy()
    w["W_f"][:, d:] = 1.0
    assert not np.allclose(_run(w), a)


def test_linear_in_memory_and_samples_independent():
    B, d, din = 4, 8, 8
    x = _inputs(B, d, din, 7)
    y = dict(x)
    y["C"] = np.random.default_rng(8).standard_normal((B, d, d))
    diff = (_run(x) - _run(y)) / (x["C"] - y["C"])     # = f_i, the same along j
    assert np.max(np.abs(diff - diff[:, :, :1])) < 1e-12
    assert np.all((diff > 0) & (diff < 1))
    perm = np.array([2, 0, 3, 1])
    xp = {k: (v[perm] if k in ("C", "H", "X") else v) for k, v in x.items()}
    assert np.array_equal(_run(xp), _run(x)[perm])
