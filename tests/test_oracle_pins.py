"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something the mathematics fixes:
closed forms of special cases (gate 0, constant gate, K = 1), the explicit
solution of the linear recurrence, exact identities of the loss (Euler
homogeneity, linearity, additivity, equivariance) and central finite
differences of the forward.  Inputs here come from numpy's own generator in
float64 so that nothing shares code with the oracle.
"""
import math

import numpy as np
import pytest

import oracle


def _inputs(B, K, SH2, D, seed):
    rng = np.random.default_rng(seed)
    return dict(
        h_history=rng.standard_normal((B * K, SH2)),
        h_s2=rng.standard_normal((B, SH2)),
        W_A=rng.standard_normal((SH2, D)) / math.sqrt(SH2),
        W_B=rng.standard_normal((SH2, D)) / math.sqrt(SH2),
        W_C=rng.standard_normal((SH2, D)) / math.sqrt(SH2),
        d_context=rng.standard_normal((B, D)),
    )


def _fwd(x, K, a_shift=0.0):
    return oracle.forward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K, a_shift)


def _bwd(x, K, a_shift=0.0, d=None):
    d = x["d_context"] if d is None else d
    return oracle.backward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K, d,
                           a_shift)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))


@pytest.mark.parametrize("B,K,SH2,D", [(5, 8, 64, 16), (3, 3, 7, 5), (2, 1, 4, 3)])
def test_gate_zero_closed_form(B, K, SH2, D):
    # sigmoid(A - 1e4) == 0 exactly in float64, so x_K = B_{K-1}.
    x = _inputs(B, K, SH2, D, 1)
    a_shift = -1.0e4
    Cv = x["h_s2"] @ x["W_C"]
    last = x["h_history"][np.arange(B) * K + K - 1]
    Bl = last @ x["W_B"]
    assert _rel(_fwd(x, K, a_shift), Cv * Bl) < 1e-12
    dWA, dWB, dWC = _bwd(x, K, a_shift)
    assert np.all(dWA == 0.0)
    dc = x["d_context"]
    assert _rel(dWB, last.T @ (dc * Cv)) < 1e-12
    assert _rel(dWC, x["h_s2"].T @ (dc * Bl)) < 1e-12


@pytest.mark.parametrize("a_shift", [30.0, -30.0, 0.0])
def test_k2_closed_form_saturated_gates(a_shift):
    # K = 2: x_1 = B_0 and x_2 = g_1 B_0 + B_1 (g_0 multiplies x_0 = 0), so
    # dL/dA_1 = d * C * B_0 * sigma'(a_1) and dL/dA_0 = 0.  The logistic
    # derivative is written here as e^{-a} / (1 + e^{-a})^2, which keeps full
    # relative precision at a = +30 where the gate is 1 - 1e-13; an oracle
    # forming 1 - g by subtraction would be off by about 1e-3 there.
    B, SH2, D = 6, 24, 5
    K = 2
    x = _inputs(B, K, SH2, D, 13)
    Cv = x["h_s2"] @ x["W_C"]
    A = x["h_history"] @ x["W_A"] + a_shift
    Bv = x["h_history"] @ x["W_B"]
    r0, r1 = np.arange(B) * K, np.arange(B) * K + 1
    a1 = A[r1]
    e = np.exp(-a1)
    dsig = e / (1.0 + e) ** 2
    g1 = 1.0 / (1.0 + e)
    dc = x["d_context"]
    dA1 = dc * Cv * Bv[r0] * dsig
    dWA, dWB, dWC = _bwd(x, K, a_shift)
    assert _rel(dWA, x["h_history"][r1].T @ dA1) < 1e-12
    lam = dc * Cv
    expect_B = x["h_history"][r1].T @ lam + x["h_history"][r0].T @ (lam * g1)
    assert _rel(dWB, expect_B) < 1e-12
    assert _rel(dWC, x["h_s2"].T @ (dc * (g1 * Bv[r0] + Bv[r1]))) < 1e-12


@pytest.mark.parametrize("g", [0.5, 0.9])
@pytest.mark.parametrize("K", [1, 4, 8])
def test_constant_gate_geometric_sum(g, K):
    B, SH2, D = 4, 32, 6
    x = _inputs(B, K, SH2, D, 2)
    x["W_A"] = np.zeros_like(x["W_A"])
    a_shift = math.log(g / (1.0 - g))
    Cv = x["h_s2"] @ x["W_C"]
    Bv = (x["h_history"] @ x["W_B"]).reshape(B, K, D)
    weights = np.array([g ** (K - 1 - t) for t in range(K)])
    xK = np.einsum("t,btd->bd", weights, Bv)
    assert _rel(_fwd(x, K, a_shift), Cv * xK) < 1e-12


@pytest.mark.parametrize("a_shift", [-3.0, 0.0, 2.0])
def test_k1_reduces_to_c_times_b(a_shift):
    B, SH2, D = 9, 48, 16
    x = _inputs(B, 1, SH2, D, 3)
    expect = (x["h_s2"] @ x["W_C"]) * (x["h_history"] @ x["W_B"])
    assert _rel(_fwd(x, 1, a_shift), expect) < 1e-12
    dWA, _, _ = _bwd(x, 1, a_shift)
    assert np.all(dWA == 0.0)  # x_0 = 0 removes every gate gradient


@pytest.mark.parametrize("a_shift", [-3.0, 0.0, 2.0])
@pytest.mark.parametrize("B,K,SH2,D", [(3, 5, 20, 4), (2, 9, 16, 3)])
def test_explicit_solution_of_recurrence(a_shift, B, K, SH2, D):
    # x_K = sum_t (prod_{u>t} g_u) * B_t with g_u = sigmoid(A_u + a_shift):
    # the solved form of the recurrence, oldest step first.
    x = _inputs(B, K, SH2, D, 4)
    A = (x["h_history"] @ x["W_A"]).reshape(B, K, D) + a_shift
    Bv = (x["h_history"] @ x["W_B"]).reshape(B, K, D)
    g = 1.0 / (1.0 + np.exp(-A))
    xK = np.zeros((B, D))
    for t in range(K):
        w = np.ones((B, D))
        for u in range(t + 1, K):
            w = w * g[:, u, :]
        xK += w * Bv[:, t, :]
    expect = (x["h_s2"] @ x["W_C"]) * xK
    assert _rel(_fwd(x, K, a_shift), expect) < 1e-12


@pytest.mark.parametrize("a_shift", [-1.0, 0.0, 2.0])
def test_euler_homogeneity(a_shift):
    # L is 1-homogeneous in W_B and in W_C separately: <W, dL/dW> = L.
    B, K, SH2, D = 7, 6, 24, 8
    x = _inputs(B, K, SH2, D, 5)
    L = float(np.sum(x["d_context"] * _fwd(x, K, a_shift)))
    _, dWB, dWC = _bwd(x, K, a_shift)
    assert abs(np.sum(x["W_B"] * dWB) - L) <= 1e-11 * (1 + abs(L))
    assert abs(np.sum(x["W_C"] * dWC) - L) <= 1e-11 * (1 + abs(L))


def test_linear_in_upstream_gradient():
    B, K, SH2, D = 6, 5, 16, 4
    x = _inputs(B, K, SH2, D, 6)
    rng = np.random.default_rng(60)
    d1 = rng.standard_normal((B, D))
    d2 = rng.standard_normal((B, D))
    g1 = _bwd(x, K, 0.5, d1)
    g2 = _bwd(x, K, 0.5, d2)
    g12 = _bwd(x, K, 0.5, d1 + 2.0 * d2)
    for a, b, c in zip(g1, g2, g12):
        assert _rel(c, a + 2.0 * b) < 1e-12


def test_batch_additivity_and_thread_independence():
    B, K, SH2, D = 150, 3, 16, 4  # crosses the oracle's 64-sample blocks
    x = _inputs(B, K, SH2, D, 7)
    full = _bwd(x, K, -0.5)
    cut = 70
    first = {k: v for k, v in x.items()}
    first.update(h_history=x["h_history"][:cut * K], h_s2=x["h_s2"][:cut],
                 d_context=x["d_context"][:cut])
    second = {k: v for k, v in x.items()}
    second.update(h_history=x["h_history"][cut * K:], h_s2=x["h_s2"][cut:],
                  d_context=x["d_context"][cut:])
    a = _bwd(first, K, -0.5)
    b = _bwd(second, K, -0.5)
    for f, p, q in zip(full, a, b):
        assert _rel(f, p + q) < 1e-12
    prev = oracle.max_threads()
    try:
        oracle.set_threads(1)
        one = _bwd(x, K, -0.5)
        oracle.set_threads(max(2, prev))
        many = _bwd(x, K, -0.5)
    finally:
        oracle.set_threads(prev)
    for p, q in zip(one, many):
        assert np.array_equal(p, q)


def test_sample_permutation_equivariance():
    B, K, SH2, D = 11, 4, 16, 4
    x = _inputs(B, K, SH2, D, 8)
    perm = np.random.default_rng(80).permutation(B)
    rows = (perm[:, None] * K + np.arange(K)[None, :]).reshape(-1)
    y = dict(x)
    y.update(h_history=x["h_history"][rows], h_s2=x["h_s2"][perm])
    assert np.array_equal(_fwd(y, K, 0.3), _fwd(x, K, 0.3)[perm])


@pytest.mark.parametrize("a_shift", [-3.0, 0.0, 2.0])
def test_central_finite_differences(a_shift):
    # Deliberately unaligned tiny shape; every weight entry is checked.
    B, K, SH2, D = 3, 4, 5, 3
    x = _inputs(B, K, SH2, D, 9)
    dW = dict(zip(("W_A", "W_B", "W_C"), _bwd(x, K, a_shift)))
    eps = 1e-6

    def loss(y):
        return float(np.sum(y["d_context"] * _fwd(y, K, a_shift)))

    for name in ("W_A", "W_B", "W_C"):
        for i in range(SH2):
            for s in range(D):
                yp = dict(x)
                ym = dict(x)
                wp = x[name].copy()
                wm = x[name].copy()
                wp[i, s] += eps
                wm[i, s] -= eps
                yp[name] = wp
                ym[name] = wm
                fd = (loss(yp) - loss(ym)) / (2 * eps)
                an = dW[name][i, s]
                assert abs(fd - an) <= 1e-7 * (1 + abs(an)), (name, i, s, fd, an)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    got = oracle.widen(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 0.0 and np.signbit(got[4]) and got[5] == float.fromhex("0x1.fep127")


# ----------------------------------------------------------- input gradients
def _bin(x, K, a_shift=0.0, d=None):
    d = x["d_context"] if d is None else d
    return oracle.backward_inputs(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K,
                                  d, a_shift)


@pytest.mark.parametrize("a_shift", [-3.0, 0.0, 2.0])
def test_input_grad_central_finite_differences(a_shift):
    # Every entry of h_history and h_s2 of a deliberately unaligned shape.
    B, K, SH2, D = 3, 4, 5, 3
    x = _inputs(B, K, SH2, D, 19)
    dh, dhs = _bin(x, K, a_shift)
    eps = 1e-6

    def loss(y):
        return float(np.sum(y["d_context"] * _fwd(y, K, a_shift)))

    for name, grad in (("h_history", dh), ("h_s2", dhs)):
        rows, cols = x[name].shape
        for r in range(rows):
            for i in range(cols):
                yp = dict(x)
                ym = dict(x)
                hp = x[name].copy()
                hm = x[name].copy()
                hp[r, i] += eps
                hm[r, i] -= eps
                yp[name] = hp
                ym[name] = hm
                fd = (loss(yp) - loss(ym)) / (2 * eps)
                an = grad[r, i]
                assert abs(fd - an) <= 1e-7 * (1 + abs(an)), (name, r, i, fd, an)


@pytest.mark.parametrize("B,K,SH2,D", [(5, 8, 64, 16), (3, 3, 7, 5), (2, 1, 4, 3)])
def test_input_grad_gate_zero_closed_form(B, K, SH2, D):
    # gate 0: only the last step feeds x_K = B_{K-1}, and dA = 0 everywhere
    x = _inputs(B, K, SH2, D, 21)
    a_shift = -1.0e4
    dh, dhs = _bin(x, K, a_shift)
    Cv = x["h_s2"] @ x["W_C"]
    last = np.arange(B) * K + K - 1
    Bl = x["h_history"][last] @ x["W_B"]
    dc = x["d_context"]
    expect = np.zeros_like(dh)
    expect[last] = (dc * Cv) @ x["W_B"].T
    assert _rel(dh, expect) < 1e-12
    assert np.all(dh[np.setdiff1d(np.arange(B * K), last)] == 0.0)
    assert _rel(dhs, (dc * Bl) @ x["W_C"].T) < 1e-12


@pytest.mark.parametrize("a_shift", [-1.0, 0.0, 2.0])
def test_input_grad_euler_identities(a_shift):
    # L is linear in h_s2 (C_vals is, x_K does not depend on it): <h_s2, dL/dh_s2> = L.
    # With W_A = 0 the gates are constants and L is linear in h_history too.
    B, K, SH2, D = 7, 6, 24, 8
    x = _inputs(B, K, SH2, D, 23)
    L = float(np.sum(x["d_context"] * _fwd(x, K, a_shift)))
    _, dhs = _bin(x, K, a_shift)
    assert abs(np.sum(x["h_s2"] * dhs) - L) <= 1e-11 * (1 + abs(L))
    y = dict(x)
    y["W_A"] = np.zeros_like(x["W_A"])
    Ly = float(np.sum(y["d_context"] * _fwd(y, K, a_shift)))
    dh, _ = _bin(y, K, a_shift)
    assert abs(np.sum(y["h_history"] * dh) - Ly) <= 1e-11 * (1 + abs(Ly))


def test_input_grad_k1_and_linearity():
    # K = 1: x_0 = 0 kills the gate's gradient, d_h = (d_ctx * Cv) W_B^T.
    B, SH2, D = 6, 16, 4
    x = _inputs(B, 1, SH2, D, 25)
    dh, _ = _bin(x, 1, 0.7)
    Cv = x["h_s2"] @ x["W_C"]
    assert _rel(dh, (x["d_context"] * Cv) @ x["W_B"].T) < 1e-12
    # linear in the upstream gradient
    K = 5
    y = _inputs(B, K, SH2, D, 26)
    rng = np.random.default_rng(27)
    d1 = rng.standard_normal((B, D))
    d2 = rng.standard_normal((B, D))
    g1 = _bin(y, K, -0.5, d1)
    g2 = _bin(y, K, -0.5, d2)
    g12 = _bin(y, K, -0.5, d1 - 3.0 * d2)
    for a, b, c in zip(g1, g2, g12):
        assert _rel(c, a - 3.0 * b) < 1e-12


# ------------------------------------------------ bias-gradient reduction
def test_column_sums_exact_cases():
    # integers (exact in fp64 at this size), a constant column, an empty batch
    rng = np.random.default_rng(31)
    g = rng.integers(-1000, 1000, size=(5000, 7)).astype(np.float64)
    assert np.array_equal(oracle.column_sums(g), g.sum(axis=0, dtype=np.int64).astype(np.float64))
    c = np.full((1234, 3), 0.75)
    assert np.array_equal(oracle.column_sums(c), np.full(3, 1234 * 0.75))
    assert np.array_equal(oracle.column_sums(np.zeros((0, 4))), np.zeros(4))


def test_column_sums_against_correctly_rounded_sums():
    # math.fsum is the correctly rounded sum: the plain fp64 running sum of
    # n float32 values stays within n * 2^-53 * sum|x| of it
    rng = np.random.default_rng(32)
    g = rng.standard_normal((20000, 3)).astype(np.float32)
    got = oracle.column_sums(g)
    for j in range(3):
        col = g[:, j].astype(np.float64)
        exact = math.fsum(col.tolist())
        assert abs(got[j] - exact) <= len(col) * 2.0 ** -53 * np.abs(col).sum()
    # columns are not mixed: permuting columns permutes the result
    perm = [2, 0, 1]
    assert np.array_equal(oracle.column_sums(np.ascontiguousarray(g[:, perm])), got[perm])


@pytest.mark.parametrize("ld,off", [(16, 0), (40, 24), (37, 5)])
def test_forward_enrich_adds_context_in_place(ld, off):
    # the fold of the context into h_enriched (Forward Step 2's closing
    # comment, Step 3): the D columns at the offset gain exactly the pinned
    # forward's context, every other column is returned unchanged
    B, K, SH2, D = 6, 3, 20, 16
    x = _inputs(B, K, SH2, D, 21)
    rng = np.random.default_rng(22)
    h0 = rng.standard_normal((B, ld))
    out = oracle.forward_enrich(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K, h0,
                                off, 0.5)
    ctx = _fwd(x, K, 0.5)
    keep = np.ones(ld, dtype=bool)
    keep[off:off + D] = False
    assert np.array_equal(out[:, keep], h0[:, keep])
    assert np.array_equal(out[:, off:off + D], h0[:, off:off + D] + ctx)
    z = oracle.forward_enrich(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K,
                              np.zeros((B, ld)), off, 0.5)
    assert np.array_equal(z[:, off:off + D], ctx)
    with pytest.raises(ValueError):
        oracle.forward_enrich(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], K, h0,
                              ld - D + 1, 0.5)
