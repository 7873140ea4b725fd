"""The oracle's pins must catch plausible mistakes.

Each case compiles a copy of the oracle's C source with one planted mistake
(a dropped term, a wrong sign, a wrong index, a transposed operand, a
reversed time order) into a temporary library and checks that at least one
pin from test_oracle_pins fails against it.  CPU only; the real oracle is
untouched.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gscan_oracle.c")

MUTANTS = {
    "forward_recurrence_wrong": ("x[s] = g * x[s] + Bv[s];", "x[s] = x[s] + g * Bv[s];"),
    "dA_drops_state": ("dA[s] = lam[s] * xs[t * D + s] * g * gc[t * D + s];",
                       "dA[s] = lam[s] * g * gc[t * D + s];"),
    # the complement 1 - g taken with the wrong sign of the argument (g * g)
    "dA_wrong_sign": ("gc[t * D + s] = sigmoid(-(Av[s] + a_shift));",
                      "gc[t * D + s] = sigmoid(Av[s] + a_shift);"),
    "reverse_drops_gate": ("lam[s] = g * lam[s];", "lam[s] = lam[s];"),
    "dC_literal_upstream": ("dC[s] = d_context[b * D + s] * xs[K * D + s];",
                            "dC[s] = d_context[b * D + s];"),
    "projection_transposed": ("out[s] += row[i] * W[i * D + s];",
                              "out[s] += row[i] * W[(i * D + s) % SH2 * D + (i * D + s) / SH2];"),
    "time_reversed": ("const double *row = h_history + (b * K + t) * SH2;\n            project(row, W_A, SH2, D, Av);\n            project(row, W_B, SH2, D, Bv);\n            for (s = 0; s < D; ++s) {\n                const double g = sigmoid(Av[s] + a_shift);\n                x[s]",
                      "const double *row = h_history + (b * K + (K - 1 - t)) * SH2;\n            project(row, W_A, SH2, D, Av);\n            project(row, W_B, SH2, D, Bv);\n            for (s = 0; s < D; ++s) {\n                const double g = sigmoid(Av[s] + a_shift);\n                x[s]"),
    "a_shift_ignored": ("sigmoid(Av[s] + a_shift);\n                    gs", "sigmoid(Av[s]);\n                    gs"),
    "dWC_wrong_row": ("pC[ii * D + s] += h_s2[b * SH2 + ii] * dC[s];",
                      "pC[ii * D + s] += h_s2[(b + 1) % B * SH2 + ii] * dC[s];"),
    # input gradients
    "dh_weights_swapped": ("v += dA[s] * W_A[ii * D + s] + dB[s] * W_B[ii * D + s];",
                           "v += dA[s] * W_B[ii * D + s] + dB[s] * W_A[ii * D + s];"),
    "dh_drops_gate_term": ("v += dA[s] * W_A[ii * D + s] + dB[s] * W_B[ii * D + s];",
                           "v += dB[s] * W_B[ii * D + s];"),
    "dh_transposed_weight": ("v += dA[s] * W_A[ii * D + s] + dB[s] * W_B[ii * D + s];",
                             "v += dA[s] * W_A[(ii * D + s) % SH2 * D + (ii * D + s) / SH2]"
                             " + dB[s] * W_B[(ii * D + s) % SH2 * D + (ii * D + s) / SH2];"),
    "dh_rows_reversed": ("double *out = d_h_history + (b * K + t) * SH2;",
                         "double *out = d_h_history + (b * K + (K - 1 - t)) * SH2;"),
    "dh_reverse_drops_gate": ("adj[s] = gt * adj[s];", "adj[s] = adj[s];"),
    "dh_dA_drops_state": ("dA[s] = adj[s] * xs[t * D + s] * gt * gc[t * D + s];",
                          "dA[s] = adj[s] * gt * gc[t * D + s];"),
    "dh_complement_wrong_sign": ("gc[t * D + s] = sigmoid(-(a_shift + Av[s]));",
                                 "gc[t * D + s] = sigmoid(a_shift + Av[s]);"),
    # the complement by subtraction: loses its precision at saturated gates
    "dA_complement_by_subtraction": ("gc[t * D + s] = sigmoid(-(Av[s] + a_shift));",
                                     "gc[t * D + s] = 1.0 - g;"),
    "dhs2_literal_upstream": ("dC[s] = xs[K * D + s] * d_context[b * D + s];",
                              "dC[s] = d_context[b * D + s];"),
    "dhs2_wrong_weight": ("v += dC[s] * W_C[ii * D + s];", "v += dC[s] * W_B[ii * D + s];"),
    "dh_a_shift_ignored": ("sigmoid(a_shift + Av[s]);", "sigmoid(Av[s]);"),
    # CIFG matrix-memory update
    "cifg_concat_swapped": ("concat[k] = h[k];\n        for (k = 0; k < d_input; ++k)\n            concat[d + k] = X[b * d_input + k];",
                            "concat[d_input + k] = h[k];\n        for (k = 0; k < d_input; ++k)\n            concat[k] = X[b * d_input + k];"),
    "cifg_gate_per_column": ("C_out[e] = f[i] * C_in[e] + fc[i] * (h[i] * h[j]);",
                             "C_out[e] = f[j] * C_in[e] + fc[j] * (h[i] * h[j]);"),
    "cifg_candidate_h_x": ("fc[i] * (h[i] * h[j]);", "fc[i] * (h[i] * X[b * d_input + j % d_input]);"),
    "cifg_no_bias": ("double a = b_f[i];", "double a = 0.0;"),
    "cifg_complement_is_gate": ("fc[i] = sigmoid(-a);", "fc[i] = sigmoid(a);"),
    # bias-gradient reduction
    "colsum_transposed": ("acc += grad[r * cols + j];", "acc += grad[j * rows + r];"),
    "colsum_drops_last_row": ("for (r = 0; r < rows; ++r)\n            acc",
                              "for (r = 0; r + 1 < rows; ++r)\n            acc"),
    "colsum_shifted_column": ("acc += grad[r * cols + j];",
                              "acc += grad[r * cols + (j + 1) % cols];"),
}


def _pins():
    yield lambda: pins.test_gate_zero_closed_form(5, 8, 64, 16)
    yield lambda: pins.test_constant_gate_geometric_sum(0.9, 8)
    yield lambda: pins.test_k2_closed_form_saturated_gates(30.0)
    yield lambda: pins.test_k1_reduces_to_c_times_b(2.0)
    yield lambda: pins.test_explicit_solution_of_recurrence(2.0, 3, 5, 20, 4)
    yield lambda: pins.test_euler_homogeneity(2.0)
    for a in (-3.0, 0.0, 2.0):
        yield lambda a=a: pins.test_central_finite_differences(a)
    yield lambda: pins.test_input_grad_gate_zero_closed_form(5, 8, 64, 16)
    yield lambda: pins.test_input_grad_euler_identities(2.0)
    yield lambda: pins.test_input_grad_k1_and_linearity()
    for a in (-3.0, 0.0, 2.0):
        yield lambda a=a: pins.test_input_grad_central_finite_differences(a)
    from tests import test_oracle_cifg_pins as cp
    yield lambda: cp.test_gate_one_keeps_memory(3, 8, 5)
    yield lambda: cp.test_gate_zero_gives_outer_product(3, 8, 5)
    yield lambda: cp.test_constant_gate(0.25)
    yield cp.test_gate_is_per_row
    yield cp.test_concat_order_h_then_x
    yield cp.test_linear_in_memory_and_samples_independent
    yield pins.test_column_sums_exact_cases
    yield pins.test_column_sums_against_correctly_rounded_sums


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mut.c"
    src.write_text(text.replace(old, new))
    lib_path = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", str(src), "-o",
                    str(lib_path), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(str(lib_path))
    for fn in ("oracle_forward", "oracle_backward", "oracle_backward_inputs", "oracle_column_sums",
               "oracle_cifg_update", "oracle_max_threads", "oracle_set_threads"):
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
        getattr(mut, fn).restype = getattr(real, fn).restype
    caught = False
    oracle._lib = mut
    try:
        for pin in _pins():
            try:
                pin()
            except AssertionError:
                caught = True
                break
    finally:
        oracle._lib = real
    assert caught, f"no pin caught mutant {name}"
