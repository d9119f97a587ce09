"""The oracle's pins must catch plausible mistakes.

Each mutant is the oracle's C source with one planted mistake, made here by
replacing one passage of ``oracle/ssm_oracle.c`` (the first string of its MUTANTS
entry, which must occur exactly once) by a wrong one, and built on the CPU in a
temporary directory; the oracle itself carries no test hooks.  The mutants are
scan, token update, convolution and backward mistakes.  Every mutant must fail
at least one pin in ``test_oracle_pins.py``, and the unmutated build must pass
them.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
from tests import test_oracle_pins as pins

MUTANTS = {
    1: ('readout before update',
        '      const double w = d * j->B[xn + n] * x;\n      h[n] = a * h[n] + w;\n      acc += j->C[xn + n] * h[n];\n      if (j->states) j->states[((bi * L + t) * E + e) * N + n] = h[n];',
        '      const double w = d * j->B[xn + n] * x;\n      acc += j->C[xn + n] * h[n];\n      h[n] = a * h[n] + w;\n      if (j->states) j->states[((bi * L + t) * E + e) * N + n] = h[n];'),
    2: ('dropped D*x',
        '    }\n    double yv = acc + (j->D ? j->D[e] * x : 0.0);\n    if (j->z) yv *= oracle_silu(j->z[xe]);',
        '    }\n    double yv = acc;\n    if (j->z) yv *= oracle_silu(j->z[xe]);'),
    3: ('bias after softplus',
        '    const double x = j->u[xe];\n    double d = j->delta[xe] + (j->bias ? j->bias[e] : 0.0);\n    if (j->softplus) d = oracle_softplus(d);\n    double acc = 0.0;\n    for (int64_t n = 0; n < N; n++) {\n      const double a = exp(d * j->A[e * N + n]);',
        '    const double x = j->u[xe];\n    double d = j->delta[xe] + (j->bias ? j->bias[e] : 0.0);\n    if (j->softplus) d = oracle_softplus(d);\n    if (j->softplus && j->bias) d = oracle_softplus(j->delta[xe]) + j->bias[e];\n    double acc = 0.0;\n    for (int64_t n = 0; n < N; n++) {\n      const double a = exp(d * j->A[e * N + n]);'),
    4: ('sign of A flipped',
        '    for (int64_t n = 0; n < N; n++) {\n      const double a = exp(d * j->A[e * N + n]);\n      const double w = d * j->B[xn + n] * x;',
        '    for (int64_t n = 0; n < N; n++) {\n      const double a = exp(-d * j->A[e * N + n]);\n      const double w = d * j->B[xn + n] * x;'),
    5: ('write term without the step',
        '      const double a = exp(d * j->A[e * N + n]);\n      const double w = d * j->B[xn + n] * x;\n      h[n] = a * h[n] + w;',
        '      const double a = exp(d * j->A[e * N + n]);\n      const double w = j->B[xn + n] * x;\n      h[n] = a * h[n] + w;'),
    6: ('gate without its z factor',
        '  return z / (1.0 + exp(-z));',
        '  return 1.0 / (1.0 + exp(-z));'),
    7: ('reversed state index on B',
        '      const double a = exp(d * j->A[e * N + n]);\n      const double w = d * j->B[xn + n] * x;\n      h[n] = a * h[n] + w;',
        '      const double a = exp(d * j->A[e * N + n]);\n      const double w = d * j->B[xn + (N - 1 - n)] * x;\n      h[n] = a * h[n] + w;'),
    8: ('C read one step late',
        '      h[n] = a * h[n] + w;\n      acc += j->C[xn + n] * h[n];\n      if (j->states) j->states[((bi * L + t) * E + e) * N + n] = h[n];',
        '      h[n] = a * h[n] + w;\n      acc += j->C[(t > 0 ? xn - N : xn) + n] * h[n];\n      if (j->states) j->states[((bi * L + t) * E + e) * N + n] = h[n];'),
    9: ('softplus sign error',
        '  if (x > 0.0) return x + log1p(exp(-x));',
        '  if (x > 0.0) return x + log1p(exp(x));'),
    10: ('B and C swapped in the token update',
        '      double* s = &j->state[c * N + n];\n      *s = exp(d * j->A[e * N + n]) * *s + d * j->B[bi * N + n] * x;\n      acc += j->C[bi * N + n] * *s;\n    }',
        '      double* s = &j->state[c * N + n];\n      *s = exp(d * j->A[e * N + n]) * *s + d * j->C[bi * N + n] * x;\n      acc += j->B[bi * N + n] * *s;\n    }'),
    11: ('convolution without its silu',
        '        }\n        x[(bi * L + t) * E + c] = oracle_silu(acc);\n      }',
        '        }\n        x[(bi * L + t) * E + c] = acc;\n      }'),
    12: ('reversed taps in the convolution token update',
        '      double acc = cb ? cb[c] : 0.0;\n      for (int64_t k = 0; k < K; k++) acc += q[c * K + k] * st[k];\n      x[bi * E + c] = oracle_silu(acc);',
        '      double acc = cb ? cb[c] : 0.0;\n      for (int64_t k = 0; k < K; k++) acc += q[c * K + (K - 1 - k)] * st[k];\n      x[bi * E + c] = oracle_silu(acc);'),
    13: ('backward: retention gradient uses h_t instead of h_{t-1}',
        '      dut += G * d * j->B[xn + n];\n      const double ha = h_prev * a;\n      dd += G * x * j->B[xn + n] + G * ha * j->A[e * N + n];',
        '      dut += G * d * j->B[xn + n];\n      const double ha = h_t * a;\n      dd += G * x * j->B[xn + n] + G * ha * j->A[e * N + n];'),
    14: ('backward: state gradient not decayed by the retention',
        '      j->dA[e * N + n] += G * ha * d;\n      X[n] = a * G;\n    }',
        '      j->dA[e * N + n] += G * ha * d;\n      X[n] = G;\n    }'),
    15: ('backward: step gradient without the softplus derivative',
        '    j->du[xe] = dut;\n    const double ddelta = j->softplus ? dd * oracle_sigmoid(raw) : dd;\n    j->ddelta[xe] = ddelta;',
        '    j->du[xe] = dut;\n    const double ddelta = dd;\n    j->ddelta[xe] = ddelta;'),
    16: ('backward: C gradient uses h_{t-1}',
        '      const double a = exp(d * j->A[e * N + n]);\n      j->dC[xn + n] += dq * h_t;\n      j->dB[xn + n] += G * d * x;',
        '      const double a = exp(d * j->A[e * N + n]);\n      j->dC[xn + n] += dq * h_prev;\n      j->dB[xn + n] += G * d * x;'),
    17: ('backward: gate gradient uses the logistic instead of the silu derivative',
        '      const double zz = j->z[xe], sg = oracle_sigmoid(zz);\n      j->dz[xe] = j->dy[xe] * q[t] * sg * (1.0 + zz * (1.0 - sg));\n      dq *= oracle_silu(zz);',
        '      const double zz = j->z[xe], sg = oracle_sigmoid(zz);\n      j->dz[xe] = j->dy[xe] * q[t] * sg;\n      dq *= oracle_silu(zz);'),
    18: ('backward: B gradient without the step',
        '      j->dC[xn + n] += dq * h_t;\n      j->dB[xn + n] += G * d * x;\n      dut += G * d * j->B[xn + n];',
        '      j->dC[xn + n] += dq * h_t;\n      j->dB[xn + n] += G * x;\n      dut += G * d * j->B[xn + n];'),
    19: ('backward: gradient of the last state ignored',
        '  for (int64_t n = 0; n < N; n++) X[n] = j->dlast ? j->dlast[(bi * E + e) * N + n] : 0.0;\n  for (int64_t t = L - 1; t >= 0; t--) {',
        '  for (int64_t n = 0; n < N; n++) X[n] = j->dlast ? j->dlast[(bi * E + e) * N + n] : 0.0;\n  for (int64_t n = 0; n < N; n++) X[n] = 0.0;\n  for (int64_t t = L - 1; t >= 0; t--) {'),
}

# cheap pins first; each mutant stops at its first failing pin
PIN_CALLS = [
    pins.test_softplus_matches_library,
    pins.test_silu_matches_library,
    pins.test_gate_and_direct_path_with_zero_readout,
    pins.test_no_D_no_gate_is_plain_readout,
    pins.test_bias_is_added_before_softplus,
    pins.test_p9_retention_in_unit_interval,
    pins.test_p5_geometric_series,
    pins.test_p6_lti_convolution,
    pins.test_p2_prefix_equals_sequential,
    pins.test_p7_scan_equals_token_steps,
    lambda: pins.test_p3_zero_step_keeps_state_bitwise(False),
    pins.test_p4_large_step_resets_state,
    pins.test_p1_quadratic_closed_form_L64,
    pins.test_p1_hand_unrolled_L5_in_50_digits,
    lambda: pins.test_conv_matches_numpy_convolve(4),
    pins.test_conv_token_steps_equal_sequence,
    lambda: pins.test_bwd_matches_finite_differences(True, True, True, True, True, True),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def mutant_source(k, directory):
    """ssm_oracle.c with mutant k's passage replaced, written to directory; returns its path."""
    with open(oracle_build.SRC) as f:
        src = f.read()
    old, new = MUTANTS[k][1], MUTANTS[k][2]
    assert src.count(old) == 1, f"mutant {k}: its passage no longer occurs exactly once in the oracle"
    path = os.path.join(directory, f"mut{k}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    return path


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_every_mutant_fails_a_pin(k, mutant_dir):
    d = str(mutant_dir)
    lib = oracle_build.build(out=os.path.join(d, f"mut{k}.so"), src=mutant_source(k, d))
    oracle.use_library(lib)
    try:
        caught = None
        for call in PIN_CALLS:
            try:
                call()
            except (AssertionError, RuntimeError, FloatingPointError, ValueError) as exc:
                caught = exc
                break
        assert caught is not None, f"mutant {k} ({MUTANTS[k][0]}) passed every pin"
    finally:
        oracle.use_library(None)


def test_unmutated_build_passes_all_listed_pins(mutant_dir):
    lib = oracle_build.build(out=os.path.join(str(mutant_dir), "mut0.so"))
    oracle.use_library(lib)
    try:
        for call in PIN_CALLS:
            call()
    finally:
        oracle.use_library(None)
