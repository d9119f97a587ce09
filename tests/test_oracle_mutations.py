"""The oracle's pins must catch plausible mistakes.

Each mutant is the oracle C source built with one planted mistake
(``-DORACLE_MUTATION=k``, CPU only); see MUTANTS for the list (scan,
token update, convolution and backward mistakes).  Every mutant must fail at least
one pin in ``test_oracle_pins.py``, and the unmutated build must pass them.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
from tests import test_oracle_pins as pins

MUTANTS = {
    1: "readout before update",
    2: "dropped D*x",
    3: "bias after softplus",
    4: "sign of A flipped",
    5: "write term without the step",
    6: "gate without its z factor",
    7: "reversed state index on B",
    8: "C read one step late",
    9: "softplus sign error",
    10: "B and C swapped in the token update",
    11: "convolution without its silu",
    12: "reversed taps in the convolution token update",
    13: "backward: retention gradient uses h_t instead of h_{t-1}",
    14: "backward: state gradient not decayed by the retention",
    15: "backward: step gradient without the softplus derivative",
    16: "backward: C gradient uses h_{t-1}",
    17: "backward: gate gradient uses the logistic instead of the silu derivative",
    18: "backward: B gradient without the step",
    19: "backward: gradient of the last state ignored",
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


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_every_mutant_fails_a_pin(k, mutant_dir):
    lib = oracle_build.build(out=os.path.join(str(mutant_dir), f"mut{k}.so"), mutation=k)
    oracle.use_library(lib)
    try:
        caught = None
        for call in PIN_CALLS:
            try:
                call()
            except (AssertionError, RuntimeError, FloatingPointError, ValueError) as exc:
                caught = exc
                break
        assert caught is not None, f"mutant {k} ({MUTANTS[k]}) passed every pin"
    finally:
        oracle.use_library(None)


def test_unmutated_build_passes_all_listed_pins(mutant_dir):
    lib = oracle_build.build(out=os.path.join(str(mutant_dir), "mut0.so"), mutation=0)
    oracle.use_library(lib)
    try:
        for call in PIN_CALLS:
            call()
    finally:
        oracle.use_library(None)
