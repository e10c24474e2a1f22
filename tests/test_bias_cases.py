"""CPU checks that the GPU parity inputs of bias_cases.py can tell a right
kernel from a wrong one (only the oracle and torch's CPU attention run).

The GPU tests repeat these checks on their own inputs; here the small cases
run in the CPU suite, so a change to the inputs that made them blind fails
without a GPU."""

import numpy as np

import bias_cases as bc
import workloads


def test_wide_tables_discriminate():
    for (gh, gw, d, sigma, qs) in ((14, 14, 64, 2.0, 1.0), (7, 9, 64, 2.0, 1.0), (3, 32, 64, 2.0, 1.0),
                                   (20, 20, 64, 1.0, 8.0), (7, 9, 72, 2.0, 1.0)):
        inp = workloads.make_inputs(1, 2, gh * gw, d, seed=5000 + gh * gw + d, grid=(gh, gw),
                                    table_sigma=sigma, q_scale=qs)
        seps = bc.assert_discriminates(inp, bc.oracle_o(inp))
        assert min(seps.values()) > 2 * bc.SEP_FACTOR * bc.TOL, seps


def test_workload_tables_do_not_discriminate():
    """Why the wide tables exist: on a workload's own 0.02 table, dropping
    the bias moves O by less than the bar."""
    inp = workloads.make_inputs(1, 3, 196, 64, seed=1, grid=(14, 14))
    ref = bc.oracle_o(inp)
    assert bc.rel_err(bc.oracle_o(inp, table=None), ref, inp["v"]) < bc.TOL


def test_one_hot_closed_form():
    inp = bc.one_hot_inputs(1, 2, 14, 14, 64, 5214, 3, -5, 20.0)
    ref = bc.oracle_o(inp)
    assert bc.rel_err(ref, bc.one_hot_expected(inp, 3, -5), inp["v"]) < 1e-4
    bc.assert_discriminates(inp, ref)


def test_textbook_rows_match_oracle():
    inp = bc.constant_magnitude_inputs(1, 3, 6, 7, 32, 5342)
    rows = np.arange(42)
    assert bc.rel_err(bc.oracle_o(inp, rows), bc.textbook_rows(inp, rows), inp["v"]) < 1e-9


def test_signed_zero_inputs_discriminate():
    inp = bc.signed_zero_inputs(1, 2, 7, 9, 72, 5409)
    ref = bc.oracle_o(inp)
    wrong = bc.oracle.binary_attention_rows(
        bc.signbit_zero_mutation(inp["q"]), bc.signbit_zero_mutation(inp["k"]), bc.np64(inp["v"]),
        bc.np64(inp["table"]), 7, 9)["O"]
    assert bc.rel_err(wrong, ref, inp["v"]) > bc.SEP_FACTOR * bc.TOL


def test_growing_keys_rescale_late():
    inp = bc.growing_key_inputs(1, 1, 16, 32, 64, 5532)
    assert bc.late_rescales(inp, np.arange(0, 512, 17)) > 0
