"""The oracle against values worked by hand from the pages (tests/golden)."""
import numpy as np

from helpers import load_golden, stutter_inputs


def test_stutter_example(ora):
    inp, exp = stutter_inputs()
    out = ora.run(inp)
    np.testing.assert_array_equal(out["cand_id"][0], np.array(exp["cand_id"]))
    S = out["S"][0]
    np.testing.assert_array_equal(S[0, 0], exp["S_row0_t0"])
    assert np.all(np.isneginf(S[0, 1:]))
    np.testing.assert_array_equal(S[1, 1], exp["S_row1_t1"])
    np.testing.assert_array_equal(S[2, 1], exp["S_row1_t2"])
    np.testing.assert_array_equal(out["path_tok"][0], exp["path_tok"])
    np.testing.assert_array_equal(out["path_slot"][0], exp["path_slot"])
    np.testing.assert_array_equal(out["path_s"][0], exp["path_s"])


def test_stutter_example_without_pair_term_is_top1(ora):
    inp, exp = stutter_inputs(zero_pair=True)
    out = ora.run(inp)
    np.testing.assert_array_equal(out["path_tok"][0], exp["top1_path_tok"])


def test_projection_shape_matches_published_parameter_count():
    g = load_golden("selector_params.json")
    d, r, V = g["drafter_width_d"], g["rank_r"], g["vocab"]
    three_projections = 3 * d * r  # W_A, W_B, W_H, each r x d
    assert abs(three_projections - g["published_params"]) <= g["published_rounding"]
    vocab_tables = 2 * V * r  # the alternative reading: A, B as vocab x r tables
    assert abs(vocab_tables - g["published_params"]) > 10 * g["published_rounding"]
