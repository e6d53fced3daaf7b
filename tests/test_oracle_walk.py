"""Pins of the oracle's walk ("DFlash 2: Keep Drafting Parallel", Method, last
paragraph; "DFlash 2: The Drafter Stopped Guessing Alone", "Selection beats
correction"): start at the last verified token, follow the best successor
(greedy) or draw from the same scores (sampled).

Greedy is checked against numpy's argmax (first occurrence = lowest slot) and
the closed form W_A = 0 -> per-position top-1 (the plain one-pass drafter's
pick); sampling against scipy's softmax, a chi-square frequency test, u = 0,
dominant rows and the T -> 0 limit."""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import synth

K = 16


def _rand_S(rng, B=3, L=6):
    S = rng.standard_normal((B, L, K, K))
    S[:, 0, 1:] = -np.inf
    return S


def test_greedy_is_argmax_chain(ora):
    rng = np.random.default_rng(0)
    S = _rand_S(rng)
    cid = rng.integers(0, 1000, size=(3, 6, K)).astype(np.int32)
    w = ora.walk(S, cid)
    for b in range(3):
        row = 0
        for t in range(6):
            j = int(np.argmax(S[b, t, row]))
            assert w["path_slot"][b, t] == j and w["path_tok"][b, t] == cid[b, t, j]
            assert w["path_s"][b, t] == S[b, t, row, j]
            srt = np.sort(S[b, t, row])
            assert w["aux"][b, t] == srt[-1] - srt[-2]
            row = j


def test_greedy_ties_and_nan(ora):
    S = np.full((K, K), -1.0)
    S[0, [3, 7, 9]] = 2.0  # three-way tie -> lowest slot
    assert ora.step(S, 0)[0] == 3
    S[1, :] = np.nan
    S[1, 12] = -np.inf  # NaN ranks below -inf
    assert ora.step(S, 1)[0] == 12
    S[2, :] = np.nan
    assert ora.step(S, 2)[0] == 0


def test_zero_pair_weight_walk_is_top1(ora):
    """W_A = 0: the selector reduces to the per-position top-1."""
    cfg = synth.CONFIGS["c0"]
    inp = synth.make(cfg)
    inp["W_A"] = np.zeros_like(inp["W_A"])
    out = ora.run(inp)
    assert np.all(out["path_slot"] == 0)
    np.testing.assert_array_equal(out["path_tok"], np.argmax(inp["logits"], axis=-1))


def test_tiny_workload_departs_from_top1(ora):
    """With the pair term on, the tiny workload's injected repeats get walked around."""
    cfg = synth.CONFIGS["c0"]
    out = ora.run(synth.make(cfg))
    assert np.any(out["path_slot"] != 0)


def test_sampled_matches_softmax_and_edges(ora):
    rng = np.random.default_rng(1)
    s = rng.standard_normal((K, K)) * 2
    for T in (0.5, 1.0, 3.0):
        for u in (0.0, 0.1, 0.5, 0.999):
            j, margin, q = ora.step(s, 4, 1, u, T)
            p = softmax(s[4] / T)
            np.testing.assert_allclose(q, p, rtol=1e-12)
            cdf = np.cumsum(p)
            assert j == int(np.searchsorted(cdf, u, side="right"))
            edges = np.array([0.0 if j == 0 else cdf[j - 1], cdf[j]])
            np.testing.assert_allclose(margin, np.min(np.abs(u - edges)), rtol=1e-9, atol=1e-15)
    assert ora.step(s, 4, 1, 0.0, 1.0)[0] == 0


def test_sampled_dominant_row_and_low_temperature(ora):
    s = np.zeros((K, K))
    s[0, 11] = 60.0
    for u in (0.01, 0.3, 0.999999):
        assert ora.step(s, 0, 1, u, 1.0)[0] == 11
    assert ora.step(s, 0, 1, 0.0, 1.0)[0] == 0  # u = 0 takes the first slot of nonzero weight
    rng = np.random.default_rng(2)
    S = _rand_S(rng)
    g = ora.walk(S, np.zeros((3, 6, K), np.int32))
    smp = ora.walk(S, np.zeros((3, 6, K), np.int32), 1, rng.random((3, 6)).astype(np.float32), 1e-4)
    np.testing.assert_array_equal(g["path_slot"], smp["path_slot"])


def test_sampled_frequencies_chi_square(ora):
    rng = np.random.default_rng(3)
    s = rng.standard_normal((K, K))
    n = 100_000
    S = np.broadcast_to(s, (n, 1, K, K)).copy()
    u = rng.random((n, 1)).astype(np.float32)
    w = ora.walk(S, np.zeros((n, 1, K), np.int32), 1, u, 1.0)
    counts = np.bincount(w["path_slot"][:, 0], minlength=K)
    p = softmax(s[0])
    assert stats.chisquare(counts, n * p).pvalue > 1e-3


def test_step_table_reproduces_walk(ora):
    rng = np.random.default_rng(4)
    S = _rand_S(rng)
    u = rng.random((3, 6)).astype(np.float32)
    for mode, uu in ((0, None), (1, u)):
        ch, _ = ora.step_table(S, mode, uu, 1.0)
        w = ora.walk(S, np.zeros((3, 6, K), np.int32), mode, uu, 1.0)
        for b in range(3):
            row = 0
            for t in range(6):
                assert ch[b, t, row] == w["path_slot"][b, t]
                row = ch[b, t, row]
        assert np.all(ch[:, 0, 1:] == -1)


def test_bad_temperature_is_rejected(ora):
    with pytest.raises(ValueError):
        ora.step(np.zeros((K, K)), 0, 1, 0.5, 0.0)


def test_time_selector_runs_the_stages_of_run(ora):
    """The timed whole-selector entry (the benchmark's CPU baseline) calls the
    same stages in the same order: its path equals run()'s, in both modes."""
    import synth

    cfg = synth.CONFIGS["c0"]
    inp = synth.make(cfg, seed=4)
    for mode in (0, 1):
        slot, sec, threads = ora.time_selector(inp, mode, 1.0)
        assert np.array_equal(slot, ora.run(inp, mode, 1.0)["path_slot"])
        assert set(sec) == {"select_topk", "project", "score_pairs", "walk"} and all(v >= 0 for v in sec.values())
        assert threads >= 1
