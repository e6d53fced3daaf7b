"""Pins of the oracle's LM head with the fused top-16.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: the
candidates are the drafter's own 16 best logits and the selector needs no
extra LM-head forward.)  The oracle computes z = h W^T in fp64 and keeps the
first 16 of every row, value descending, ties to the lower id.  Pinned against
a library matrix product and a full library sort, one-hot hidden states
(closed form: a column of W) and exact integer ties."""
import numpy as np

import oracle
import synth

K = 16


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def _f(u):
    return synth.bf16_bits_to_f32(u).astype(np.float64)


def _lex_top(z, k):
    """Library sort of each row: value descending, then id ascending."""
    ids = np.arange(z.shape[-1])
    return np.stack([np.lexsort((ids, -row))[:k] for row in z])


def test_matches_library_product_and_sort():
    rng = np.random.default_rng(0)
    rows, V, d = 6, 700, 48
    h = _bits(rng.standard_normal((rows, d)))
    W = _bits(rng.standard_normal((V, d)) / np.sqrt(d))
    cid, cz = oracle.lmhead_topk(h, W)
    z = _f(h) @ _f(W).T
    want = _lex_top(z, K + 1)
    assert np.array_equal(cid, want[:, :K])
    np.testing.assert_allclose(cz, np.take_along_axis(z, want, 1), rtol=1e-12, atol=1e-12)


def test_one_hot_hidden_state_reads_a_column():
    rng = np.random.default_rng(1)
    rows, V, d = 4, 300, 32
    W = _bits(rng.standard_normal((V, d)))
    cols = [0, 5, 17, 31]
    h = np.zeros((rows, d), np.float32)
    h[np.arange(rows), cols] = 1.0
    cid, cz = oracle.lmhead_topk(_bits(h), W)
    Wf = _f(W)
    for r, c in enumerate(cols):
        want = _lex_top(Wf[:, c][None], K + 1)[0]
        assert np.array_equal(cid[r], want[:K])
        assert np.array_equal(cz[r], Wf[want, c])


def test_exact_ties_go_to_the_lower_id():
    """Integer inputs: many exactly equal logits; the list must be the lexsort."""
    rng = np.random.default_rng(2)
    rows, V, d = 5, 400, 8
    h = _bits(rng.integers(-1, 2, (rows, d)))
    W = _bits(rng.integers(-1, 2, (V, d)))
    cid, cz = oracle.lmhead_topk(h, W)
    z = _f(h) @ _f(W).T
    assert np.array_equal(cid, _lex_top(z, K))
    assert len(np.unique(z)) < V // 10  # the case really is tie-heavy


def test_sixteen_entries_are_distinct_and_sorted():
    rng = np.random.default_rng(3)
    h = _bits(rng.standard_normal((3, 64)))
    W = _bits(rng.standard_normal((16, 64)))
    cid, cz = oracle.lmhead_topk(h, W)
    for r in range(3):
        assert sorted(cid[r]) == list(range(16))
        assert np.all(np.diff(cz[r, :K]) <= 0)
    assert np.all(np.isneginf(cz[:, K]))  # V = 16: nothing was left out
