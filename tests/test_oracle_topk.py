"""Pins of the oracle's top-16 ("DFlash 2: Keep Drafting Parallel", Method >
Lightweight Path Selector: 16 candidates kept per draft position).

The oracle is checked against a full lexicographic sort (numpy), numpy's argmax
(first occurrence = lower id, the tie rule), crafted rows with known answers and
invariants on the tiny workload."""
import numpy as np
import pytest

import synth

K = 16


def brute_topk(x: np.ndarray, V: int):
    """Full sort of one row by (non-NaN first, value desc, id asc)."""
    x = x[:V].astype(np.float64)
    nan = np.isnan(x)
    key = np.where(nan, 0.0, -x)
    order = np.lexsort((np.arange(V), key, nan))
    return order[:K].astype(np.int32)


def _rows(kind, rng, n, V):
    if kind == "normal":
        return rng.standard_normal((n, V)).astype(np.float32)
    if kind == "ties":  # values from {0, 0.25, ..., 4}: many exact ties
        return (rng.integers(0, 17, size=(n, V)) * 0.25).astype(np.float32)
    if kind == "special":
        choices = np.array([0.0, -0.0, -np.inf, np.inf, np.nan, 1.0, -1.0], np.float32)
        return rng.choice(choices, size=(n, V)).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("V", [16, 17, 23, 31, 100, 1000, 4099])
@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
def test_topk_matches_full_sort_f32(ora, V, kind):
    rng = np.random.default_rng(V * 7 + len(kind))
    x = _rows(kind, rng, 6, V)
    cid, cu = ora.select_topk(x)
    for i in range(x.shape[0]):
        ref = brute_topk(x[i], V)
        np.testing.assert_array_equal(cid[i], ref)
        np.testing.assert_array_equal(cu[i].view(np.uint32), x[i, ref].view(np.uint32))


@pytest.mark.parametrize("V", [16, 19, 1000, 4101])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_topk_matches_full_sort_bf16(ora, V, kind):
    rng = np.random.default_rng(V)
    xf = _rows(kind, rng, 5, V) * np.float32(3.0)
    xb = synth.f32_to_bf16_bits(xf)
    cid, cu = ora.select_topk(xb)
    x = synth.bf16_bits_to_f32(xb)
    for i in range(xb.shape[0]):
        ref = brute_topk(x[i], V)
        np.testing.assert_array_equal(cid[i], ref)
        np.testing.assert_array_equal(cu[i], x[i, ref])


def test_head_is_argmax(ora):
    rng = np.random.default_rng(1)
    x = (rng.integers(0, 9, size=(64, 777)) * 0.5).astype(np.float32)
    cid, _ = ora.select_topk(x)
    np.testing.assert_array_equal(cid[:, 0], np.argmax(x, axis=1))


def test_crafted_rows(ora):
    V = 40
    eq = np.full((1, V), 2.5, np.float32)
    asc = np.arange(V, dtype=np.float32)[None]
    desc = asc[:, ::-1].copy()
    signed_zero = np.zeros((1, V), np.float32)
    signed_zero[0, ::2] = -0.0
    assert np.array_equal(ora.select_topk(eq)[0][0], np.arange(16))
    assert np.array_equal(ora.select_topk(asc)[0][0], np.arange(V - 1, V - 17, -1))
    assert np.array_equal(ora.select_topk(desc)[0][0], np.arange(16))
    assert np.array_equal(ora.select_topk(signed_zero)[0][0], np.arange(16))  # -0 == +0
    nan_row = np.full((1, V), np.nan, np.float32)
    nan_row[0, 30] = -np.inf
    got = ora.select_topk(nan_row)[0][0]
    assert got[0] == 30 and np.array_equal(got[1:], np.arange(15))  # NaN ranks below -inf


def test_ld_padding_is_ignored(ora):
    rng = np.random.default_rng(5)
    V, ld = 50, 64
    x = np.full((3, ld), np.inf, np.float32)
    x[:, :V] = rng.standard_normal((3, V))
    cid, _ = ora.select_topk(x, vocab=V)
    for i in range(3):
        np.testing.assert_array_equal(cid[i], brute_topk(x[i], V))


def test_vocab_below_k_is_rejected(ora):
    with pytest.raises(ValueError):
        ora.select_topk(np.zeros((1, 15), np.float32))


def test_invariants_on_tiny_workload(ora):
    cfg = synth.CONFIGS["c0"]
    x = synth.make_logits(cfg)
    cid, cu = ora.select_topk(x)
    flat = x.reshape(-1, cfg.vocab)
    ids = cid.reshape(-1, K)
    vals = cu.reshape(-1, K)
    for i in range(flat.shape[0]):
        row, c, v = flat[i], ids[i], vals[i]
        assert len(set(c.tolist())) == K and c.min() >= 0 and c.max() < cfg.vocab
        np.testing.assert_array_equal(v, row[c])
        for k in range(K - 1):  # sorted by (value desc, id asc)
            assert v[k] > v[k + 1] or (v[k] == v[k + 1] and c[k] < c[k + 1])
        rest = np.setdiff1d(np.arange(cfg.vocab), c)  # completeness
        assert np.all((row[rest] < v[-1]) | ((row[rest] == v[-1]) & (rest > c[-1])))
