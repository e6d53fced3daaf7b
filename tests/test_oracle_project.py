"""Pins of the oracle's projections ("DFlash 2: Keep Drafting Parallel", Method >
Lightweight Path Selector, eq. S_t: A and B map tokens to compact vectors, H(h_t)
gates them; the walk starts from the last verified token).

Checked against a full-vocabulary fp64 table built with numpy's BLAS matmul and
scipy's expit, and against closed forms that hold exactly in any summation
order."""
import numpy as np
import pytest
from scipy.special import expit

import synth

K = 16


def _inputs(rng, B=3, L=4, V=64, d=96, r=32, e_std=1.0):
    E = synth.f32_to_bf16_bits(rng.standard_normal((V, d)).astype(np.float32) * e_std)
    W = [synth.f32_to_bf16_bits(rng.standard_normal((r, d)).astype(np.float32) / np.sqrt(d))
         for _ in range(3)]
    h = synth.f32_to_bf16_bits(rng.standard_normal((B, L, d)).astype(np.float32))
    cand = np.stack([rng.permutation(V)[:K] for _ in range(B * L)]).reshape(B, L, K).astype(np.int32)
    ver = rng.integers(0, V, size=B).astype(np.int32)
    return E, W, h, cand, ver


def _f64(u):
    return synth.bf16_bits_to_f32(u).astype(np.float64)


def test_projection_matches_vocab_table(ora):
    rng = np.random.default_rng(0)
    E, (WA, WB, WH), h, cand, ver = _inputs(rng)
    A, Bm, G = ora.project(E, WA, WB, WH, h, cand, ver)
    TA = _f64(E) @ _f64(WA).T  # [V, r]: A of every token
    TB = _f64(E) @ _f64(WB).T
    B, L = cand.shape[:2]
    for b in range(B):
        np.testing.assert_allclose(A[b, 0, 0], TA[ver[b]], rtol=1e-12, atol=1e-12)
        assert np.all(A[b, 0, 1:] == 0.0)
        for t in range(1, L):
            np.testing.assert_allclose(A[b, t], TA[cand[b, t - 1]], rtol=1e-12, atol=1e-12)
        for t in range(L):
            np.testing.assert_allclose(Bm[b, t], TB[cand[b, t]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(G, expit(_f64(h) @ _f64(WH).T), rtol=1e-13, atol=1e-15)


def test_one_hot_rows_are_exact(ora):
    """E rows one-hot, W small integers: every partial sum is an exact integer."""
    rng = np.random.default_rng(1)
    V, d, r, B, L = 48, 64, 32, 2, 3
    Ef = np.zeros((V, d), np.float32)
    Ef[np.arange(V), np.arange(V) % d] = 1.0
    Wf = [rng.integers(-8, 9, size=(r, d)).astype(np.float32) for _ in range(3)]
    E = synth.f32_to_bf16_bits(Ef)
    WA, WB, WH = (synth.f32_to_bf16_bits(w) for w in Wf)
    h = synth.f32_to_bf16_bits(np.zeros((B, L, d), np.float32))
    cand = np.stack([rng.permutation(V)[:K] for _ in range(B * L)]).reshape(B, L, K).astype(np.int32)
    ver = np.array([5, 40], np.int32)
    A, Bm, G = ora.project(E, WA, WB, WH, h, cand, ver)
    for b in range(B):
        assert np.array_equal(A[b, 0, 0], Wf[0][:, ver[b] % d])
        for t in range(L):
            assert np.array_equal(Bm[b, t], Wf[1][:, cand[b, t] % d].T)
            if t:
                assert np.array_equal(A[b, t], Wf[0][:, cand[b, t - 1] % d].T)
    assert np.all(G == 0.5)  # h = 0


def test_zero_weights(ora):
    rng = np.random.default_rng(2)
    E, (WA, WB, WH), h, cand, ver = _inputs(rng)
    z = np.zeros_like(WA)
    A, Bm, G = ora.project(E, z, z, z, h, cand, ver)
    assert np.all(A == 0.0) and np.all(Bm == 0.0) and np.all(G == 0.5)


def test_out_of_range_ids_are_rejected(ora):
    rng = np.random.default_rng(3)
    E, (WA, WB, WH), h, cand, ver = _inputs(rng)
    bad = cand.copy()
    bad[1, 2, 3] = E.shape[0]
    with pytest.raises(ValueError):
        ora.project(E, WA, WB, WH, h, bad, ver)
    with pytest.raises(ValueError):
        ora.project(E, WA, WB, WH, h, cand, np.array([0, -1, 0], np.int32))
