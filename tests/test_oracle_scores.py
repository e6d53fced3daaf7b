"""Pins of the oracle's pair scores, eq. S_t of "DFlash 2: Keep Drafting
Parallel" (Method > Lightweight Path Selector):
S_t(a, b) = U_t(b) + <A(a) (.) H(h_t), B(b)>.

The brute force scores *every* pair of vocabulary tokens at every position
(numpy fp64 BLAS) and then looks the candidate pairs up by token id, which also
checks the predecessor wiring.  Closed forms: W_A = 0 or W_B = 0 gives S = U
exactly; W_A = W_B with a zero gate weight gives S(a, a) = U(a) + |A(a)|^2 / 2."""
import numpy as np

import synth

K = 16


def _f64(u):
    return synth.bf16_bits_to_f32(u).astype(np.float64)


def _setup(ora, seed, V=40, d=32, r=24, B=2, L=5, zero=None):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((B, L, V)).astype(np.float32) * 2
    E = synth.f32_to_bf16_bits(rng.standard_normal((V, d)).astype(np.float32))
    W = [synth.f32_to_bf16_bits(rng.standard_normal((r, d)).astype(np.float32) / np.sqrt(d))
         for _ in range(3)]
    if zero is not None:
        W[zero] = np.zeros_like(W[zero])
    h = synth.f32_to_bf16_bits(rng.standard_normal((B, L, d)).astype(np.float32))
    ver = rng.integers(0, V, size=B).astype(np.int32)
    cid, cu = ora.select_topk(logits)
    A, Bm, G = ora.project(E, W[0], W[1], W[2], h, cid, ver)
    S = ora.score_pairs(cu, A, Bm, G)
    return dict(logits=logits, E=E, W=W, h=h, ver=ver, cid=cid, cu=cu, S=S)


def test_scores_match_vocab_pair_table(ora):
    x = _setup(ora, 0)
    E, (WA, WB, WH) = _f64(x["E"]), (_f64(w) for w in x["W"])
    TA, TB = E @ WA.T, E @ WB.T  # [V, r]
    Gt = 1.0 / (1.0 + np.exp(-(_f64(x["h"]) @ WH.T)))  # [B, L, r]
    B, L, V = x["logits"].shape
    for b in range(B):
        for t in range(L):
            P = (TA * Gt[b, t]) @ TB.T  # every (a, b') pair of the vocabulary, [V, V]
            U = x["logits"][b, t].astype(np.float64)
            cur = x["cid"][b, t]
            preds = [x["ver"][b]] if t == 0 else list(x["cid"][b, t - 1])
            for i, a in enumerate(preds):
                np.testing.assert_allclose(x["S"][b, t, i], U[cur] + P[a, cur], rtol=1e-12, atol=1e-12)
            if t == 0:
                assert np.all(np.isneginf(x["S"][b, 0, 1:]))


def test_zero_pair_weight_gives_raw_logits(ora):
    for zero in (0, 1):
        x = _setup(ora, 1 + zero, zero=zero)
        S, cu = x["S"], x["cu"].astype(np.float64)
        for t in range(S.shape[1]):
            n = 1 if t == 0 else K
            assert np.array_equal(S[:, t, :n], np.broadcast_to(cu[:, t, None, :], S[:, t, :n].shape))


def test_self_pair_closed_form(ora):
    """W_A = W_B and W_H = 0 (gate 1/2): S(a, a) = U(a) + |A(a)|^2 / 2."""
    rng = np.random.default_rng(7)
    V, d, r, B, L = 30, 16, 8, 1, 3
    row = rng.standard_normal(V).astype(np.float32)
    logits = np.broadcast_to(row, (B, L, V)).copy()  # same candidates at every position
    E = synth.f32_to_bf16_bits(rng.standard_normal((V, d)).astype(np.float32))
    W = synth.f32_to_bf16_bits(rng.standard_normal((r, d)).astype(np.float32))
    cid, cu = ora.select_topk(logits)
    A, Bm, G = ora.project(E, W, W, np.zeros_like(W), synth.f32_to_bf16_bits(np.ones((B, L, d), np.float32)),
                           cid, np.zeros(B, np.int32))
    S = ora.score_pairs(cu, A, Bm, G)
    TA = _f64(E) @ _f64(W).T
    for t in range(1, L):
        for i in range(K):
            a = cid[0, t, i]
            np.testing.assert_allclose(S[0, t, i, i], row[a] + 0.5 * TA[a] @ TA[a], rtol=1e-12)
