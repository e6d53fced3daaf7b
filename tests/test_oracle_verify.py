"""Pins of the oracle's verification step (lossless rejection sampling).

("DFlash 2: Keep Drafting Parallel", Method, last paragraph, and Setup: the
sampled walk stays lossless through rejection sampling; "DFlash 2: The Drafter
Stopped Guessing Alone", "One pass to draft, one pass to verify": the accepted
prefix is kept and the first miss is replaced by the target's own choice.)

The pages print no worked example; these tests pin the oracle to the textbook
identity that makes the scheme lossless (the verified token is distributed as
the target's softmax whatever the draft distribution), to closed forms and to
library routines."""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

K = 16


def _inverse_cdf(w, u):
    c = np.cumsum(w)
    return int(np.searchsorted(c, u * c[-1], side="right"))


def _single_block(rng, V, L, T=1.0):
    z = (rng.standard_normal((1, L + 1, V)) * 2).astype(np.float32)
    cand = np.stack([rng.permutation(V)[:K] for _ in range(L)]).reshape(1, L, K).astype(np.int32)
    q = rng.random((1, L, K)) + 0.05
    q /= q.sum(-1, keepdims=True)
    return z, cand, q


def test_first_token_follows_the_target_distribution(ora):
    """The textbook identity: draw the drafted token from q, verify, and the
    emitted token of position 0 is distributed as softmax(z_0 / T)."""
    rng = np.random.default_rng(1)
    V, L, T, n = 24, 1, 0.8, 60000
    z, cand, q = _single_block(rng, V, L)
    slots = np.array([rng.choice(K, p=q[0, 0]) for _ in range(n)], np.int32).reshape(n, 1)
    res = ora.verify(np.broadcast_to(z, (n, L + 1, V)).copy(), np.broadcast_to(cand, (n, L, K)).copy(),
                     slots, np.broadcast_to(q, (n, L, K)).copy(), mode=1, T=T,
                     u_acc=rng.random((n, L)).astype(np.float32), u_res=rng.random(n).astype(np.float32))
    counts = np.bincount(res["out_tok"][:, 0], minlength=V)
    p = softmax(z[0, 0].astype(np.float64) / T)
    assert stats.chisquare(counts, n * p).pvalue > 1e-3
    # and it really rejects sometimes: q is not the target
    assert 0.05 < np.mean(res["n_acc"] == 0) < 0.95


def test_bonus_token_is_the_inverse_cdf_of_the_last_row(ora):
    """Target mass only on the candidates, equal to the draft's q there: every
    position is accepted (u q < p = q), and the extra token is the inverse-CDF
    draw from row L."""
    rng = np.random.default_rng(2)
    V, L, T = 40, 3, 1.0
    z, cand, _ = _single_block(rng, V, L)
    q = np.zeros((1, L, K))
    for t in range(L):
        zt = np.full(V, -np.inf, np.float32)
        zt[cand[0, t]] = z[0, t, cand[0, t]]
        z[0, t] = zt
        q[0, t] = softmax(zt[cand[0, t]].astype(np.float64) / T)
    slots = rng.integers(0, K, size=(1, L)).astype(np.int32)
    for u in (0.0, 0.3, 0.77, 0.999):
        res = ora.verify(z, cand, slots, q, mode=1, T=T, u_acc=np.full((1, L), 0.999, np.float32),
                         u_res=np.array([u], np.float32))
        assert res["n_acc"][0] == L
        assert np.array_equal(res["out_tok"][0, :L], cand[0, np.arange(L), slots[0]])
        assert res["out_tok"][0, L] == _inverse_cdf(softmax(z[0, L].astype(np.float64) / T), np.float32(u))


def test_zero_target_mass_rejects_and_draws_from_the_target(ora):
    """q one-hot on the drafted token x with p(x) = 0: rejected, and the
    residual max(0, p - q) is p itself."""
    rng = np.random.default_rng(3)
    V, L = 50, 2
    z, cand, _ = _single_block(rng, V, L)
    q = np.zeros((1, L, K))
    q[0, :, 5] = 1.0
    slots = np.full((1, L), 5, np.int32)
    z[0, 0, cand[0, 0, 5]] = -np.inf
    u = np.float32(0.4)
    res = ora.verify(z, cand, slots, q, mode=1, T=1.0, u_acc=np.zeros((1, L), np.float32),
                     u_res=np.array([u], np.float32))
    assert res["n_acc"][0] == 0
    assert res["out_tok"][0, 0] == _inverse_cdf(softmax(z[0, 0].astype(np.float64)), u)
    assert np.all(res["out_tok"][0, 1:] == -1)


def test_residual_draw_closed_form(ora):
    """A rejected position draws from max(0, p - q) renormalised (library
    routines: softmax, cumsum, searchsorted)."""
    rng = np.random.default_rng(4)
    V, L, T = 30, 2, 1.3
    z, cand, q = _single_block(rng, V, L)
    for u in (0.05, 0.5, 0.95):
        tok, margin = ora.verify_draw(z, 0, 1, True, cand, q, T=T, u_res=np.array([u], np.float32))
        p = softmax(z[0, 1].astype(np.float64) / T)
        qv = np.zeros(V)
        qv[cand[0, 1]] = q[0, 1]
        assert tok == _inverse_cdf(np.maximum(0.0, p - qv), np.float32(u))
        assert margin >= 0.0


def test_acceptance_is_min_one_p_over_q(ora):
    """Over many uniforms the acceptance rate of a fixed drafted token is
    min(1, p(x) / q(x))."""
    rng = np.random.default_rng(5)
    V, L, n = 20, 1, 40000
    z, cand, q = _single_block(rng, V, L)
    p = softmax(z[0, 0].astype(np.float64))
    for slot in (0, 7):
        x = cand[0, 0, slot]
        res = ora.verify(np.broadcast_to(z, (n, 2, V)).copy(), np.broadcast_to(cand, (n, 1, K)).copy(),
                         np.full((n, 1), slot, np.int32), np.broadcast_to(q, (n, 1, K)).copy(), mode=1,
                         u_acc=rng.random((n, 1)).astype(np.float32), u_res=rng.random(n).astype(np.float32))
        rate = np.mean(res["n_acc"] == 1)
        want = min(1.0, p[x] / q[0, 0, slot])
        assert abs(rate - want) < 4 * np.sqrt(want * (1 - want) / n) + 1e-3


def test_greedy_accepts_the_argmax_prefix(ora):
    rng = np.random.default_rng(6)
    V, L = 64, 5
    z, cand, _ = _single_block(rng, V, L)
    slots = np.zeros((1, L), np.int32)
    # positions 0 and 1 draft the target's arg max; position 2 does not
    for t in range(3):
        top = int(np.argmax(z[0, t]))
        if t < 2:
            cand[0, t, 0] = top
        else:
            cand[0, t, 0] = (top + 1) % V
            cand[0, t, 1:] = [v for v in range(V) if v not in (top, cand[0, t, 0])][:K - 1]
    # a tie at position 2: the lower id wins
    z[0, 2, 3] = z[0, 2, 11] = z[0, 2].max() + 1
    res = ora.verify(z, cand, slots, mode=0)
    assert res["n_acc"][0] == 2
    assert list(res["out_tok"][0]) == [cand[0, 0, 0], cand[0, 1, 0], 3, -1, -1, -1]
    # all accepted: the extra token is row L's arg max
    for t in range(L):
        cand[0, t, 0] = int(np.argmax(z[0, t]))
    res = ora.verify(z, cand, slots, mode=0)
    assert res["n_acc"][0] == L and res["out_tok"][0, L] == int(np.argmax(z[0, L]))


def test_bf16_rows_with_padding_match_fp32(ora):
    import synth

    rng = np.random.default_rng(7)
    V, L, ld = 37, 2, 48
    z, cand, q = _single_block(rng, V, L)
    bits = synth.f32_to_bf16_bits(z)
    widened = synth.bf16_bits_to_f32(bits)
    padded = np.zeros((1, L + 1, ld), np.uint16)
    padded[..., :V] = bits
    kw = dict(mode=1, T=1.0, u_acc=rng.random((1, L)).astype(np.float32),
              u_res=rng.random(1).astype(np.float32))
    slots = rng.integers(0, K, (1, L)).astype(np.int32)
    a = ora.verify(padded, cand, slots, q, vocab=V, **kw)
    b = ora.verify(widened, cand, slots, q, **kw)
    assert np.array_equal(a["n_acc"], b["n_acc"]) and np.array_equal(a["out_tok"], b["out_tok"])
