"""Pins of the oracle's ragged batches (a length per block).

The block size is a per-request knob: "DFlash 2: Keep Drafting Parallel",
supplementary deployment notes (oMLX runs blocks of 5, the release tables use
8 and 16); "DFlash 2: The Drafter Stopped Guessing Alone", "What to check on
your own serving" (a block longer than the acceptance length wastes draft work,
a shorter one leaves tokens behind).  In a ragged batch block b keeps the padded
[batch, block] layout and has block_len[b] valid positions.

The pages print no ragged example.  What pins the oracle is causality: the
selector's position t reads positions t - 1 and t only, the walk and the
acceptance test run front to back, so every result of a block cut to n
positions must equal the first n results of the full block -- computed here by
the uniform oracle at full length, a different call with a different L.  A
dropped offset, a wrong start row or a bonus row taken at the padded length
instead of the block's own fails one of these.  The extra token of a cut block
comes from its row n, checked against numpy's arg max and an inverse CDF."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

K = 16
TINY = synth.CONFIGS["c0"].replace(batch=6)


def _lens(seed, B, L, lo=0):
    return np.random.default_rng(seed).integers(lo, L + 1, size=B).astype(np.int32)


def _with_garbage(inp, lens):
    """Padding rows of every per-position input replaced by NaN / huge values."""
    out = dict(inp)
    lg = inp["logits"].copy()
    h = inp["h"].copy()
    u = inp["uniforms"].copy()
    for b, n in enumerate(lens):
        lg[b, n:] = np.float32(np.nan) if lg.dtype == np.float32 else 0x7FC0
        h[b, n:] = 0x7F7F  # bf16 3.4e38
        u[b, n:] = np.float32(np.nan)
    out.update(logits=lg, h=h, uniforms=u)
    return out


@pytest.mark.parametrize("mode", [oracle.GREEDY, oracle.SAMPLED])
def test_cut_block_equals_prefix_of_full_block(mode):
    inp = synth.make(TINY, seed=3)
    lens = np.array([0, 1, 3, 8, 5, 2], np.int32)
    full = oracle.run(inp, mode, T=0.7)
    rag = oracle.run_ragged(inp, lens, mode, T=0.7)
    for k in ("cand_id", "cand_u", "A_prev", "B_cur", "G", "S", "path_tok", "path_slot", "path_s", "q"):
        for b, n in enumerate(lens):
            np.testing.assert_array_equal(rag[k][b, :n], full[k][b, :n], err_msg=f"{k} block {b}")
            pad = rag[k][b, n:]
            assert np.all(pad == -1) if pad.dtype == np.int32 else np.all(np.isnan(pad)), k


def test_padding_is_never_read():
    inp = synth.make(TINY, seed=4)
    lens = _lens(4, TINY.batch, TINY.block)
    a = oracle.run_ragged(inp, lens, oracle.SAMPLED, T=1.0)
    b = oracle.run_ragged(_with_garbage(inp, lens), lens, oracle.SAMPLED, T=1.0)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_full_lengths_are_the_uniform_batch():
    inp = synth.make(TINY, seed=5)
    lens = np.full(TINY.batch, TINY.block, np.int32)
    full = oracle.run(inp)
    rag = oracle.run_ragged(inp, lens)
    for k in ("cand_id", "S", "path_tok", "path_slot", "path_s"):
        np.testing.assert_array_equal(rag[k], full[k])


def test_lengths_out_of_range_are_rejected():
    inp = synth.make(TINY, seed=5)
    for bad in ([9, 1, 1, 1, 1, 1], [-1, 1, 1, 1, 1, 1], [1, 1]):
        with pytest.raises(ValueError):
            oracle.run_ragged(inp, np.array(bad, np.int32))


def _draft(rng, B, L, V):
    cand = np.stack([rng.permutation(V)[:K] for _ in range(B * L)]).reshape(B, L, K).astype(np.int32)
    slot = rng.integers(0, K, size=(B, L)).astype(np.int32)
    q = rng.random((B, L, K)) + 0.05
    q /= q.sum(-1, keepdims=True)
    return cand, slot, q


def _agreeing_target(rng, cand, slot, V, agree):
    """Target logits whose arg max is the drafted token with probability `agree`."""
    B, L = slot.shape
    z = (rng.standard_normal((B, L + 1, V)) * 2).astype(np.float32)
    for b in range(B):
        for t in range(L):
            if rng.random() < agree:
                z[b, t, cand[b, t, slot[b, t]]] = z[b, t].max() + 1.0
    return z


def test_greedy_verify_of_cut_blocks():
    rng = np.random.default_rng(11)
    B, L, V = 40, 8, 300
    cand, slot, q = _draft(rng, B, L, V)
    z = _agreeing_target(rng, cand, slot, V, 0.85)
    lens = _lens(12, B, L)
    full = oracle.verify(z, cand, slot)
    rag = oracle.verify_ragged(z, lens, cand, slot)
    seen = {"miss inside": 0, "ran past": 0, "empty": 0}
    for b in range(B):
        n, nf = int(lens[b]), int(full["n_acc"][b])
        if nf < n:
            seen["miss inside"] += 1
            assert rag["n_acc"][b] == nf
            np.testing.assert_array_equal(rag["out_tok"][b, :nf + 1], full["out_tok"][b, :nf + 1])
        else:
            seen["empty" if n == 0 else "ran past"] += 1
            assert rag["n_acc"][b] == n
            np.testing.assert_array_equal(rag["out_tok"][b, :n], cand[b, np.arange(n), slot[b, :n]])
            assert rag["out_tok"][b, n] == int(np.argmax(z[b, n]))  # the block's own next row
        assert np.all(rag["out_tok"][b, rag["n_acc"][b] + 1:] == -1)
    assert min(seen.values()) > 0, seen


def test_sampled_verify_of_cut_blocks():
    rng = np.random.default_rng(13)
    B, L, V, T = 48, 6, 200, 0.9
    cand, slot, q = _draft(rng, B, L, V)
    z = _agreeing_target(rng, cand, slot, V, 0.7)
    u_acc = rng.random((B, L)).astype(np.float32)
    u_res = rng.random(B).astype(np.float32)
    lens = _lens(14, B, L)
    full = oracle.verify(z, cand, slot, q, mode=oracle.SAMPLED, T=T, u_acc=u_acc, u_res=u_res)
    rag = oracle.verify_ragged(z, lens, cand, slot, q, mode=oracle.SAMPLED, T=T, u_acc=u_acc, u_res=u_res)
    checked = 0
    for b in range(B):
        n, nf = int(lens[b]), int(full["n_acc"][b])
        if nf < n:
            assert rag["n_acc"][b] == nf
            np.testing.assert_array_equal(rag["out_tok"][b, :nf + 1], full["out_tok"][b, :nf + 1])
        else:
            assert rag["n_acc"][b] == n
            p = softmax(z[b, n].astype(np.float64) / T)
            c = np.cumsum(p)
            want = int(np.searchsorted(c, u_res[b] * c[-1], side="right"))
            edges = np.concatenate([[0.0], c])
            if min(abs(u_res[b] * c[-1] - edges[want]), abs(edges[want + 1] - u_res[b] * c[-1])) > 1e-9:
                assert rag["out_tok"][b, n] == want
                checked += 1
    assert checked > 5


def test_empty_block_is_plain_decoding():
    rng = np.random.default_rng(15)
    B, L, V = 5, 4, 64
    cand, slot, q = _draft(rng, B, L, V)
    z = (rng.standard_normal((B, L + 1, V))).astype(np.float32)
    lens = np.zeros(B, np.int32)
    g = oracle.verify_ragged(z, lens, cand, slot)
    assert np.all(g["n_acc"] == 0)
    np.testing.assert_array_equal(g["out_tok"][:, 0], np.argmax(z[:, 0], axis=1))
    assert np.all(g["out_tok"][:, 1:] == -1)
    u_res = rng.random(B).astype(np.float32)
    s = oracle.verify_ragged(z, lens, cand, slot, q, mode=oracle.SAMPLED, T=1.0,
                             u_acc=rng.random((B, L)).astype(np.float32), u_res=u_res)
    for b in range(B):
        c = np.cumsum(softmax(z[b, 0].astype(np.float64)))
        assert s["out_tok"][b, 0] == int(np.searchsorted(c, u_res[b] * c[-1], side="right"))


def test_conv_of_cut_blocks():
    cfg = synth.CONFIGS["c0"].replace(batch=5, d=64)
    cv = synth.make_conv(cfg, seed=2)
    lens = np.array([0, 1, 8, 3, 6], np.int32)
    y, corr = oracle.dyn_conv(cv["x"], cv["x_prev"], cv["base"], cv["W_c"])
    x = cv["x"].copy()
    for b, n in enumerate(lens):
        x[b, n:] = 0x7F7F  # padding is never read
    yr, cr = oracle.dyn_conv_ragged(x, cv["x_prev"], cv["base"], cv["W_c"], lens)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(yr[b, :n], y[b, :n])
        np.testing.assert_array_equal(cr[b, :n], corr[b, :n])
        assert np.all(np.isnan(yr[b, n:]))


def test_default_length_mix():
    lens = synth.make_block_len(synth.CONFIGS["c2"], seed=0)
    assert lens.shape == (64,) and lens.dtype == np.int32
    assert set(np.unique(lens)) == {5, 8, 16}
    assert set(np.unique(synth.make_block_len(synth.CONFIGS["c3"], seed=0))) == {5, 8}
    with pytest.raises(ValueError):
        synth.make_block_len(synth.CONFIGS["c3"], choices=[9])
