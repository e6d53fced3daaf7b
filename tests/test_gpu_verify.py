"""verify on the GPU against the oracle.

("DFlash 2: Keep Drafting Parallel", Method, last paragraph, and Setup:
lossless rejection sampling; "DFlash 2: The Drafter Stopped Guessing Alone",
"One pass to draft, one pass to verify".)

Greedy verification compares input logits only, so it must match bit for bit.
The sampled rule takes integer decisions from floating point: the GPU forms
p_t(x) and the draw's CDF in fp32, the oracle in fp64.  A decision may differ
only where the oracle's own margin is within the fp32 error:
  * acceptance  |u q - p| <= 1e-5 u q  (p in fp32: a few ulp of exp2 and of Z),
  * draw        distance of u Z to the nearest CDF edge <= 1e-5 Z (fp32 sums of
                a few hundred tokens per thread and a 256-wide prefix).
Such steps are counted; the test then continues from the GPU's decision
(teacher forcing) and checks that a flagged draw is still a valid one: the
GPU's token's fp64 CDF interval must contain u Z within that tolerance."""
import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax

import draft_selection_amd as ds
import synth

pytestmark = pytest.mark.gpu
K = 16
ACC_TOL, DRAW_TOL = 1e-5, 1e-5


def _widen(tl):
    return tl.astype(np.float64) if tl.dtype == np.float32 else synth.bf16_bits_to_f32(tl).astype(np.float64)


def _dev_logits(tl, dev):
    if tl.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(tl).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(tl)).to(dev)


def _draw_weights(z, T, cand, q, residual):
    p = softmax(z / T)
    if residual:
        qv = np.zeros_like(p)
        qv[cand] = q
        p = np.maximum(0.0, p - qv)
    return p


def check_verify(ora, tl, cand, slots, q, mode, T, u_acc, u_res, n_gpu, tok_gpu, vocab=None):
    """Compare one call's outputs with the oracle (rules in the module doc);
    returns the number of flagged decisions."""
    ref = ora.verify(tl, cand, slots, q, mode=mode, T=T, u_acc=u_acc, u_res=u_res, vocab=vocab)
    B, L = slots.shape
    V = tl.shape[-1] if vocab is None else vocab
    flagged = 0
    for b in range(B):
        n, nr = int(n_gpu[b]), int(ref["n_acc"][b])
        if n != nr:
            assert mode == 1, f"block {b}: greedy acceptance differs ({n} vs {nr})"
            t = min(n, nr)
            uq = float(u_acc[b, t]) * float(q[b, t, slots[b, t]])
            assert ref["m_acc"][b, t] <= ACC_TOL * uq + 1e-30, f"block {b}: acceptance at {t} not near its edge"
            flagged += 1
        acc = cand[b, np.arange(n), slots[b, :n]]
        assert np.array_equal(tok_gpu[b, :n], acc), f"block {b}: accepted tokens"
        assert np.all(tok_gpu[b, n + 1:] == -1)
        if n == nr:
            want, margin = int(ref["out_tok"][b, n]), float(ref["m_draw"][b])
        else:
            want, margin = ora.verify_draw(tl, b, n, n < L, cand, q, mode=mode, T=T, u_res=u_res, vocab=vocab)
        got = int(tok_gpu[b, n])
        if got == want:
            continue
        assert mode == 1 and margin <= DRAW_TOL, f"block {b}: extra token {got} vs {want} (margin {margin})"
        w = _draw_weights(_widen(tl[b, n, :V]), T, cand[b, n] if n < L else None,
                          q[b, n] if n < L else None, n < L)
        c = np.cumsum(w)
        tau = float(u_res[b]) * c[-1]
        lo = c[got - 1] if got > 0 else 0.0
        assert w[got] > 0 and lo - DRAW_TOL * c[-1] <= tau <= c[got] + DRAW_TOL * c[-1]
        flagged += 1
    return flagged


def _random_case(seed, B, L, V, dtype, T=1.0):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((B, L + 1, V)) * 2.5).astype(np.float32)
    cand = np.stack([rng.permutation(V)[:K] for _ in range(B * L)]).reshape(B, L, K).astype(np.int32)
    # target and draft agree in part: lift the candidates' target logits to
    # about the top of the row (the expected max of V normals is ~sqrt(2 ln V))
    lift = np.float32(2.5 * np.sqrt(2 * np.log(V)))
    for b in range(B):
        for t in range(L):
            z[b, t, cand[b, t]] += lift + rng.random(K).astype(np.float32) * 4
    q = rng.random((B, L, K)) ** 3 + 1e-3
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    slots = np.stack([[rng.choice(K, p=q[b, t] / q[b, t].sum()) for t in range(L)] for b in range(B)]).astype(np.int32)
    tl = z if dtype == "f32" else synth.f32_to_bf16_bits(z)
    return tl, cand, slots, q, rng.random((B, L)).astype(np.float32), rng.random(B).astype(np.float32)


def _run(tl, cand, slots, q, mode, T, ua, ur, dev, vocab=None):
    n, tok = ds.verify(_dev_logits(tl, dev), torch.from_numpy(cand).to(dev), torch.from_numpy(slots).to(dev),
                       torch.from_numpy(q).to(dev) if mode == 1 else None, mode=mode, temperature=T,
                       u_acc=torch.from_numpy(ua).to(dev) if mode == 1 else None,
                       u_res=torch.from_numpy(ur).to(dev) if mode == 1 else None, vocab=vocab)
    torch.cuda.synchronize()
    return n.cpu().numpy(), tok.cpu().numpy()


@pytest.mark.parametrize("B,L,V,dtype", [(40, 5, 3000, "f32"), (30, 8, 5000, "bf16"), (7, 1, 16, "f32"),
                                         (5, 32, 2104, "bf16"), (12, 16, 40000, "f32")])
@pytest.mark.parametrize("mode,T", [(0, 1.0), (1, 1.0), (1, 0.6)])
def test_verify_matches_oracle(ora, dev, B, L, V, dtype, mode, T):
    tl, cand, slots, q, ua, ur = _random_case(B * 7 + L + V, B, L, V, dtype, T)
    n, tok = _run(tl, cand, slots, q, mode, T, ua, ur, dev)
    flagged = check_verify(ora, tl, cand, slots, q.astype(np.float64), mode, T, ua, ur, n, tok)
    assert flagged <= max(1, B // 10)
    if mode == 1 and B >= 12:
        assert 0 < n.sum() < B * L  # the case exercises both acceptance and rejection


def test_verify_padded_rows(ora, dev):
    """ld > vocab (16-byte aligned rows): the padding is never read."""
    rng = np.random.default_rng(5)
    B, L, V, ld = 9, 4, 1000, 1024
    tl, cand, slots, q, ua, ur = _random_case(5, B, L, V, "bf16")
    padded = np.full((B, L + 1, ld), 0x7F80, np.uint16)  # +inf in the padding
    padded[..., :V] = tl
    for mode in (0, 1):
        n, tok = _run(padded, cand, slots, q, mode, 1.0, ua, ur, dev, vocab=V)
        check_verify(ora, padded, cand, slots, q.astype(np.float64), mode, 1.0, ua, ur, n, tok, vocab=V)


def test_verify_output_follows_target_distribution(dev):
    """The textbook identity on the GPU: the first emitted token of a block
    whose drafted token was drawn from q is distributed as softmax(z_0)."""
    rng = np.random.default_rng(11)
    n, V = 100_000, 24
    z = (rng.standard_normal((1, 2, V)) * 2).astype(np.float32)
    cand = rng.permutation(V)[:K].astype(np.int32)
    q = rng.random(K).astype(np.float32) + 0.05
    q /= q.sum()
    pq = q.astype(np.float64)
    slots = rng.choice(K, size=(n, 1), p=pq / pq.sum()).astype(np.int32)
    tl = np.broadcast_to(z, (n, 2, V)).copy()
    _, tok = _run(tl, np.broadcast_to(cand, (n, 1, K)).copy(), slots, np.broadcast_to(q, (n, 1, K)).copy(),
                  1, 1.0, rng.random((n, 1)).astype(np.float32), rng.random(n).astype(np.float32), dev)
    counts = np.bincount(tok[:, 0], minlength=V)
    assert stats.chisquare(counts, n * softmax(z[0, 0].astype(np.float64))).pvalue > 1e-3


def test_verify_all_accepted_and_greedy_ties(ora, dev):
    rng = np.random.default_rng(12)
    B, L, V = 6, 3, 64
    z = np.full((B, L + 1, V), -np.inf, np.float32)
    cand = np.stack([rng.permutation(V)[:K] for _ in range(B * L)]).reshape(B, L, K).astype(np.int32)
    q = np.zeros((B, L, K), np.float32)
    for b in range(B):
        for t in range(L):
            z[b, t, cand[b, t]] = rng.standard_normal(K)
            q[b, t] = softmax(z[b, t, cand[b, t]].astype(np.float64))
        z[b, L] = rng.standard_normal(V)
    z[:, L, 7] = z[:, L, 40] = 9.0  # greedy tie in the last row: lower id
    slots = rng.integers(0, K, (B, L)).astype(np.int32)
    ua = np.full((B, L), 0.999, np.float32)
    ur = rng.random(B).astype(np.float32)
    n, tok = _run(z, cand, slots, q, 1, 1.0, ua, ur, dev)
    assert np.all(n == L)
    check_verify(ora, z, cand, slots, q.astype(np.float64), 1, 1.0, ua, ur, n, tok)
    # greedy: the drafted token is the arg max everywhere, then the tie
    for b in range(B):
        for t in range(L):
            slots[b, t] = int(np.argmax(z[b, t, cand[b, t]]))
    n, tok = _run(z, cand, slots, q, 0, 1.0, ua, ur, dev)
    assert np.all(n == L) and np.all(tok[:, L] == 7)


@pytest.mark.parametrize("name,mode,nblocks", [("c2", 0, 8), ("c3", 1, 8), ("c4", 1, 3)])
def test_verify_workload_blocks(ora, dev, name, mode, nblocks):
    """Full-vocabulary target rows of the workloads, drafted by the GPU path."""
    cfg = synth.CONFIGS[name]
    blocks = np.random.default_rng(21).choice(cfg.batch, size=nblocks, replace=False)
    W_A, W_B, W_H = synth.make_weights(cfg)
    sub = dict(logits=synth.make_logits(cfg, blocks=blocks), E=synth.make_E(cfg), W_A=W_A, W_B=W_B, W_H=W_H,
               h=synth.make_h(cfg, blocks=blocks), verified=synth.make_verified(cfg)[blocks],
               uniforms=synth.make_uniforms(cfg)[blocks])
    d = synth.to_device(sub, dev)
    res = ds.select_path(d["logits"], d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"], mode=mode,
                         uniforms=d["uniforms"], want_q=True)
    torch.cuda.synchronize()
    cand = res["cand_id"].cpu().numpy()
    slots = res["path_slot"].cpu().numpy()
    q = res["q"].cpu().numpy()
    tl = synth.make_target_logits(cfg, blocks=blocks)
    ua_all, ur_all = synth.make_verify_uniforms(cfg)
    ua, ur = ua_all[blocks], ur_all[blocks]
    n, tok = _run(tl, cand, slots, q, mode, cfg.temperature, ua, ur, dev)
    flagged = check_verify(ora, tl, cand, slots, q.astype(np.float64), mode, cfg.temperature, ua, ur, n, tok)
    assert flagged <= nblocks // 2
