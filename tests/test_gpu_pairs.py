"""score_pairs and walk on the GPU against the oracle.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: eq.
S_t scores every adjacent pair in one parallel pass; the walk from the last
verified token is the only sequential step, greedy or sampled.)

The pair kernel is fed the oracle's projections rounded to fp32 (its own input
precision) so that this file checks the pair arithmetic and the walk alone."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
from helpers import K, check_scores, check_walk

pytestmark = pytest.mark.gpu


def _inputs(seed, B, L, r, pair_scale=1.0):
    rng = np.random.default_rng(seed)
    cand_u = (rng.standard_normal((B, L, K)) * 3).astype(np.float32)
    cand_u = -np.sort(-cand_u, axis=-1)  # sorted like a top-16 list
    A = (rng.standard_normal((B, L, K, r)) * pair_scale).astype(np.float32)
    A[:, 0, 1:] = 0.0
    Bm = (rng.standard_normal((B, L, K, r)) * pair_scale / np.sqrt(r)).astype(np.float32)
    G = rng.random((B, L, r)).astype(np.float32)
    cand_id = rng.integers(0, 1 << 20, size=(B, L, K)).astype(np.int32)
    u = rng.random((B, L)).astype(np.float32)
    return cand_u, A, Bm, G, cand_id, u


def _dev(*arrs, dev):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in arrs]


@pytest.mark.parametrize("B,L,r", [(1, 1, 32), (3, 3, 32), (5, 8, 64), (4, 16, 256), (2, 17, 128),
                                   (2, 32, 256), (37, 16, 256), (3, 5, 96), (2, 9, 160),
                                   (7, 12, 224), (1, 32, 192)])
@pytest.mark.parametrize("mode", [0, 1])
def test_pairs_and_fused_walk(ora, dev, B, L, r, mode):
    cand_u, A, Bm, G, cand_id, u = _inputs(B * 100 + L + r, B, L, r)
    S_ref = ora.score_pairs(cand_u, A.astype(np.float64), Bm.astype(np.float64), G.astype(np.float64))
    d_u, d_A, d_B, d_G, d_id, d_un = _dev(cand_u, A, Bm, G, cand_id, u, dev=dev)
    res = ds.score_pairs(d_u, d_A, d_B, d_G, want_S=True, walk_mode=mode, cand_id=d_id,
                         uniforms=d_un, temperature=1.0, want_q=True)
    torch.cuda.synchronize()
    S = res["S"].cpu().numpy()
    eps, tol, eps_p, tol_p = check_scores(S, S_ref, cand_u)
    gpu = {k: v.cpu().numpy() for k, v in res.items()}
    check_walk(ora, gpu, S_ref, S, cand_id, mode, u, 1.0, eps)
    # the fused walk equals the stand-alone walk over the same scores
    alone = ds.walk(res["S"], d_id, mode=mode, uniforms=d_un, want_q=True)
    torch.cuda.synchronize()
    for k in ("path_slot", "path_tok"):
        assert torch.equal(alone[k], res[k])
    assert torch.equal(alone["q"].view(torch.int32), res["q"].view(torch.int32))
    # q: one-hot (greedy) or the step's softmax (sampled)
    q = gpu["q"].astype(np.float64)
    np.testing.assert_allclose(q.sum(-1), 1.0, rtol=1e-5)
    if mode == 0:
        assert np.all(q[np.arange(B)[:, None], np.arange(L)[None], gpu["path_slot"]] == 1.0)


@pytest.mark.parametrize("mode", [0, 1])
def test_walk_alone_bit_exact(ora, dev, mode):
    """Same fp32 scores on both sides: greedy decisions are exact compares."""
    rng = np.random.default_rng(7 + mode)
    B, L = 50, 16
    S = (rng.integers(-8, 8, size=(B, L, K, K)) * 0.5).astype(np.float32)  # many exact ties
    S[:, 0, 1:] = -np.inf
    cand_id = rng.integers(0, 1000, size=(B, L, K)).astype(np.int32)
    u = rng.random((B, L)).astype(np.float32)
    d_S, d_id, d_u = _dev(S, cand_id, u, dev=dev)
    res = ds.walk(d_S, d_id, mode=mode, uniforms=d_u, want_q=True)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in res.items()}
    S64 = S.astype(np.float64)
    flagged = check_walk(ora, gpu, S64, S, cand_id, mode, u, 1.0, 0.0)
    if mode == 0:
        ref = ora.walk(S64, cand_id, 0)
        np.testing.assert_array_equal(gpu["path_slot"], ref["path_slot"])
        assert flagged == 0


def test_walk_special_rows(ora, dev):
    """NaN ranks lowest, -inf rows, +inf entries, all-NaN rows."""
    B, L = 4, 3
    S = np.zeros((B, L, K, K), np.float32)
    S[:, 0, 1:] = -np.inf
    S[0, :, :, :] = np.nan
    S[0, :, :, 5] = -np.inf            # NaN below -inf: slot 5 everywhere
    S[1, :, :, :] = -np.inf             # no weight: greedy fallback -> slot 0
    S[2, :, :, 7] = np.inf              # one +inf
    S[3, :, :, [2, 9]] = np.inf         # two +inf: sampled splits between them
    cand_id = np.arange(B * L * K, dtype=np.int32).reshape(B, L, K)
    u = np.full((B, L), 0.75, np.float32)
    d_S, d_id, d_u = _dev(S, cand_id, u, dev=dev)
    for mode in (0, 1):
        res = ds.walk(d_S, d_id, mode=mode, uniforms=d_u)
        torch.cuda.synchronize()
        got = res["path_slot"].cpu().numpy()
        ref = ora.walk(S.astype(np.float64), cand_id, mode, u, 1.0)
        np.testing.assert_array_equal(got, ref["path_slot"])


def test_sampled_walk_frequencies(dev):
    """Slot frequencies of the GPU's sampled walk over many uniforms follow the
    step's softmax (chi-square, p > 1e-3)."""
    from scipy import stats
    from scipy.special import softmax

    rng = np.random.default_rng(9)
    row = rng.standard_normal(K).astype(np.float32)
    n = 200_000
    S = np.broadcast_to(row, (n, 1, K, K)).copy()
    u = rng.random((n, 1)).astype(np.float32)
    d_S, d_u = _dev(S, u, dev=dev)
    d_id = torch.zeros((n, 1, K), dtype=torch.int32, device=dev)
    res = ds.walk(d_S, d_id, mode=1, uniforms=d_u, temperature=0.7)
    torch.cuda.synchronize()
    counts = np.bincount(res["path_slot"].cpu().numpy()[:, 0], minlength=K)
    p = softmax(row.astype(np.float64) / 0.7)
    assert stats.chisquare(counts, n * p).pvalue > 1e-3


def test_zero_pair_weight_scores_are_raw_logits(dev):
    cand_u, A, Bm, G, cand_id, u = _inputs(1, 6, 8, 64)
    A[:] = 0.0
    d_u, d_A, d_B, d_G, d_id = _dev(cand_u, A, Bm, G, cand_id, dev=dev)
    res = ds.score_pairs(d_u, d_A, d_B, d_G, want_S=True, walk_mode=0, cand_id=d_id)
    torch.cuda.synchronize()
    S = res["S"].cpu().numpy()
    assert np.array_equal(S[:, 1:], np.broadcast_to(cand_u[:, 1:, None, :], S[:, 1:].shape))
    assert np.array_equal(S[:, 0, 0], cand_u[:, 0])
    assert np.all(res["path_slot"].cpu().numpy() == 0)  # top-1 path
