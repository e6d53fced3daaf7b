"""project on the GPU against the oracle.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector, the
paragraph after eq. S_t: A(x) = W_A E[x], B(x) = W_B E[x], H(h) = sigmoid(W_H h).)

Tolerance: every product of two bf16 numbers is exact in fp32, so the GPU's
only error is fp32 accumulation over d terms, bounded in any summation order by
gamma_d * sum_k |x_k w_k| with gamma_d = d u / (1 - d u), u = 2^-24.  The test
applies that bound element by element (plus sigmoid's own few-ulp error on G)."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth
from helpers import K, bf16_dev, to_dev

pytestmark = pytest.mark.gpu


def _f64(u):
    return synth.bf16_bits_to_f32(u).astype(np.float64)


def _gamma(d):
    u = 2.0 ** -24
    return d * u / (1 - d * u)


def _abs_bounds(inp, cand_id):
    """sum_k |x_k w_k| for every output element, in the oracle's layout."""
    E, WA, WB, WH, h = (np.abs(_f64(inp[k])) for k in ("E", "W_A", "W_B", "W_H", "h"))
    ver = inp["verified"]
    B, L = cand_id.shape[:2]
    r = WA.shape[0]
    A = np.zeros((B, L, K, r))
    A[:, 0, 0] = E[ver] @ WA.T
    A[:, 1:] = E[cand_id[:, :-1]] @ WA.T
    Bm = E[cand_id] @ WB.T
    G = h @ WH.T
    return A, Bm, G


def _check(ora, dev, inp, cand_id):
    d = to_dev(inp, dev)
    A, Bm, G = ds.project(d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"],
                          torch.from_numpy(cand_id).to(dev), d["verified"])
    torch.cuda.synchronize()
    A, Bm, G = (x.cpu().numpy().astype(np.float64) for x in (A, Bm, G))
    rA, rB, rG = ora.project(inp["E"], inp["W_A"], inp["W_B"], inp["W_H"], inp["h"], cand_id,
                             inp["verified"])
    bA, bB, bG = _abs_bounds(inp, cand_id)
    dd = inp["E"].shape[1]
    g = _gamma(dd)
    assert np.all(np.abs(A - rA) <= g * bA + 1e-30), "A_prev beyond the fp32 accumulation bound"
    assert np.all(np.abs(Bm - rB) <= g * bB + 1e-30), "B_cur beyond the fp32 accumulation bound"
    # sigmoid is 1-Lipschitz/4 in its argument, plus a few ulp of its own
    assert np.all(np.abs(G - rG) <= 0.25 * g * bG + 8 * 2.0 ** -24), "G beyond bound"
    assert np.all(A[:, 0, 1:] == 0.0)
    assert ds.device_error() == 0
    return A, Bm, G


def _rand_inputs(seed, B, L, V, d, r, e_std=1.0):
    rng = np.random.default_rng(seed)
    inp = dict(
        E=synth.f32_to_bf16_bits(rng.standard_normal((V, d)).astype(np.float32) * e_std),
        W_A=synth.f32_to_bf16_bits(rng.standard_normal((r, d)).astype(np.float32) / np.sqrt(d)),
        W_B=synth.f32_to_bf16_bits(rng.standard_normal((r, d)).astype(np.float32) / np.sqrt(d)),
        W_H=synth.f32_to_bf16_bits(rng.standard_normal((r, d)).astype(np.float32) / np.sqrt(d)),
        h=synth.f32_to_bf16_bits(rng.standard_normal((B, L, d)).astype(np.float32)),
        verified=rng.integers(0, V, size=B).astype(np.int32),
        uniforms=np.zeros((B, L), np.float32),
        logits=np.zeros((B, L, 16), np.float32),
    )
    cand = np.stack([rng.permutation(V)[:K] for _ in range(B * L)]).reshape(B, L, K).astype(np.int32)
    return inp, cand


@pytest.mark.parametrize("B,L,V,d,r", [
    (1, 1, 64, 64, 32),       # one position: only the verified row and B rows
    (3, 5, 500, 128, 32),     # small-tile path, ragged row tiles
    (2, 16, 3000, 192, 64),
    (5, 8, 4000, 256, 128),   # big-tile path
    (9, 7, 20000, 320, 256),  # big-tile path, ragged M, several K steps
    (2, 3, 700, 448, 96),     # r = 96: three 32-column tiles, 7 K steps
    (4, 32, 5000, 256, 160),  # longest block, five 32-column tiles
    (6, 1, 1000, 512, 192),   # one position per block, three 64-column tiles
    (40, 16, 30000, 128, 256),  # 80 row tiles, gate split along K
    (70, 9, 9000, 640, 224),  # 79 row tiles (not a multiple of the 8 XCDs), 7 column tiles
    (1, 16, 20000, 2560, 256),  # one block: both GEMMs split along K (10 ways)
    (2, 8, 5000, 1024, 128),  # candidate GEMM split 4 ways
    (24, 16, 6000, 192, 256),  # 48 row tiles: 64-wide candidate tiles at r = 256 (9, 7: 32-wide; 40, 16: 128-wide)
])
def test_project_matches_oracle(ora, dev, B, L, V, d, r):
    inp, cand = _rand_inputs(B * 1000 + L, B, L, V, d, r)
    _check(ora, dev, inp, cand)


@pytest.mark.parametrize("B,L,V,d,r", [
    (3, 5, 500, 128, 32),
    (40, 16, 30000, 128, 256),  # 6 row tiles, one per workgroup
    (1, 16, 20000, 2560, 256),  # one block: 40 K steps in one workgroup
    (9, 7, 20000, 320, 256),
    (2, 3, 700, 448, 96),
])
def test_project_gate_overlap_matches_oracle(ora, dev, B, L, V, d, r):
    """The unsplit gate (dsel_project_gate_overlap) writes G and position 0's
    predecessor rows within the same fp32 bound, and nothing else of A_prev."""
    inp, cand = _rand_inputs(B * 1000 + L + 7, B, L, V, d, r)
    t = to_dev(inp, dev)
    A = torch.full((B, L, K, r), float("nan"), dtype=torch.float32, device=dev)
    G = torch.empty((B, L, r), dtype=torch.float32, device=dev)
    ds.project_gate_overlap(t["E"], t["W_A"], t["W_H"], t["h"], t["verified"], A, G)
    torch.cuda.synchronize()
    A, G = A.cpu().numpy().astype(np.float64), G.cpu().numpy().astype(np.float64)
    rA, _, rG = ora.project(inp["E"], inp["W_A"], inp["W_B"], inp["W_H"], inp["h"], cand, inp["verified"])
    bA, _, bG = _abs_bounds(inp, cand)
    g = _gamma(inp["E"].shape[1])
    assert np.all(np.abs(A[:, 0, 0] - rA[:, 0, 0]) <= g * bA[:, 0, 0] + 1e-30)
    assert np.all(A[:, 0, 1:] == 0.0)
    assert np.all(np.isnan(A[:, 1:])), "the gate wrote rows of positions >= 1"
    assert np.all(np.abs(G - rG) <= 0.25 * g * bG + 8 * 2.0 ** -24)
    assert ds.device_error() == 0


def test_project_exact_cases(ora, dev):
    """One-hot E rows with small-integer weights: every sum is exact, so the
    GPU must match bit for bit; a zero gate weight gives G = 1/2 exactly."""
    rng = np.random.default_rng(3)
    B, L, V, d, r = 4, 6, 300, 128, 128
    Ef = np.zeros((V, d), np.float32)
    Ef[np.arange(V), np.arange(V) % d] = 1.0
    inp = dict(E=synth.f32_to_bf16_bits(Ef),
               W_A=synth.f32_to_bf16_bits(rng.integers(-8, 9, (r, d)).astype(np.float32)),
               W_B=synth.f32_to_bf16_bits(rng.integers(-8, 9, (r, d)).astype(np.float32)),
               W_H=np.zeros((r, d), np.uint16),
               h=synth.f32_to_bf16_bits(rng.standard_normal((B, L, d)).astype(np.float32)),
               verified=rng.integers(0, V, size=B).astype(np.int32),
               uniforms=np.zeros((B, L), np.float32), logits=np.zeros((B, L, 16), np.float32))
    cand = np.stack([rng.permutation(V)[:K] for _ in range(B * L)]).reshape(B, L, K).astype(np.int32)
    A, Bm, G = _check(ora, dev, inp, cand)
    rA, rB, rG = ora.project(inp["E"], inp["W_A"], inp["W_B"], inp["W_H"], inp["h"], cand,
                             inp["verified"])
    assert np.array_equal(A, rA) and np.array_equal(Bm, rB) and np.all(G == 0.5)


def test_project_out_of_range_token_sets_error(dev):
    inp, cand = _rand_inputs(5, 2, 4, 100, 64, 32)
    cand[1, 2, 3] = 100   # == vocab
    inp["verified"][0] = -1
    d = to_dev(inp, dev)
    assert ds.device_error() == 0
    A, Bm, G = ds.project(d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"],
                          torch.from_numpy(cand).to(dev), d["verified"])
    assert ds.device_error() == 1
    assert ds.device_error() == 0  # reading clears it
    assert torch.all(Bm[1, 2, 3] == 0) and torch.all(A[1, 3, 3] == 0) and torch.all(A[0, 0, 0] == 0)


def test_project_empty_batch(dev):
    z = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((32, 64), dtype=torch.bfloat16, device=dev)
    A, Bm, G = ds.project(z, w, w, w, torch.zeros((0, 4, 64), dtype=torch.bfloat16, device=dev),
                          torch.zeros((0, 4, K), dtype=torch.int32, device=dev),
                          torch.zeros((0,), dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert A.shape == (0, 4, K, 32)


@pytest.mark.parametrize("name,nblocks", [("c2", 6), ("c3", 4), ("c4", 3)])
def test_project_workload_sampled_blocks(ora, dev, name, nblocks):
    """Full-size tables and weights; oracle candidates for a few blocks."""
    cfg = synth.CONFIGS[name]
    W_A, W_B, W_H = synth.make_weights(cfg)
    blocks = np.random.default_rng(11).choice(cfg.batch, size=nblocks, replace=False)
    logits = synth.make_logits(cfg, blocks=blocks)
    cand, _ = ora.select_topk(logits)
    inp = dict(E=synth.make_E(cfg), W_A=W_A, W_B=W_B, W_H=W_H, h=synth.make_h(cfg, blocks=blocks),
               verified=synth.make_verified(cfg)[blocks], uniforms=np.zeros((nblocks, cfg.block), np.float32),
               logits=np.zeros((nblocks, cfg.block, 16), np.float32))
    _check(ora, dev, inp, cand)
