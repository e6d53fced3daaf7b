"""lmhead_topk on the GPU against the oracle.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: the
candidates are the drafter's own 16 best logits, with no extra LM-head
forward.)

The GPU orders fp32 logits from bf16 MFMA products (exact) summed in the
hardware's order, each within e_v = gamma_d * sum_k |h_k W_vk| of the fp64
logit (gamma_d = d u / (1 - d u), u = 2^-24).  The oracle orders fp64 logits.
So a row's 16 ids must equal the oracle's exactly unless the boundary between
the 16th and 17th is within that error band; such rows are counted, and the
GPU's list must still be valid: every returned logit within e_v of its fp64
value, every left-out oracle candidate no better than the GPU's 16th by more
than the band, and the list sorted by its own values (ties to the lower id)."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth

pytestmark = pytest.mark.gpu
K = 16
U = 2.0 ** -24


def _dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def _f(u):
    return synth.bf16_bits_to_f32(u).astype(np.float64)


def check_lmhead(ora, h, W, cid_gpu, cu_gpu, rows=None):
    """Compare the rows `rows` (default all); returns the number of flagged rows."""
    rows = np.arange(h.shape[0]) if rows is None else np.asarray(rows)
    hs = h[rows]
    cid, cz = ora.lmhead_topk(hs, W)
    d = h.shape[1]
    gam = d * U / (1 - d * U)
    Hf, Wf = _f(hs), _f(W)
    flagged = 0
    for i, r in enumerate(rows):
        g_id, g_u = cid_gpu[r], cu_gpu[r].astype(np.float64)
        assert len(set(g_id.tolist())) == K and g_id.min() >= 0 and g_id.max() < W.shape[0]
        # its own order: value descending, ties to the lower id
        for j in range(K - 1):
            assert g_u[j] > g_u[j + 1] or (g_u[j] == g_u[j + 1] and g_id[j] < g_id[j + 1])
        z64 = Wf[g_id] @ Hf[i]
        e = gam * (np.abs(Wf[g_id]) @ np.abs(Hf[i]))
        assert np.all(np.abs(g_u - z64) <= e + 1e-30), f"row {r}: logit beyond the fp32 bound"
        if np.array_equal(g_id, cid[i]):
            continue
        emax = gam * np.max(np.abs(Wf) @ np.abs(Hf[i]))
        # a disagreement must sit inside the error band of the 16 / 17 boundary
        assert cz[i, K - 1] - cz[i, K] <= 4 * emax, f"row {r}: ids differ away from a near-tie"
        assert np.min(z64) >= cz[i, K - 1] - 2 * emax, f"row {r}: a returned id is too far down"
        flagged += 1
    return flagged


def _rand(seed, R, V, d):
    rng = np.random.default_rng(seed)
    h = synth.f32_to_bf16_bits(rng.standard_normal((R, d)).astype(np.float32))
    W = synth.f32_to_bf16_bits((rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32))
    return h, W


@pytest.mark.parametrize("R,V,d", [
    (5, 300, 64),        # one ragged vocab tile per split
    (130, 2000, 128),    # two row tiles, the second with 2 rows
    (64, 5000, 256),
    (16, 151936, 2560),  # one block of 16 positions, full vocabulary
])
def test_lmhead_matches_oracle(ora, dev, R, V, d):
    h, W = _rand(R + V + d, R, V, d)
    cid, cu = ds.lmhead_topk(_dev(h, dev), _dev(W, dev))
    torch.cuda.synchronize()
    flagged = check_lmhead(ora, h, W, cid.cpu().numpy(), cu.cpu().numpy())
    assert flagged <= max(1, R // 20)


def test_lmhead_workload_sampled_rows(ora, dev):
    """64 blocks x 16 positions at d 2560 against E (tied embeddings): all rows
    on the GPU, a sample of rows in the oracle."""
    cfg = synth.CONFIGS["c2"]
    E = synth.make_E(cfg)
    h = synth.make_h(cfg).reshape(cfg.batch * cfg.block, cfg.d)
    cid, cu = ds.lmhead_topk(_dev(h, dev), _dev(E, dev))
    torch.cuda.synchronize()
    rows = [0, 1, 15, 16, 511, 777, 1023]
    flagged = check_lmhead(ora, h, E, cid.cpu().numpy(), cu.cpu().numpy(), rows)
    assert flagged <= 1


def test_lmhead_largest_workload_sampled_rows(ora, dev):
    """256 blocks x 16 positions at d 6144 against a vocabulary of 202,048 (the
    largest workload, 10 TFLOP): all 4,096 rows on the GPU in one call, six of
    them in the oracle."""
    cfg = synth.CONFIGS["c4"]
    E = synth.make_E(cfg)
    h = synth.make_h(cfg).reshape(cfg.batch * cfg.block, cfg.d)
    Ed = _dev(E, dev)
    cid, cu = ds.lmhead_topk(_dev(h, dev), Ed)
    torch.cuda.synchronize()
    del Ed
    rows = [0, 1, 1234, 2047, 3000, 4095]
    flagged = check_lmhead(ora, h, E, cid.cpu().numpy(), cu.cpu().numpy(), rows)
    assert flagged <= 1


def test_lmhead_ties_and_equals_select_topk_on_the_same_logits(dev):
    """Integer inputs make every logit exact in fp32: the fused result must then
    equal dsel_select_topk over the materialised logits, bit for bit."""
    rng = np.random.default_rng(9)
    R, V, d = 40, 3000, 64
    h = synth.f32_to_bf16_bits(rng.integers(-2, 3, (R, d)).astype(np.float32))
    W = synth.f32_to_bf16_bits(rng.integers(-2, 3, (V, d)).astype(np.float32))
    cid, cu = ds.lmhead_topk(_dev(h, dev), _dev(W, dev))
    z = (_f(h) @ _f(W).T).astype(np.float32)
    rid, ru = ds.select_topk(torch.from_numpy(z[None]).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(cid.cpu().numpy(), rid[0].cpu().numpy())
    assert np.array_equal(cu.cpu().numpy(), ru[0].cpu().numpy())


def test_lmhead_empty_and_deterministic(dev):
    h, W = _rand(3, 33, 1000, 128)
    a = ds.lmhead_topk(_dev(h, dev), _dev(W, dev))
    b = ds.lmhead_topk(_dev(h, dev), _dev(W, dev))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    e = ds.lmhead_topk(_dev(h[:0], dev), _dev(W, dev))
    assert e[0].shape == (0, K)
