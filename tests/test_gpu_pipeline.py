"""The whole selector on the GPU, end to end, against the oracle.

Matching rules: top-16 ids and values bit-exact; pair scores within
2e-3 * max|S| (and the pair term P = S - U within 2e-3 * max|P|); walk paths
bit-exact except at steps whose top-2 gap / CDF margin is within the observed
score error, which are flagged and counted (the walk is then teacher-forced
along the GPU's path).  Full workloads compare every block's top-16 and a
sample of blocks' scores and walks."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth
from helpers import check_scores, check_walk, stutter_inputs, sub_inputs, to_dev

pytestmark = pytest.mark.gpu
K = 16

_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        _CACHE.clear()  # keep one big workload in host memory at a time
        _CACHE[name] = synth.make(synth.CONFIGS[name])
    return _CACHE[name]


def _run(inp, dev, mode, T=1.0, want_AB=False):
    d = to_dev(inp, dev)
    res = ds.select_path(d["logits"], d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"],
                         mode=mode, temperature=T, uniforms=d["uniforms"], want_S=True, want_q=True,
                         want_AB=want_AB)
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    return {k: v.cpu().numpy() for k, v in res.items()}


def _compare(ora, gpu, inp, mode, blocks, T=1.0):
    sub = sub_inputs(inp, blocks)
    ref = ora.run(sub, mode, T)
    g = {k: (v[blocks] if v.ndim >= 2 and v.shape[0] == inp["logits"].shape[0] else v)
         for k, v in gpu.items()}
    np.testing.assert_array_equal(g["cand_id"], ref["cand_id"])
    np.testing.assert_array_equal(g["cand_u"].view(np.uint32), ref["cand_u"].view(np.uint32))
    eps, tol, eps_p, tol_p = check_scores(g["S"], ref["S"], ref["cand_u"])
    flagged = check_walk(ora, g, ref["S"], g["S"], ref["cand_id"], mode, sub["uniforms"], T, eps)
    print(f"  blocks={len(blocks)} mode={mode} max|dS|={eps:.3g} (tol {tol:.3g}) "
          f"max|dP|={eps_p:.3g} (tol {tol_p:.3g}) flagged steps={flagged}", flush=True)
    return flagged


def test_stutter_example_on_gpu(dev):
    """The hand-worked example, padded to d = 64 and r = 32 with zeros (the
    padding adds nothing to any dot product)."""
    inp, exp = stutter_inputs()
    pad = dict(inp)
    V, d0 = 16, 16
    E = np.zeros((V, 64), np.float32)
    E[:, :d0] = np.eye(V, d0)
    WA = np.zeros((32, 64), np.float32)
    WA[:d0, :d0] = -4.0 * np.eye(d0)
    WB = np.zeros((32, 64), np.float32)
    WB[:d0, :d0] = np.eye(d0)
    pad.update(E=synth.f32_to_bf16_bits(E), W_A=synth.f32_to_bf16_bits(WA),
               W_B=synth.f32_to_bf16_bits(WB), W_H=np.zeros((32, 64), np.uint16),
               h=np.zeros((1, 3, 64), np.uint16))
    g = _run(pad, dev, 0)
    np.testing.assert_array_equal(g["cand_id"][0], np.array(exp["cand_id"]))
    np.testing.assert_array_equal(g["S"][0, 0, 0], exp["S_row0_t0"])
    np.testing.assert_array_equal(g["S"][0, 1, 1], exp["S_row1_t1"])
    np.testing.assert_array_equal(g["S"][0, 2, 1], exp["S_row1_t2"])
    np.testing.assert_array_equal(g["path_tok"][0], exp["path_tok"])
    np.testing.assert_array_equal(g["path_slot"][0], exp["path_slot"])
    np.testing.assert_array_equal(g["path_s"][0], exp["path_s"])


@pytest.mark.parametrize("mode", [0, 1])
def test_tiny_workload(ora, dev, mode):
    inp = _workload("c0")
    g = _run(inp, dev, mode)
    _compare(ora, g, inp, mode, np.arange(inp["logits"].shape[0]))


@pytest.mark.parametrize("name,mode,nblocks", [
    ("c1", 0, 1), ("c2", 0, 64), ("c3", 1, 24), ("c4", 0, 8), ("c4", 1, 8)])
def test_workloads(ora, dev, name, mode, nblocks):
    inp = _workload(name)
    cfg = synth.CONFIGS[name]
    g = _run(inp, dev, mode)
    rid, _ = ora.select_topk(inp["logits"])  # every block's top-16
    np.testing.assert_array_equal(g["cand_id"], rid)
    blocks = np.sort(np.random.default_rng(5).choice(cfg.batch, size=nblocks, replace=False))
    _compare(ora, g, inp, mode, blocks)


def test_zero_pair_weight_gives_top1_path(dev):
    """W_A = 0: the selector reduces to the per-position top-1 (the one-pass
    drafter's own pick)."""
    inp = dict(_workload("c1"))
    inp["W_A"] = np.zeros_like(inp["W_A"])
    g = _run(inp, dev, 0)
    assert np.all(g["path_slot"] == 0)
    x = inp["logits"]
    top1 = np.argmax(synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x, axis=-1)
    np.testing.assert_array_equal(g["path_tok"], top1)


def test_strong_pair_stress(ora, dev):
    """Embeddings with std 1 make the pair term dominate, so the walk leaves
    the top-1 path often; shapes of the one-block latency workload."""
    cfg = synth.CONFIGS["c1"].replace(e_std=1.0, batch=4)
    inp = synth.make(cfg)
    g = _run(inp, dev, 0)
    flagged = _compare(ora, g, inp, 0, np.arange(cfg.batch))
    assert np.mean(g["path_slot"] != 0) > 0.2
    assert flagged <= 2


def test_tie_heavy_stress(ora, dev):
    cfg = synth.CONFIGS["c0"].replace(batch=6, block=16, vocab=4096, d=128, r=64)
    inp = synth.make(cfg)
    rng = np.random.default_rng(2)
    inp["logits"] = (rng.integers(0, 17, size=inp["logits"].shape) * 0.25).astype(np.float32)
    for mode in (0, 1):
        g = _run(inp, dev, mode)
        _compare(ora, g, inp, mode, np.arange(cfg.batch))


def test_pipeline_is_deterministic(dev):
    inp = _workload("c2")
    a = _run(inp, dev, 0, want_AB=True)
    b = _run(inp, dev, 0, want_AB=True)
    for k in ("cand_id", "path_slot", "path_tok"):
        assert np.array_equal(a[k], b[k])
    for k in ("S", "A_prev", "B_cur", "G", "q"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
