"""dsel_select_path (the whole selector in one call) against the separate calls.

Same kernels, same order, same arithmetic: every output must come out bit for
bit as from dsel_select_topk, dsel_project_gate, dsel_project_cand and
dsel_score_pairs called one after the other (which the other GPU tests pin to
the oracle).  Shapes cover the gate split (reduction inside the top-16 launch),
split top-16 rows (merge kernel), the unsplit gate of large batches, ragged
batches and both walks."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth
from helpers import to_dev

pytestmark = pytest.mark.gpu
K = 16
KEYS = ("cand_id", "cand_u", "A_prev", "B_cur", "G", "S", "path_tok", "path_slot", "path_s", "q")


def _separate(d, mode, lens, T=1.0):
    B, L = d["h"].shape[:2]
    r = d["W_A"].shape[0]
    dev = d["E"].device
    A = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
    Bc = torch.empty_like(A)
    G = torch.empty((B, L, r), dtype=torch.float32, device=dev)
    ds.project_gate(d["E"], d["W_A"], d["W_H"], d["h"], d["verified"], A, G, block_len=lens)
    cid, cu = ds.select_topk(d["logits"], block_len=lens)
    ds.project_cand(d["E"], d["W_A"], d["W_B"], cid, A, Bc, block_len=lens)
    res = ds.score_pairs(cu, A, Bc, G, want_S=True, walk_mode=mode, cand_id=cid, temperature=T,
                         uniforms=d["uniforms"], want_q=True, block_len=lens)
    res.update(cand_id=cid, cand_u=cu, A_prev=A, B_cur=Bc, G=G)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def _fused(d, mode, lens, T=1.0):
    res = ds.select_path(d["logits"], d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"], mode=mode,
                         temperature=T, uniforms=d["uniforms"], want_S=True, want_q=True, want_AB=True,
                         block_len=lens)
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    return {k: v.cpu().numpy() for k, v in res.items()}


def _small(d, mode, lens, T=1.0):
    res = ds.select_path(d["logits"], d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"], mode=mode,
                         temperature=T, uniforms=d["uniforms"], want_S=True, want_q=True, block_len=lens)
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    return {k: v.cpu().numpy() for k, v in res.items()}


def _equal(a, b, lens, L, keys=KEYS):
    n_of = [L] * a["cand_id"].shape[0] if lens is None else lens
    for k in keys:
        for blk, n in enumerate(n_of):
            x, y = a[k][blk, :n], b[k][blk, :n]
            if x.dtype.kind == "f":
                x, y = x.view(np.uint32), y.view(np.uint32)
            np.testing.assert_array_equal(x, y, err_msg=f"{k} block {blk}")


@pytest.mark.parametrize("name,mode,ragged", [
    ("c0", 0, False), ("c0", 1, True), ("c1", 0, False), ("c1", 1, False),
    ("c2", 0, False), ("c2", 0, True), ("c3", 1, False), ("c3", 1, True)])
def test_path_equals_separate_calls(dev, name, mode, ragged):
    cfg = synth.CONFIGS[name]
    d = to_dev(synth.make(cfg, seed=11), dev)
    lens_np = synth.make_block_len(cfg, seed=11) if ragged else None
    if ragged and name == "c0":
        lens_np = np.array([0, 8, 3, 5], np.int32)
    lens = None if lens_np is None else torch.from_numpy(lens_np).to(dev)
    a = _fused(d, mode, lens)
    b = _separate(d, mode, lens)
    _equal(a, b, None if lens_np is None else lens_np, cfg.block)


SMALL_CASES = {
    # one block of 16 (the latency shape), both walks
    "c1": (synth.CONFIGS["c1"], None),
    # four blocks of 8, one empty and one short
    "c1x4": (synth.CONFIGS["c1"].replace(batch=4, block=8), [8, 5, 0, 3]),
    # two blocks at lengths of the 5 / 8 / 16 mix (the top-16 rows split fewer ways)
    "c1x2": (synth.CONFIGS["c1"].replace(batch=2), [8, 5]),
    # blocks of 8 at d 5120, sampled
    "c3x4": (synth.CONFIGS["c3"].replace(batch=4), None),
    # rank 96: groups of 32 columns, 32-wide candidate tiles
    "r96": (synth.CONFIGS["c1"].replace(batch=2, r=96), None),
    # fp32 logits
    "f32": (synth.CONFIGS["c1"].replace(batch=2, logits_dtype="f32"), None),
    # the longest block (32 positions) at rank 160: five groups of 32 columns
    "L32r160": (synth.CONFIGS["c1"].replace(batch=1, block=32, r=160), [29]),
    # blocks of one position: every step starts from the verified token
    "L1": (synth.CONFIGS["c1"].replace(batch=32, block=1), None),
}


@pytest.mark.parametrize("case,mode", [("c1", 0), ("c1", 1), ("c1x4", 0), ("c1x2", 1), ("c3x4", 1), ("r96", 0),
                                       ("f32", 1), ("L32r160", 1), ("L1", 0)])
def test_small_batch_route_equals_separate_calls(dev, case, mode):
    """The three-launch route of small batches (top-16 beside the gate GEMM;
    candidate GEMM with the list merge; split sums, pair tables and the walk
    by each block's last workgroup): the bits of the separate calls."""
    cfg, lens_spec = SMALL_CASES[case]
    dt = torch.bfloat16 if cfg.logits_dtype == "bf16" else torch.float32
    assert ds.select_path_route(cfg.batch, cfg.block, cfg.vocab, dt, cfg.d, cfg.r) == ds.ROUTE_SMALL
    d = to_dev(synth.make(cfg, seed=21), dev)
    if lens_spec == "mix":
        lens_np = synth.make_block_len(cfg, seed=21)
    else:
        lens_np = None if lens_spec is None else np.asarray(lens_spec, np.int32)
    lens = None if lens_np is None else torch.from_numpy(lens_np).to(dev)
    for rep in range(2):  # the arrival counters start from zero on every call
        a = _small(d, mode, lens)
        b = _separate(d, mode, lens)
        _equal(a, b, lens_np, cfg.block,
               keys=("cand_id", "cand_u", "S", "path_tok", "path_slot", "path_s", "q"))


def test_path_large_batch_unsplit_gate(dev):
    """256 blocks of 16 at d 2560: the gate GEMM needs no split, so nothing
    rides in the top-16 launch."""
    cfg = synth.CONFIGS["c2"].replace(batch=256)
    d = to_dev(synth.make(cfg, seed=12), dev)
    assert ds.lib().dsel_project_workspace_bytes(256, 16, 2560, 256) >= 0
    _equal(_fused(d, 0, None), _separate(d, 0, None), None, cfg.block)


def test_path_with_padded_logit_rows(dev):
    """bf16 logit rows padded past the vocabulary (ld > vocab) and E with more
    rows than the vocabulary in use: the same bits as the separate calls."""
    cfg = synth.CONFIGS["c1"].replace(batch=3, vocab=150000)
    inp = synth.make(cfg, seed=14)
    d = to_dev(inp, dev)
    V, ld = 149000, 150016
    wide = torch.full((cfg.batch, cfg.block, ld), -3.0e38, dtype=torch.bfloat16, device=dev)
    wide[..., :V] = d["logits"][..., :V]
    d["logits"] = wide
    a = ds.select_path(wide, d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"], vocab=V, want_S=True,
                       want_q=True, uniforms=d["uniforms"])
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    cid, cu = ds.select_topk(wide, vocab=V)
    assert torch.equal(a["cand_id"], cid) and torch.equal(a["cand_u"].view(torch.int32), cu.view(torch.int32))
    assert int(a["cand_id"].max()) < V
