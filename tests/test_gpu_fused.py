"""The fused route of dsel_select_path: candidate projections and pair term in
one kernel per tile of whole blocks and column group of the rank, the walk
adding the groups' partial tables.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: eq.
S_t scores every adjacent candidate pair in one parallel pass.)

Shapes are chosen so that the fused route runs (blocks of at most 16 positions
and at least 128 workgroups: ceil(batch / floor(16 / block)) tiles times r / CW
column groups); the tiny width keeps the oracle fast.  Uniform batches with
at least 512 tiles x group pairs (r / CW even, CW = 64) take the wide tile,
two groups per workgroup with 32-deep K steps; WIDE lists such shapes (their
ragged form runs the narrow tile and must give the same bits).  Every case checks the
oracle (exact top-16, |dS| and the stricter |dP| bound, walk with flags) and
that the fused route gives the same bits as the separate calls, with and
without the optional intermediates."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth
from helpers import check_scores, check_walk, to_dev

pytestmark = pytest.mark.gpu
K = 16


def _cw(r):
    return 64 if (r % 64 == 0 and r >= 128) else 32


def _fused_route(B, L, r):
    nb = 16 // L if L <= 16 else 0
    return nb > 0 and -(-B // nb) * (r // _cw(r)) >= 128


def _wide(B, L, r):
    nb = 16 // L
    return _cw(r) == 64 and (r // 64) % 2 == 0 and -(-B // nb) * (r // 128) >= 512


def _cfg(B, L, r, d=64, V=1024, e_std=1.0):
    return synth.CONFIGS["c0"].replace(batch=B, block=L, r=r, d=d, vocab=V, e_std=e_std)


def _path(d, mode, lens=None, want_AB=False, want_S=True):
    res = ds.select_path(d["logits"], d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"], mode=mode,
                         uniforms=d["uniforms"], want_S=want_S, want_q=True, want_AB=want_AB, block_len=lens)
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    return {k: v.cpu().numpy() for k, v in res.items()}


def _separate(d, mode, lens=None):
    B, L = d["h"].shape[:2]
    r = d["W_A"].shape[0]
    A = torch.empty((B, L, K, r), dtype=torch.float32, device=d["E"].device)
    Bc = torch.empty_like(A)
    G = torch.empty((B, L, r), dtype=torch.float32, device=A.device)
    ds.project_gate(d["E"], d["W_A"], d["W_H"], d["h"], d["verified"], A, G, block_len=lens)
    cid, cu = ds.select_topk(d["logits"], block_len=lens)
    ds.project_cand(d["E"], d["W_A"], d["W_B"], cid, A, Bc, block_len=lens)
    res = ds.score_pairs(cu, A, Bc, G, want_S=True, walk_mode=mode, cand_id=cid, uniforms=d["uniforms"],
                         want_q=True, block_len=lens)
    res.update(cand_id=cid, cand_u=cu, A_prev=A, B_cur=Bc, G=G)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def _bits_equal(a, b, keys, lens=None):
    for k in keys:
        x, y = a[k], b[k]
        if lens is not None:
            x = np.concatenate([x[i, :n] for i, n in enumerate(lens)])
            y = np.concatenate([y[i, :n] for i, n in enumerate(lens)])
        if x.dtype.kind == "f":
            x, y = x.view(np.uint32), y.view(np.uint32)
        np.testing.assert_array_equal(x, y, err_msg=k)


SHAPES = [  # (batch, block, r): tiles of 1, 2, 3 and 16 blocks, every column-group width
    (256, 8, 32), (64, 16, 256), (192, 5, 64), (2048, 1, 32), (96, 12, 128), (130, 16, 224), (136, 7, 96),
]
# the wide tile: blocks of 16 at r = 256; 3 blocks per tile at r = 128; 386 tiles (the grid
# rounds up to 392 for the XCD order) whose last holds one block of two
WIDE = [(256, 16, 256), (1536, 5, 128), (771, 8, 256)]


def test_wide_shapes_take_the_wide_tile():
    assert all(_fused_route(*s) and _wide(*s) for s in WIDE)
    assert not any(_wide(*s) for s in SHAPES)
    assert _wide(256, 16, 256) and not _wide(64, 16, 256) and not _wide(128, 8, 256)  # c4 / c2 / c3


@pytest.mark.parametrize("B,L,r", SHAPES + WIDE)
@pytest.mark.parametrize("mode", [0, 1])
def test_fused_route_against_oracle(ora, dev, B, L, r, mode):
    assert _fused_route(B, L, r)
    cfg = _cfg(B, L, r)
    inp = synth.make(cfg, seed=B + L + r)
    d = to_dev(inp, dev)
    g = _path(d, mode)
    ref = ora.run(inp, mode, 1.0)
    np.testing.assert_array_equal(g["cand_id"], ref["cand_id"])
    eps, tol, eps_p, tol_p = check_scores(g["S"], ref["S"], ref["cand_u"])
    flagged = check_walk(ora, g, ref["S"], g["S"], ref["cand_id"], mode, inp["uniforms"], 1.0, eps)
    print(f"  {B}x{L} r={r} mode={mode}: max|dS|={eps:.3g} (tol {tol:.3g}) max|dP|={eps_p:.3g} "
          f"(tol {tol_p:.3g}) flagged={flagged}", flush=True)
    assert flagged <= max(1, B * L // 500)


@pytest.mark.parametrize("B,L,r", SHAPES[:4] + [(64, 16, 256)] + WIDE)
def test_fused_route_equals_separate_calls(dev, B, L, r):
    """Same bits as dsel_select_topk + dsel_project_gate + dsel_project_cand +
    dsel_score_pairs, with the optional outputs asked for or not."""
    cfg = _cfg(B, L, r, e_std=0.5)
    d = to_dev(synth.make(cfg, seed=3 * B + r), dev)
    for mode in (0, 1):
        sep = _separate(d, mode)
        full = _path(d, mode, want_AB=True)
        _bits_equal(full, sep, ("cand_id", "cand_u", "A_prev", "B_cur", "G", "S", "path_tok", "path_slot",
                                "path_s", "q"))
        lean = _path(d, mode, want_AB=False)
        _bits_equal(lean, sep, ("cand_id", "cand_u", "S", "path_tok", "path_slot", "path_s", "q"))
        bare = _path(d, mode, want_S=False)
        _bits_equal(bare, sep, ("path_tok", "path_slot", "path_s", "q"))


@pytest.mark.parametrize("B,L,r", [(256, 8, 32), (64, 16, 256), (192, 5, 64)] + WIDE)
def test_fused_route_ragged(dev, B, L, r):
    """Ragged batches on the fused route: every block as alone at its own
    length (bits equal to the separate calls at every valid position)."""
    cfg = _cfg(B, L, r)
    d = to_dev(synth.make(cfg, seed=7), dev)
    lens_np = np.random.default_rng(B).integers(0, L + 1, size=B).astype(np.int32)
    lens_np[:3] = [0, L, 1]
    lens = torch.from_numpy(lens_np).to(dev)
    for mode in (0, 1):
        sep = _separate(d, mode, lens)
        got = _path(d, mode, lens, want_AB=True)
        _bits_equal(got, sep, ("cand_id", "A_prev", "B_cur", "G", "S", "path_slot", "path_s", "q"), lens_np)
        lean = _path(d, mode, lens)
        _bits_equal(lean, sep, ("S", "path_slot", "q"), lens_np)


@pytest.mark.parametrize("name,mode", [("c2", 0), ("c3", 1), ("c4", 1)])
def test_fused_route_workloads_equal_separate_calls(dev, name, mode):
    """The graded workloads (64 x 16, 128 x 8 and 256 x 16 positions, the
    last on the wide tile) run the fused route; the separate calls, pinned to
    the oracle elsewhere, give the same bits."""
    cfg = synth.CONFIGS[name]
    assert _fused_route(cfg.batch, cfg.block, cfg.r)
    d = to_dev(synth.make(cfg, seed=5), dev)
    sep = _separate(d, mode)
    got = _path(d, mode)
    _bits_equal(got, sep, ("cand_id", "S", "path_tok", "path_slot", "path_s", "q"))


@pytest.mark.parametrize("name,B,L,r,d,mode", [
    ("c1", 1, 16, 256, 2560, 0), ("c1", 2, 16, 256, 2560, 1), ("c0", 4, 8, 32, 64, 0), ("c0", 3, 1, 32, 64, 1),
    ("c0", 5, 3, 160, 128, 0), ("c0", 2, 16, 128, 64, 1), ("c0", 7, 9, 64, 192, 0)])
def test_project_pairs_and_walk_pairs_against_oracle(ora, dev, name, B, L, r, d, mode):
    """The two stages of the fused route as their own calls, at small batches
    (few workgroups).  Against the oracle: exact top-16, the score bounds and
    the walk; A_prev / B_cur within the fp32 accumulation bound
    gamma_d * sum |x w|.  (Here the separate calls split the candidate GEMM
    along d, which rounds differently, so the bits are compared only between
    the two ways of passing A(verified), and with and without S.)"""
    cfg = synth.CONFIGS[name].replace(batch=B, block=L, r=r, d=d, vocab=min(synth.CONFIGS[name].vocab, 4096))
    inp = synth.make(cfg, seed=B * L + r)
    d_ = to_dev(inp, dev)
    A = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
    G = torch.empty((B, L, r), dtype=torch.float32, device=dev)
    ds.project_gate(d_["E"], d_["W_A"], d_["W_H"], d_["h"], d_["verified"], A, G)
    cid, cu = ds.select_topk(d_["logits"])
    pp = ds.project_pairs(d_["E"], d_["W_A"], d_["W_B"], cid, G, A, ver_stride=L * K * r, want_AB=True)
    assert pp["partials"].shape == (B, L, ds.pair_groups(r), K, K)
    res = ds.walk_pairs(cu, pp["partials"], cid, mode=mode, uniforms=d_["uniforms"], want_S=True, want_q=True)
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    g = {k: v.cpu().numpy() for k, v in res.items()}
    g["cand_id"] = cid.cpu().numpy()
    ref = ora.run(inp, mode, 1.0)
    np.testing.assert_array_equal(g["cand_id"], ref["cand_id"])
    eps, tol, eps_p, tol_p = check_scores(g["S"], ref["S"], ref["cand_u"])
    flagged = check_walk(ora, g, ref["S"], g["S"], ref["cand_id"], mode, inp["uniforms"], 1.0, eps)
    assert flagged <= 1
    # A_prev (positions >= 1) and B_cur within the fp32 accumulation bound
    rA, rB, _ = ora.project(inp["E"], inp["W_A"], inp["W_B"], inp["W_H"], inp["h"], ref["cand_id"],
                            inp["verified"])
    E = np.abs(synth.bf16_bits_to_f32(inp["E"]).astype(np.float64))
    WA = np.abs(synth.bf16_bits_to_f32(inp["W_A"]).astype(np.float64))
    WB = np.abs(synth.bf16_bits_to_f32(inp["W_B"]).astype(np.float64))
    gam = d * 2.0 ** -24 / (1 - d * 2.0 ** -24)
    Ag = pp["A_prev"].cpu().numpy().astype(np.float64)[:, 1:]
    Bg = pp["B_cur"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Ag - rA[:, 1:]) <= gam * (E[ref["cand_id"][:, :-1]] @ WA.T) + 1e-30)
    assert np.all(np.abs(Bg - rB) <= gam * (E[ref["cand_id"]] @ WB.T) + 1e-30)
    # compact A(verified) [B, r] and no S: the same partials, the same walk
    Av = A[:, 0, 0].contiguous()
    pp2 = ds.project_pairs(d_["E"], d_["W_A"], d_["W_B"], cid, G, Av)
    res2 = ds.walk_pairs(cu, pp2["partials"], cid, mode=mode, uniforms=d_["uniforms"], want_q=True)
    torch.cuda.synchronize()
    assert torch.equal(pp2["partials"].view(torch.int32), pp["partials"].view(torch.int32))
    _bits_equal({k: v.cpu().numpy() for k, v in res2.items()}, g, ("path_slot", "path_s", "q"))
