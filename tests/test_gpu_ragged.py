"""Ragged batches on the GPU: a length per block in the padded layout.

(Block size is a per-request knob: "DFlash 2: Keep Drafting Parallel",
supplementary deployment notes; "DFlash 2: The Drafter Stopped Guessing
Alone", "What to check on your own serving".)

Three rules, each checked through the C ABI:
  * parity: every valid position matches the oracle run on its block alone at
    its own length, under the rules of the uniform tests (top-16 bit-exact,
    scores within 2e-3 max|S|, walks and verification exact up to flagged
    near-ties, convolution within its derived bound);
  * same bits: a valid position comes out bit for bit as in the uniform batch
    (no kernel's arithmetic for a position depends on its block's length);
  * padding: outputs there are never written (sentinels survive) and inputs
    there never matter (NaN padding gives the same bits)."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth
from helpers import check_scores, check_walk, to_dev
from test_gpu_conv import _bound as conv_bound
from test_gpu_conv import _dev as conv_dev
from test_gpu_conv import _rand as conv_rand
from test_gpu_verify import _dev_logits, _random_case, check_verify

pytestmark = pytest.mark.gpu
K = 16


def _lens_dev(lens, dev):
    return torch.from_numpy(np.ascontiguousarray(lens, np.int32)).to(dev)


def _select(d, mode, lens, T=1.0):
    res = ds.select_path(d["logits"], d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"], mode=mode,
                         temperature=T, uniforms=d["uniforms"], want_S=True, want_q=True, want_AB=True,
                         block_len=lens)
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    return {k: v.cpu().numpy() for k, v in res.items()}


def _valid_equal(a, b, lens, keys):
    for k in keys:
        for blk, n in enumerate(lens):
            x, y = a[k][blk, :n], b[k][blk, :n]
            if x.dtype.kind == "f":
                x, y = x.view(np.uint32), y.view(np.uint32)
            np.testing.assert_array_equal(x, y, err_msg=f"{k} block {blk}")


KEYS = ("cand_id", "cand_u", "A_prev", "B_cur", "G", "S", "path_tok", "path_slot", "path_s", "q")


@pytest.mark.parametrize("name,mode,lens", [
    ("c0", 0, [0, 1, 2, 3, 5, 8, 8, 4, 7, 6, 1, 0]),
    ("c0", 1, [8, 0, 3, 1, 6, 2, 5, 8, 4, 7, 2, 3]),
    ("c1", 0, [16, 0, 5, 8, 1, 11]),
])
def test_ragged_selector_matches_oracle(ora, dev, name, mode, lens):
    cfg = synth.CONFIGS[name].replace(batch=len(lens))
    inp = synth.make(cfg, seed=21)
    lens = np.array(lens, np.int32)
    g = _select(to_dev(inp, dev), mode, _lens_dev(lens, dev))
    ref = ora.run_ragged(inp, lens, mode)
    flagged = 0
    for b, n in enumerate(lens):
        if n == 0:
            continue
        sl = lambda a: a[b:b + 1, :n]
        gb = {k: sl(v) for k, v in g.items()}
        np.testing.assert_array_equal(gb["cand_id"], sl(ref["cand_id"]))
        np.testing.assert_array_equal(gb["cand_u"].view(np.uint32), sl(ref["cand_u"]).view(np.uint32))
        eps, _, _, _ = check_scores(gb["S"], sl(ref["S"]), sl(ref["cand_u"]))
        flagged += check_walk(ora, gb, sl(ref["S"]), gb["S"], sl(ref["cand_id"]), mode,
                              sl(inp["uniforms"]), 1.0, eps)
    assert flagged <= 1


@pytest.mark.parametrize("name,mode", [("c2", 0), ("c3", 1)])
def test_ragged_is_bitwise_the_uniform_batch(dev, name, mode):
    """The full workload shapes with the 5 / 8 / 16 mix: every valid position
    equals the uniform batch bit for bit (which the uniform tests pin to the
    oracle)."""
    cfg = synth.CONFIGS[name]
    d = to_dev(synth.make(cfg), dev)
    lens = synth.make_block_len(cfg)
    print(f"  {name}: {int(lens.sum())} of {cfg.rows} positions", flush=True)
    uni = _select(d, mode, None)
    rag = _select(d, mode, _lens_dev(lens, dev))
    _valid_equal(rag, uni, lens, KEYS)


def test_ragged_many_blocks_bitwise_the_uniform_batch(dev):
    """4,500 blocks of 2 positions (lengths 0, 1 or 2): more than 64 blocks per
    lane in the compaction scan of the top-16 (its second level runs twice), and
    thousands of blocks packed into the fused projection's tiles by length
    class; every valid position equals the uniform batch bit for bit."""
    cfg = synth.CONFIGS["c0"].replace(batch=4500, block=2)
    d = to_dev(synth.make(cfg, seed=23), dev)
    lens = np.random.default_rng(23).integers(0, 3, size=cfg.batch).astype(np.int32)
    uni = _select(d, 0, None)
    rag = _select(d, 0, _lens_dev(lens, dev))
    _valid_equal(rag, uni, lens, KEYS)


def test_ragged_wide_batch_bitwise_the_uniform_batch(dev):
    """256 blocks of 16 at r = 256: the uniform batch runs the fused
    projection's wide tile (two rank groups per workgroup, 32-deep K steps),
    the ragged batch the narrow tile (one group, 64-deep steps); every valid
    position has the same bits."""
    cfg = synth.CONFIGS["c0"].replace(batch=256, block=16, r=256, d=128, vocab=2048)
    d = to_dev(synth.make(cfg, seed=29), dev)
    lens = np.random.default_rng(29).integers(0, 17, size=cfg.batch).astype(np.int32)
    uni = _select(d, 0, None)
    rag = _select(d, 0, _lens_dev(lens, dev))
    _valid_equal(rag, uni, lens, KEYS)


def test_padding_is_never_read(dev):
    cfg = synth.CONFIGS["c1"].replace(batch=5)
    inp = synth.make(cfg, seed=3)
    lens = np.array([3, 16, 0, 9, 1], np.int32)
    dirty = dict(inp)
    lg, h, u = inp["logits"].copy(), inp["h"].copy(), inp["uniforms"].copy()
    for b, n in enumerate(lens):
        lg[b, n:] = 0x7FC0        # bf16 NaN
        h[b, n:] = 0x7F7F         # bf16 3.4e38
        u[b, n:] = np.float32(np.nan)
    dirty.update(logits=lg, h=h, uniforms=u)
    L = _lens_dev(lens, dev)
    for mode in (0, 1):
        a = _select(to_dev(inp, dev), mode, L)
        b = _select(to_dev(dirty, dev), mode, L)
        _valid_equal(a, b, lens, KEYS)


def test_padding_is_never_written(dev):
    """Every output buffer starts as a sentinel; padding positions keep it."""
    cfg = synth.CONFIGS["c0"].replace(batch=6)
    inp = synth.make(cfg, seed=4)
    d = to_dev(inp, dev)
    lens_np = np.array([0, 8, 3, 1, 5, 7], np.int32)
    lens = _lens_dev(lens_np, dev)
    B, L, r = cfg.batch, cfg.block, cfg.r
    SI, SF = -7, -1.25
    cid = torch.full((B, L, K), SI, dtype=torch.int32, device=dev)
    cu = torch.full((B, L, K), SF, dtype=torch.float32, device=dev)
    ds.select_topk(d["logits"], out=(cid, cu), block_len=lens)
    A = torch.full((B, L, K, r), SF, dtype=torch.float32, device=dev)
    Bc = torch.full((B, L, K, r), SF, dtype=torch.float32, device=dev)
    G = torch.full((B, L, r), SF, dtype=torch.float32, device=dev)
    ds.project_gate(d["E"], d["W_A"], d["W_H"], d["h"], d["verified"], A, G, block_len=lens)
    ds.project_cand(d["E"], d["W_A"], d["W_B"], cid, A, Bc, block_len=lens)
    S = torch.full((B, L, K, K), SF, dtype=torch.float32, device=dev)
    wa, wres = ds._walk_args(cid, ds.SAMPLED, 1.0, d["uniforms"], True, True)
    for t in wres.values():
        t.fill_(SI if t.dtype == torch.int32 else SF)
    st = ds.lib().dsel_score_pairs(ds._ptr(cu), ds._ptr(A), ds._ptr(Bc), ds._ptr(G), B, L, ds._ptr(lens), r,
                                   ds._ptr(S), torch_byref(wa), ds._stream())
    assert st == 0
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    outs = dict(cand_id=cid, cand_u=cu, A_prev=A, B_cur=Bc, G=G, S=S, **wres)
    for k, t in outs.items():
        a = t.cpu().numpy()
        for b, n in enumerate(lens_np):
            pad = a[b, n:]
            want = SI if a.dtype == np.int32 else SF
            assert np.all(pad == want), f"{k}: padding of block {b} written"
            assert not np.any(a[b, :n] == want), f"{k}: valid part of block {b} unwritten"


def torch_byref(wa):
    import ctypes as C

    return C.byref(wa)


@pytest.mark.parametrize("dtype,mode", [("f32", 0), ("bf16", 0), ("f32", 1), ("bf16", 1)])
def test_ragged_verify_matches_oracle(ora, dev, dtype, mode):
    B, L, V, T = 24, 8, 3000, 0.9
    tl, cand, slots, q, ua, ur = _random_case(40 + mode, B, L, V, dtype, T)
    lens = np.random.default_rng(41).integers(0, L + 1, size=B).astype(np.int32)
    lens[:3] = [0, L, 1]
    n, tok = ds.verify(_dev_logits(tl, dev), torch.from_numpy(cand).to(dev), torch.from_numpy(slots).to(dev),
                       torch.from_numpy(q).to(dev) if mode else None, mode=mode, temperature=T,
                       u_acc=torch.from_numpy(ua).to(dev) if mode else None,
                       u_res=torch.from_numpy(ur).to(dev) if mode else None, block_len=_lens_dev(lens, dev))
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    n, tok = n.cpu().numpy(), tok.cpu().numpy()
    flagged = 0
    for b, nb in enumerate(lens):
        # block b alone at its own length: rows 0 .. nb of its target logits
        flagged += check_verify(ora, np.ascontiguousarray(tl[b:b + 1, :nb + 1]), cand[b:b + 1, :nb],
                                slots[b:b + 1, :nb], q[b:b + 1, :nb], mode, T, ua[b:b + 1, :nb], ur[b:b + 1],
                                n[b:b + 1], tok[b:b + 1, :nb + 1])
        assert n[b] <= nb and np.all(tok[b, nb + 1:] == -1)
    assert flagged <= 1


def test_ragged_conv(ora, dev):
    B, L, d = 7, 16, 1024
    inp = conv_rand(9, B, L, d)
    lens = np.array([0, 16, 1, 5, 8, 13, 2], np.int32)
    t = {k: conv_dev(v, dev) for k, v in inp.items()}
    y_uni = ds.dyn_conv(t["x"], t["x_prev"], t["base"], t["W_c"])
    y = torch.full_like(t["x"], 5.0)  # sentinel
    ds.dyn_conv(t["x"], t["x_prev"], t["base"], t["W_c"], y=y, block_len=_lens_dev(lens, dev))
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    yu = y_uni.view(torch.int16).cpu().numpy().view(np.uint16)
    yr = y.view(torch.int16).cpu().numpy().view(np.uint16)
    five = synth.f32_to_bf16_bits(np.float32(5.0))
    ref, corr = ora.dyn_conv_ragged(inp["x"], inp["x_prev"], inp["base"], inp["W_c"], lens)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(yr[b, :n], yu[b, :n])
        assert np.all(yr[b, n:] == five)
        if n:
            sub = {k: (v[b:b + 1, :n] if k == "x" else v[b:b + 1] if k == "x_prev" else v) for k, v in inp.items()}
            got = synth.bf16_bits_to_f32(yr[b:b + 1, :n]).astype(np.float64)
            bnd = conv_bound(sub, ref[b:b + 1, :n], corr[b:b + 1, :n])
            assert np.all(np.abs(got - ref[b:b + 1, :n]) <= bnd)


def test_bad_lengths_flag_and_empty_the_block(dev):
    cfg = synth.CONFIGS["c0"].replace(batch=4)
    inp = synth.make(cfg, seed=6)
    d = to_dev(inp, dev)
    B, L = cfg.batch, cfg.block
    cid = torch.full((B, L, K), -7, dtype=torch.int32, device=dev)
    cu = torch.full((B, L, K), -1.25, dtype=torch.float32, device=dev)
    lens = np.array([3, -1, L + 1, L], np.int32)
    ds.select_topk(d["logits"], out=(cid, cu), block_len=_lens_dev(lens, dev))
    assert ds.device_error() == 2  # DSEL_DEVERR_BLOCK_LEN, and the word is cleared
    assert ds.device_error() == 0
    c = cid.cpu().numpy()
    assert np.all(c[1] == -7) and np.all(c[2] == -7)  # treated as empty
    assert np.all(c[0, 3:] == -7) and np.all(c[0, :3] >= 0) and np.all(c[3] >= 0)


def test_empty_batch_of_blocks(dev):
    """Every length 0: the selector writes nothing, verification takes the
    target's own token from row 0 of every block."""
    cfg = synth.CONFIGS["c0"]
    d = to_dev(synth.make(cfg, seed=7), dev)
    lens = torch.zeros(cfg.batch, dtype=torch.int32, device=dev)
    cid = torch.full((cfg.batch, cfg.block, K), -7, dtype=torch.int32, device=dev)
    cu = torch.zeros((cfg.batch, cfg.block, K), dtype=torch.float32, device=dev)
    ds.select_topk(d["logits"], out=(cid, cu), block_len=lens)
    assert torch.all(cid == -7)
    tl = np.random.default_rng(8).standard_normal((cfg.batch, cfg.block + 1, 500)).astype(np.float32)
    slots = torch.zeros((cfg.batch, cfg.block), dtype=torch.int32, device=dev)
    n, tok = ds.verify(_dev_logits(tl, dev), cid, slots, block_len=lens)
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    assert torch.all(n == 0)
    t = tok.cpu().numpy()
    np.testing.assert_array_equal(t[:, 0], np.argmax(tl[:, 0], axis=1))
    assert np.all(t[:, 1:] == -1)


def test_ragged_longest_block_and_padded_rows(ora, dev):
    """Blocks of up to 32 positions (the longest the walk takes) with fp32
    logit rows padded past the vocabulary (ld > vocab)."""
    cfg = synth.CONFIGS["c0"].replace(batch=5, block=32, vocab=700)
    inp = synth.make(cfg, seed=31)
    lens = np.array([32, 0, 17, 1, 31], np.int32)
    V, ld = cfg.vocab, 704
    wide = np.full((cfg.batch, cfg.block, ld), np.float32(1e30), np.float32)  # never read past vocab
    wide[..., :V] = inp["logits"]
    d = to_dev(inp, dev)
    d["logits"] = torch.from_numpy(wide).to(dev)
    for mode in (0, 1):
        res = ds.select_path(d["logits"], d["E"], d["W_A"], d["W_B"], d["W_H"], d["h"], d["verified"], mode=mode,
                             uniforms=d["uniforms"], vocab=V, want_S=True, block_len=_lens_dev(lens, dev))
        torch.cuda.synchronize()
        assert ds.device_error() == 0
        g = {k: v.cpu().numpy() for k, v in res.items()}
        ref = ora.run_ragged(inp, lens, mode)
        flagged = 0
        for b, n in enumerate(lens):
            if n == 0:
                continue
            sl = lambda a: a[b:b + 1, :n]
            gb = {k: sl(v) for k, v in g.items()}
            np.testing.assert_array_equal(gb["cand_id"], sl(ref["cand_id"]))
            eps, _, _, _ = check_scores(gb["S"], sl(ref["S"]), sl(ref["cand_u"]))
            flagged += check_walk(ora, gb, sl(ref["S"]), gb["S"], sl(ref["cand_id"]), mode, sl(inp["uniforms"]),
                                  1.0, eps)
        assert flagged <= 1
