"""select_topk on the GPU against the oracle: bit-exact ids and values.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: the
16 best candidates of every draft position.)"""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth
from helpers import bf16_dev

pytestmark = pytest.mark.gpu
K = 16


def _rows(kind, rng, n, V):
    if kind == "normal":
        return rng.standard_normal((n, V)).astype(np.float32) * 3
    if kind == "ties":
        return (rng.integers(0, 17, size=(n, V)) * 0.25).astype(np.float32)
    if kind == "special":
        ch = np.array([0.0, -0.0, -np.inf, np.inf, np.nan, 1.0, -1.0, 2.5], np.float32)
        return rng.choice(ch, size=(n, V)).astype(np.float32)
    if kind == "ascending":  # every element beats the running 16th: worst case for inserts
        return np.broadcast_to(np.arange(V, dtype=np.float32), (n, V)).copy()
    if kind == "descending":
        return np.broadcast_to(np.arange(V, 0, -1, dtype=np.float32), (n, V)).copy()
    raise ValueError(kind)


def _run(x_host, dtype, dev, V, offset=0, B=None, L=None):
    """x_host: [rows, ld] float32 (values representable in dtype).  `offset`
    shifts every row start by that many elements (misaligned rows)."""
    rows, ld = x_host.shape
    B = rows if B is None else B
    L = 1 if L is None else L
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x_host)
        flat = np.zeros(rows * ld + offset, np.uint16)
        flat[offset:] = bits.reshape(-1)
        t = bf16_dev(flat, dev)
        host_vals = synth.bf16_bits_to_f32(bits)
    else:
        flat = np.zeros(rows * ld + offset, np.float32)
        flat[offset:] = x_host.reshape(-1)
        t = torch.from_numpy(flat).to(dev)
        host_vals = x_host
    view = t[offset:].view(B, L, ld)
    cid, cu = ds.select_topk(view, vocab=V)
    torch.cuda.synchronize()
    return cid.cpu().numpy().reshape(rows, K), cu.cpu().numpy().reshape(rows, K), host_vals


def _expect(ora, host_vals, V):
    return ora.select_topk(np.ascontiguousarray(host_vals), vocab=V)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
@pytest.mark.parametrize("V,rows", [(16, 5), (17, 3), (23, 7), (100, 9), (1000, 33), (4099, 6),
                                    (65537, 3), (152064, 2)])
def test_topk_matches_oracle(ora, dev, dtype, kind, V, rows):
    rng = np.random.default_rng(V * 31 + rows + len(kind))
    x = _rows(kind, rng, rows, V)
    cid, cu, hv = _run(x, dtype, dev, V)
    rid, ru = _expect(ora, hv, V)
    np.testing.assert_array_equal(cid, rid)
    np.testing.assert_array_equal(cu.view(np.uint32), ru.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("offset", [1, 3, 5])
@pytest.mark.parametrize("ld_pad", [0, 3, 8])
def test_topk_misaligned_rows_and_padding(ora, dev, dtype, offset, ld_pad):
    """Rows that start off a 16-byte boundary, and a leading dimension > vocab
    whose padding holds +inf (which must never be picked)."""
    rng = np.random.default_rng(offset * 10 + ld_pad)
    V, rows = 3001, 12
    ld = V + ld_pad
    x = np.full((rows, ld), np.inf, np.float32)
    x[:, :V] = _rows("ties", rng, rows, V)
    cid, cu, hv = _run(x, dtype, dev, V, offset=offset)
    rid, ru = _expect(ora, hv, V)
    np.testing.assert_array_equal(cid, rid)
    np.testing.assert_array_equal(cu.view(np.uint32), ru.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["ascending", "descending"])
def test_topk_monotone_rows(ora, dev, dtype, kind):
    V = 20000 if dtype == "f32" else 200  # bf16 keeps integers exact only up to 256
    x = _rows(kind, np.random.default_rng(0), 4, V)
    cid, cu, hv = _run(x, dtype, dev, V)
    rid, ru = _expect(ora, hv, V)
    np.testing.assert_array_equal(cid, rid)


@pytest.mark.parametrize("rows", [1, 2, 16, 63, 300])
def test_topk_split_and_unsplit_rows(ora, dev, rows):
    """Few rows over a long vocabulary are split across workgroups and merged."""
    rng = np.random.default_rng(rows)
    V = 40000
    x = _rows("normal", rng, rows, V)
    cid, cu, hv = _run(x, "bf16", dev, V)
    rid, _ = _expect(ora, hv, V)
    np.testing.assert_array_equal(cid, rid)


def test_topk_empty_batch(dev):
    t = torch.zeros((0, 8, 1024), dtype=torch.float32, device=dev)
    cid, cu = ds.select_topk(t)
    torch.cuda.synchronize()
    assert cid.shape == (0, 8, K)


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_topk_workloads(ora, dev, name):
    """Full workload sizes: every row against the oracle."""
    cfg = synth.CONFIGS[name]
    x = synth.make_logits(cfg)
    t = bf16_dev(x, dev) if x.dtype == np.uint16 else torch.from_numpy(x).to(dev)
    cid, cu = ds.select_topk(t)
    torch.cuda.synchronize()
    rid, ru = ora.select_topk(x)
    np.testing.assert_array_equal(cid.cpu().numpy(), rid)
    np.testing.assert_array_equal(cu.cpu().numpy().view(np.uint32), ru.view(np.uint32))
    # determinism: a second call is bitwise identical
    cid2, cu2 = ds.select_topk(t)
    torch.cuda.synchronize()
    assert torch.equal(cid, cid2) and torch.equal(cu.view(torch.int32), cu2.view(torch.int32))
