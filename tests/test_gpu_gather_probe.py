"""dsel_gather_probe: the candidate gather alone, a measurement aid.

Its output words are an XOR fold of what each thread read from LDS, so the
expected words follow from which E row and which 16-byte chunk each LDS slot
holds: 128-row tiles of the gathered rows E[cand_id[m]] (an id outside
[0, vocab), and a row past the last, reads row 0), K split over workgroups in
contiguous ranges of 64-wide steps, and within a tile row rr the chunk at LDS
slot c is chunk c ^ ((rr >> 1) & 7) of the row (the bank swizzle the candidate
GEMM uses).  Matching the words shows that the probe moves the same bytes the
candidate GEMM gathers, every row and chunk once per step."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
from helpers import K

pytestmark = pytest.mark.gpu


def _nsplit(M, d):
    mt, nk = (M + 127) // 128, d // 64
    s = min((512 + mt - 1) // mt, nk // 4)
    return max(s, 1)


def _expected(E, cand, V):
    d = E.shape[1]
    nk = d // 64
    cx = np.bitwise_xor.reduce(E.view(np.uint32).reshape(V, nk, 8, 4), axis=3)  # [V, nk, 8]
    flat = cand.reshape(-1).astype(np.int64)
    M = flat.size
    mt, ns = (M + 127) // 128, _nsplit(M, d)
    tid = np.arange(256)
    out = np.zeros((ns, mt, 256), dtype=np.uint32)
    for t in range(mt):
        rows = np.arange(128) + 128 * t
        tok = np.where(rows < M, flat[np.minimum(rows, M - 1)], 0)
        tok = np.where((tok >= 0) & (tok < V), tok, 0)
        for ks in range(ns):
            k0, k1 = nk * ks // ns, nk * (ks + 1) // ns
            acc = np.zeros(256, dtype=np.uint32)
            for j in range(4):
                rr = tid // 8 + 32 * j
                c = (tid & 7) ^ ((rr >> 1) & 7)
                acc ^= np.bitwise_xor.reduce(cx[tok[rr][:, None], np.arange(k0, k1)[None, :], c[:, None]], axis=1)
            out[ks, t] = acc
    return out.reshape(-1)


@pytest.mark.parametrize("B,L,V,d", [(4, 16, 4099, 512), (3, 5, 1000, 256), (2, 3, 300, 64), (8, 16, 2048, 2560)])
def test_gather_probe_words(dev, B, L, V, d):
    g = np.random.default_rng(B * 1000 + L + d)
    E = g.integers(0, 2 ** 16, size=(V, d), dtype=np.uint16)
    cand = g.integers(0, V, size=(B, L, K)).astype(np.int32)
    cand.reshape(-1)[:: 37] = -1
    cand.reshape(-1)[5:: 41] = V
    n = int(ds.lib().dsel_gather_probe_words(B, L, d))
    assert n == ((B * L * K + 127) // 128) * _nsplit(B * L * K, d) * 256
    Ed = torch.from_numpy(E.view(np.int16)).to(dev).view(torch.bfloat16)
    cd = torch.from_numpy(cand).to(dev)
    out = ds.gather_probe(Ed, cd)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)[:n]
    np.testing.assert_array_equal(got, _expected(E, cand, V))


def test_gather_probe_rejects_short_out(dev):
    E = torch.zeros((128, 64), dtype=torch.bfloat16, device=dev)
    cand = torch.zeros((1, 2, K), dtype=torch.int32, device=dev)
    out = torch.zeros(16, dtype=torch.int32, device=dev)
    st = ds.lib().dsel_gather_probe(E.data_ptr(), 128, 64, cand.data_ptr(), 1, 2, out.data_ptr(), 16, None)
    assert st != 0
