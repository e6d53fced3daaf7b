"""The C ABI library loads and exports every function include/dsel.h declares,
and its host-side validation rejects bad arguments before any launch.

CPU only: every call below either needs no device or fails validation, which
happens on the host before anything is launched."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsel.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsel_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import draft_selection_amd as ds

    if not os.path.exists(ds.LIB_PATH):
        pytest.fail("libdsel.so is not built (run __graft_entry__.build())")
    return ds.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("dsel_select_topk", "dsel_project", "dsel_project_gate", "dsel_project_gate_overlap",
                 "dsel_project_cand",
                 "dsel_score_pairs", "dsel_walk", "dsel_verify"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), f"{name} missing from libdsel.so"


def test_version_and_status_strings(lib):
    assert lib.dsel_version() == 200
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.dsel_status_string(code).startswith(b"DSEL_")


def test_project_workspace_sizing(lib):
    # the gate GEMM of 64 blocks of 16 is split along K across workgroups
    assert lib.dsel_project_workspace_bytes(64, 16, 2560, 256) > 0
    assert lib.dsel_project_workspace_bytes(64, 16, 96, 256) == 0  # d % 64 != 0: invalid
    # one block: the candidate GEMM is split too, so the workspace grows
    assert lib.dsel_project_workspace_bytes(1, 16, 2560, 256) > lib.dsel_project_workspace_bytes(64, 16, 2560, 256) / 64
    fake = C.c_void_p(0x100000)
    args = [fake, 151936, 2560, fake, fake, fake, 256, fake, fake, fake, 64, 16, None, fake, fake, fake,
            None, 0, None]
    assert lib.dsel_project(*args) == -4  # workspace missing
    # the candidate half of one block needs its part of the workspace
    cand_args = [fake, 151936, 2560, fake, fake, 256, fake, 1, 16, None, fake, fake, None, 0, None]
    assert lib.dsel_project_cand(*cand_args) == -4
    small = list(cand_args); small[12] = fake; small[13] = 64
    assert lib.dsel_project_cand(*small) == -4


def test_topk_workspace_sizing(lib):
    # one block of 16 over a 152k vocabulary is split across workgroups
    assert lib.dsel_topk_workspace_bytes(16, 151936, 1) > 0
    assert lib.dsel_topk_workspace_bytes(1024, 151936, 1) == 0
    assert lib.dsel_topk_workspace_bytes(16, 15, 1) == 0


def test_validation_rejects_before_launch(lib):
    import draft_selection_amd as ds

    P = C.c_void_p
    fake = P(0x100000)  # never dereferenced: each call fails validation first
    odd = P(0x100001)
    # select_topk
    assert lib.dsel_select_topk(None, 1, 1, 1, None, 1024, 1024, fake, fake, None, 0, None) == -1
    assert lib.dsel_select_topk(fake, 7, 1, 1, None, 1024, 1024, fake, fake, None, 0, None) == -2
    assert lib.dsel_select_topk(fake, 1, 1, 1, None, 15, 15, fake, fake, None, 0, None) == -1
    assert lib.dsel_select_topk(fake, 1, 1, 1, None, 64, 32, fake, fake, None, 0, None) == -1
    assert lib.dsel_select_topk(odd, 1, 1, 1, None, 64, 64, fake, fake, None, 0, None) == -3
    assert lib.dsel_select_topk(fake, 1, 1, 16, None, 151936, 151936, fake, fake, None, 0, None) == -4
    # project
    args = [fake, 1000, 64, fake, fake, fake, 32, fake, fake, fake, 2, 4, None, fake, fake, fake, None, 0, None]
    bad_d = list(args); bad_d[2] = 96
    bad_r = list(args); bad_r[6] = 48
    big_r = list(args); big_r[6] = 512
    mis = list(args); mis[0] = P(0x100008)
    nul = list(args); nul[7] = None
    for a, code in ((bad_d, -1), (bad_r, -1), (big_r, -1), (mis, -3), (nul, -1)):
        assert lib.dsel_project(*a) == code
    # score_pairs / walk
    w = ds.WalkArgs(5, 1.0, None, 0x100000, 0x100000, 0x100000, None, None)
    assert lib.dsel_score_pairs(fake, fake, fake, fake, 1, 8, None, 32, fake, C.byref(w), None) == -2
    assert lib.dsel_score_pairs(fake, fake, fake, fake, 1, 33, None, 32, fake, None, None) == -1
    assert lib.dsel_score_pairs(fake, fake, fake, fake, 1, 8, None, 32, None, None, None) == -1
    w = ds.WalkArgs(0, 1.0, None, 0x100000, 0x100000, 0x100000, None, None)
    assert lib.dsel_score_pairs(fake, fake, fake, fake, 1, 8, None, 32, None, C.byref(w), None) == -1
    w = ds.WalkArgs(1, 1.0, None, 0x100000, 0x100000, 0x100000, None, None)  # sampled, no uniforms
    assert lib.dsel_walk(fake, 1, 8, None, C.byref(w), None) == -1
    w = ds.WalkArgs(1, 0.0, 0x100000, 0x100000, 0x100000, 0x100000, None, None)  # T = 0
    assert lib.dsel_walk(fake, 1, 8, None, C.byref(w), None) == -1
    assert lib.dsel_walk(fake, 1, 0, None, C.byref(w), None) == -1
    assert lib.dsel_device_error(None, None) == -1
    # ragged batches: a misaligned length array is rejected before any launch
    assert lib.dsel_select_topk(fake, 1, 1, 16, odd, 1024, 1024, fake, fake, None, 0, None) == -3
    assert lib.dsel_walk(fake, 1, 8, odd, C.byref(ds.WalkArgs(0, 1.0, None, 0x100000, 0x100000, 0x100000,
                                                              None, None)), None) == -3


def test_verify_validation(lib):
    P = C.c_void_p
    fake, odd = P(0x100000), P(0x100008)
    ws = lib.dsel_verify_workspace_bytes(4, 8, 151936)
    assert ws > 0 and lib.dsel_verify_workspace_bytes(4, 33, 151936) == 0
    assert lib.dsel_verify_workspace_bytes(4, 8, (1 << 22) + 1) == 0

    def call(**kw):
        a = dict(tl=fake, dt=1, B=4, L=8, lens=None, V=151936, ld=151936, cand=fake, slot=fake, q=fake, mode=1,
                 T=C.c_float(1.0), ua=fake, ur=fake, n=fake, out=fake, ws=fake, wsb=ws)
        a.update(kw)
        return lib.dsel_verify(a["tl"], a["dt"], a["B"], a["L"], a["lens"], a["V"], a["ld"], a["cand"], a["slot"],
                               a["q"], a["mode"], a["T"], a["ua"], a["ur"], a["n"], a["out"], a["ws"],
                               a["wsb"], None)

    assert call(dt=3) == -2 and call(mode=2) == -2
    assert call(L=33) == -1 and call(V=(1 << 22) + 1, ld=(1 << 22) + 8) == -1 and call(ld=100) == -1
    assert call(T=C.c_float(0.0)) == -1 and call(q=None) == -1 and call(ur=None) == -1
    assert call(mode=0, q=None, ua=None, ur=None, T=C.c_float(0.0), ws=None, wsb=0) == -4
    assert call(tl=odd) == -3 and call(ld=151937) == -3     # row starts must be 16-byte aligned
    assert call(ws=None) == -4 and call(wsb=ws - 1) == -4
    assert call(B=0, tl=None, cand=None) == 0               # no work: pointers may be NULL
    assert call(lens=P(0x100002)) == -3                     # ragged lengths: int32 alignment


def test_select_path_validation(lib):
    """dsel_select_path validates every step before launching anything."""
    import draft_selection_amd as ds

    P = C.c_void_p
    f = 0x100000  # never dereferenced
    w = ds.WalkArgs(0, 1.0, None, f, f, f, None, None)
    ws = lib.dsel_select_path_workspace_bytes(1, 16, 151936, 1, 2560, 256)
    assert ws > lib.dsel_project_workspace_bytes(1, 16, 2560, 256)  # top-16 partials come first

    def args(**kw):
        a = dict(logits=f, dt=1, vocab=151936, ld=151936, E=f, d=2560, W_A=f, W_B=f, W_H=f, r=256, h=f,
                 verified=f, batch=1, block=16, block_len=None, cand_id=f, cand_u=f, A_prev=f, B_cur=f, G=f, S=f)
        a.update(kw)
        return ds.PathArgs(*[a[n] for n, _ in ds.PathArgs._fields_])

    call = lambda a, walk=w, wsp=f, wsb=ws: lib.dsel_select_path(C.byref(a), C.byref(walk) if walk else None,
                                                                  P(wsp) if wsp else None, wsb, None)
    assert lib.dsel_select_path(None, C.byref(w), P(f), ws, None) == -1
    assert call(args(), walk=None) == -1
    assert call(args(), wsb=0) == -4 and call(args(), wsp=None) == -4
    assert call(args(), wsp=f + 8) == -3
    assert call(args(dt=5)) == -2
    assert call(args(d=96)) == -1 and call(args(r=48)) == -1 and call(args(block=33), wsb=1 << 40) == -1
    assert call(args(A_prev=None)) == -1 and call(args(B_cur=None)) == -1  # both or neither
    assert call(args(h=0x100002)) == -3 and call(args(block_len=0x100002)) == -3
    assert call(args(batch=0, logits=None, E=None)) == 0  # no work



def test_project_pairs_and_walk_pairs_validation(lib):
    """dsel_project_pairs / dsel_walk_pairs check their arguments on the host."""
    import draft_selection_amd as ds

    P = C.c_void_p
    f = P(0x100000)  # never dereferenced
    assert lib.dsel_pair_groups(256) == 4 and lib.dsel_pair_groups(32) == 1 and lib.dsel_pair_groups(128) == 2
    assert lib.dsel_pair_groups(224) == 7 and lib.dsel_pair_groups(48) == 0 and lib.dsel_pair_groups(288) == 0

    def pp(**kw):
        a = dict(E=f, vocab=1024, d=64, W_A=f, W_B=f, r=32, cand_id=f, G=f, A_ver=f, ver_stride=32, batch=4,
                 block=8, block_len=None, partials=f, A_prev=None, B_cur=None, stream=None)
        a.update(kw)
        return lib.dsel_project_pairs(*a.values())

    assert pp(block=17) == -1  # tiles hold whole blocks of at most 16 positions
    assert pp(ver_stride=16) == -1 and pp(partials=None) == -1 and pp(G=None) == -1
    assert pp(A_prev=f) == -1  # A_prev and B_cur go together
    assert pp(d=96) == -1 and pp(r=48) == -1
    assert pp(G=P(0x100004)) == -3 and pp(ver_stride=34) == -3
    assert pp(batch=0, E=None, W_A=None) == 0  # no work
    w = ds.WalkArgs(0, 1.0, None, 0x100000, 0x100000, 0x100000, None, None)

    def wp(walk=w, **kw):
        a = dict(cand_u=f, partials=f, batch=4, block=8, block_len=None, nq=1, S=None)
        a.update(kw)
        return lib.dsel_walk_pairs(*a.values(), C.byref(walk) if walk else None, None)

    assert wp(walk=None) == -1 and wp(nq=0) == -1 and wp(nq=9) == -1 and wp(block=33) == -1
    assert wp(partials=None) == -1 and wp(partials=P(0x100004)) == -3
    assert wp(walk=ds.WalkArgs(5, 1.0, None, 0x100000, 0x100000, 0x100000, None, None)) == -2
    assert wp(batch=0, cand_u=None, partials=None) == 0


def test_select_path_route_by_shape():
    """dsel_select_path_route is host logic (no GPU): the fused kernels once
    the batch fills the chip, the three-launch small-batch route for a few
    blocks when no intermediates are asked for, the separate kernels
    otherwise (intermediates wanted, an unsplit gate, more than 128 positions)."""
    import torch
    import draft_selection_amd as ds
    bf, f32 = torch.bfloat16, torch.float32
    V = 151936
    assert ds.select_path_route(1, 16, V, bf, 2560, 256) == ds.ROUTE_SMALL
    assert ds.select_path_route(2, 16, V, bf, 2560, 256) == ds.ROUTE_SMALL  # 32 positions
    assert ds.select_path_route(32, 1, V, bf, 2560, 256) == ds.ROUTE_SMALL
    assert ds.select_path_route(3, 16, V, bf, 2560, 256) == ds.ROUTE_SEPARATE  # 48 positions
    assert ds.select_path_route(8, 16, V, bf, 2560, 256) == ds.ROUTE_SEPARATE
    assert ds.select_path_route(2, 16, V, f32, 2560, 96) == ds.ROUTE_SMALL
    assert ds.select_path_route(1, 16, V, bf, 2560, 256, want_AB=True) == ds.ROUTE_SEPARATE
    assert ds.select_path_route(9, 16, V, bf, 2560, 256) == ds.ROUTE_SEPARATE
    assert ds.select_path_route(4, 8, 1024, f32, 64, 32) == ds.ROUTE_SEPARATE  # d 64: one K step, no split
    assert ds.select_path_route(64, 16, V, bf, 2560, 256) == ds.ROUTE_FUSED
    assert ds.select_path_route(256, 16, 202048, f32, 6144, 256, want_AB=True) == ds.ROUTE_FUSED
    assert ds.select_path_route(0, 16, V, bf, 2560, 256) == -1
