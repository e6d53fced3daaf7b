"""dsel_select_path_noalloc (the whole selector for callers that cannot
allocate: its workspace is the library's fixed per-device array) against
dsel_select_path with a caller workspace: the same bits, on two calls in a row,
the second with a smaller input and the other route; a shape beyond the array
is refused before anything is launched."""
import ctypes as C

import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth
from helpers import to_dev

pytestmark = pytest.mark.gpu
K = 16


def _outputs(d, want_AB, want_S):
    B, L = d["h"].shape[:2]
    r = d["W_A"].shape[0]
    dev = d["E"].device
    o = {"cand_id": torch.full((B, L, K), -7, dtype=torch.int32, device=dev),
         "cand_u": torch.full((B, L, K), 7.0, dtype=torch.float32, device=dev)}
    if want_AB:
        o["A_prev"] = torch.full((B, L, K, r), 7.0, dtype=torch.float32, device=dev)
        o["B_cur"] = torch.full((B, L, K, r), 7.0, dtype=torch.float32, device=dev)
        o["G"] = torch.full((B, L, r), 7.0, dtype=torch.float32, device=dev)
    if want_S:
        o["S"] = torch.full((B, L, K, K), 7.0, dtype=torch.float32, device=dev)
    return o


def _call(d, mode, want_AB, want_S, noalloc):
    lib = ds.lib()
    B, L = d["h"].shape[:2]
    V = d["logits"].shape[2]
    r, dd = d["W_A"].shape
    dt = ds.BF16 if d["logits"].dtype == torch.bfloat16 else ds.F32
    o = _outputs(d, want_AB, want_S)
    wa, wres = ds._walk_args(o["cand_id"], mode, 1.0, d["uniforms"], True, True)
    ptr = lambda k: o[k].data_ptr() if k in o else None
    pa = ds.PathArgs(d["logits"].data_ptr(), dt, V, V, d["E"].data_ptr(), dd, d["W_A"].data_ptr(),
                     d["W_B"].data_ptr(), d["W_H"].data_ptr(), r, d["h"].data_ptr(), d["verified"].data_ptr(), B, L,
                     None, ptr("cand_id"), ptr("cand_u"), ptr("A_prev"), ptr("B_cur"), ptr("G"), ptr("S"))
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = lib.dsel_select_path_noalloc(C.byref(pa), C.byref(wa), stream)
    else:
        wsb = ds.select_path_workspace_bytes(B, L, V, d["logits"].dtype, dd, r)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=d["E"].device)
        st = lib.dsel_select_path(C.byref(pa), C.byref(wa), C.c_void_p(ws.data_ptr()), wsb, stream)
    assert st == 0, st
    torch.cuda.synchronize()
    assert ds.device_error() == 0
    o.update(wres)
    return {k: v.cpu().numpy() for k, v in o.items()}


def _same_bits(a, b):
    assert a.keys() == b.keys()
    for k in a:
        x, y = a[k], b[k]
        if x.dtype.kind == "f":
            x, y = x.view(np.uint32), y.view(np.uint32)
        np.testing.assert_array_equal(x, y, err_msg=k)


def test_noalloc_equals_select_path_two_calls(dev):
    # first call: 64 blocks of 16 at d 2560 (the fused route, 9.3 MiB of workspace)
    big = to_dev(synth.make(synth.CONFIGS["c2"], seed=41), dev)
    for mode, want_AB, want_S in ((0, False, True), (1, True, True)):
        _same_bits(_call(big, mode, want_AB, want_S, True), _call(big, mode, want_AB, want_S, False))
    del big
    # second call, smaller: 3 blocks of 8 at d 64 (the separate kernels, intermediates in the array)
    small = to_dev(synth.make(synth.CONFIGS["c0"].replace(batch=3), seed=42), dev)
    for mode, want_AB, want_S in ((1, False, False), (0, True, True)):
        _same_bits(_call(small, mode, want_AB, want_S, True), _call(small, mode, want_AB, want_S, False))


def test_noalloc_refuses_shapes_beyond_its_array(dev):
    lib = ds.lib()
    f = 0x100000  # never dereferenced: the size check comes first
    need = lib.dsel_select_path_workspace_bytes(2048, 16, 202048, 0, 6144, 256)
    assert need > (48 << 20)
    w = ds.WalkArgs(0, 1.0, None, f, f, f, None, None)
    pa = ds.PathArgs(f, 0, 202048, 202048, f, 6144, f, f, f, 256, f, f, 2048, 16, None, f, f, None, None, None,
                     None)
    assert lib.dsel_select_path_noalloc(C.byref(pa), C.byref(w), None) == -4
