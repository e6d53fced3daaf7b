"""draft_selection_amd -- the DFlash 2 lightweight path selector on MI355X.

Thin ctypes binding over ``libdsel.so`` (C ABI in ``include/dsel.h``).  Every
function takes and returns ``torch`` tensors on the GPU; the binding only checks
shapes, allocates outputs with torch and passes raw pointers plus the current
HIP stream.  Every step of the selector runs in the library's HIP kernels: there
is no CPU fallback, and a missing library is an error.

Entry points (same names as the C ABI):
  select_topk(logits, vocab=None)                   -> cand_id, cand_u
  project(E, W_A, W_B, W_H, h, cand_id, verified)   -> A_prev, B_cur, G
  project_gate(...), project_gate_overlap(...), project_cand(...)  (its halves)
  score_pairs(cand_u, A_prev, B_cur, G, ...)        -> S and/or the walk
  walk(S, cand_id, ...)                             -> the walk alone
  project_pairs(E, W_A, W_B, cand_id, G, A_ver)     -> pair partials (project_cand
                                                       and the pair term fused)
  walk_pairs(cand_u, partials, cand_id, ...)        -> S and/or the walk from them
  select_path(logits, E, W_A, W_B, W_H, h, verified, ...)  -> all of the above
                                                       in one dsel_select_path call
  verify(target_logits, cand_id, path_slot, ...)    -> n_accepted, out_tok
  dyn_conv(x, x_prev, base, W_c)                    -> y
  lmhead_topk(h, W)                                 -> cand_id, cand_u
  device_error()                                    -> sticky device error bits
Every batch call takes ``block_len`` (a ragged batch: valid positions per
block, int32 on the GPU) and ``stream``.
"""
from __future__ import annotations

import ctypes as C
import functools
import inspect
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsel.so")
K = 16
MAX_BLOCK = 32
GREEDY, SAMPLED = 0, 1
F32, BF16 = 0, 1

_STATUS = {0: "DSEL_OK", -1: "DSEL_E_ARG", -2: "DSEL_E_DTYPE", -3: "DSEL_E_ALIGN",
           -4: "DSEL_E_WORKSPACE", -5: "DSEL_E_HIP"}


class DselError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)}")
        self.status = status


class WalkArgs(C.Structure):
    _fields_ = [("mode", C.c_int32), ("temperature", C.c_float), ("uniforms", C.c_void_p),
                ("cand_id", C.c_void_p), ("path_tok", C.c_void_p), ("path_slot", C.c_void_p),
                ("path_s", C.c_void_p), ("q", C.c_void_p)]


class PathArgs(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("dt", C.c_int32), ("vocab", C.c_int64), ("ld", C.c_int64),
                ("E", C.c_void_p), ("d", C.c_int64), ("W_A", C.c_void_p), ("W_B", C.c_void_p),
                ("W_H", C.c_void_p), ("r", C.c_int64), ("h", C.c_void_p), ("verified", C.c_void_p),
                ("batch", C.c_int64), ("block", C.c_int64), ("block_len", C.c_void_p),
                ("cand_id", C.c_void_p), ("cand_u", C.c_void_p), ("A_prev", C.c_void_p), ("B_cur", C.c_void_p),
                ("G", C.c_void_p), ("S", C.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (python -c "
                              "'import __graft_entry__ as g; g.build()')")
        lib = C.CDLL(LIB_PATH)
        P, I64, I32, SZ = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        sig = {
            "dsel_topk_workspace_bytes": ([I64, I64, I32], SZ),
            "dsel_select_topk": ([P, I32, I64, I64, P, I64, I64, P, P, P, SZ, P], I32),
            "dsel_project": ([P, I64, I64, P, P, P, I64, P, P, P, I64, I64, P, P, P, P, P, SZ, P], I32),
            "dsel_project_workspace_bytes": ([I64, I64, I64, I64], SZ),
            "dsel_project_gate": ([P, I64, I64, P, P, I64, P, P, I64, I64, P, P, P, P, SZ, P], I32),
            "dsel_project_gate_overlap": ([P, I64, I64, P, P, I64, P, P, I64, I64, P, P, P, P], I32),
            "dsel_project_cand": ([P, I64, I64, P, P, I64, P, I64, I64, P, P, P, P, SZ, P], I32),
            "dsel_score_pairs": ([P, P, P, P, I64, I64, P, I64, P, C.POINTER(WalkArgs), P], I32),
            "dsel_walk": ([P, I64, I64, P, C.POINTER(WalkArgs), P], I32),
            "dsel_select_path_workspace_bytes": ([I64, I64, I64, I32, I64, I64], SZ),
            "dsel_gather_probe_words": ([I64, I64, I64], SZ),
            "dsel_gather_probe": ([P, I64, I64, P, I64, I64, P, SZ, P], I32),
            "dsel_select_path": ([C.POINTER(PathArgs), C.POINTER(WalkArgs), P, SZ, P], I32),
            "dsel_select_path_noalloc": ([C.POINTER(PathArgs), C.POINTER(WalkArgs), P], I32),
            "dsel_select_path_route": ([C.POINTER(PathArgs)], I32),
            "dsel_pair_groups": ([I64], I64),
            "dsel_project_pairs": ([P, I64, I64, P, P, I64, P, P, P, I64, I64, I64, P, P, P, P, P], I32),
            "dsel_walk_pairs": ([P, P, I64, I64, P, I64, P, C.POINTER(WalkArgs), P], I32),
            "dsel_verify_workspace_bytes": ([I64, I64, I64], SZ),
            "dsel_dyn_conv_workspace_bytes": ([I64, I64, I64], SZ),
            "dsel_lmhead_topk_workspace_bytes": ([I64, I64], SZ),
            "dsel_lmhead_topk": ([P, P, I64, I64, I64, P, P, P, SZ, P], I32),
            "dsel_dyn_conv": ([P, P, P, P, I64, I64, P, I64, P, P, SZ, P], I32),
            "dsel_verify": ([P, I32, I64, I64, P, I64, I64, P, P, P, I32, C.c_float, P, P, P, P, P, SZ, P], I32),
            "dsel_device_error": ([C.POINTER(C.c_int32), P], I32),
            "dsel_status_string": ([I32], C.c_char_p),
            "dsel_version": ([], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def lib():
    """The loaded ``libdsel.so`` (ctypes handle)."""
    return _load()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run ``fn`` with its ``stream`` argument (when given) as the current
    stream, so that the outputs and workspaces it allocates belong to the
    stream its kernels are launched on (the caching allocator then never hands
    them to other work while those kernels may still use them)."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrap(*args, **kwargs):
        s = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if s is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(s):
            return fn(*args, **kwargs)

    return wrap


def _check(status: int, what: str):
    if status != 0:
        raise DselError(status, what)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _lens(block_len, B: int):
    """Checked pointer of an optional ragged-batch length array ``[B]`` int32."""
    if block_len is None:
        return None
    _need(block_len, "block_len", torch.int32, (B,))
    return _ptr(block_len)


def topk_workspace_bytes(rows: int, vocab: int, dtype: torch.dtype) -> int:
    dt = BF16 if dtype == torch.bfloat16 else F32
    return int(_load().dsel_topk_workspace_bytes(rows, vocab, dt))


def _logits_geometry(logits: torch.Tensor, vocab: Optional[int]):
    """``(batch, block, ld, vocab)`` of logits ``[batch, block, >= vocab]`` whose
    rows are evenly spaced with unit stride inside a row."""
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, block, ld]")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must be float32 or bfloat16")
    B, L, ld_shape = logits.shape
    if logits.stride(2) != 1 and ld_shape > 1:
        raise ValueError("logits must have unit stride in the last dim")
    if L > 1:
        ld = logits.stride(1)
        if B > 1 and logits.stride(0) != L * ld:
            raise ValueError("logits rows must be evenly spaced")
    elif B > 1:
        ld = logits.stride(0)
    else:
        ld = ld_shape
    if ld < ld_shape:
        raise ValueError("overlapping logits rows")
    V = ld_shape if vocab is None else int(vocab)
    if V > ld_shape:
        raise ValueError("vocab exceeds the logits width")
    return B, L, ld, V


@_on_stream
def select_topk(logits: torch.Tensor, vocab: Optional[int] = None, out=None, workspace=None,
                stream=None, block_len=None):
    """Top-16 of every draft position.  ``logits [batch, block, ld]`` fp32 or bf16
    with unit stride in the last dim; the first ``vocab`` (default ``ld``) entries
    of each row are used.  Returns ``cand_id [B,L,16] int32``, ``cand_u [B,L,16] fp32``.
    ``block_len`` (every call below takes it too): optional int32 ``[batch]`` of
    valid positions per block (a ragged batch); padding is neither read nor
    written."""
    B, L, ld, V = _logits_geometry(logits, vocab)
    dt = BF16 if logits.dtype == torch.bfloat16 else F32
    dev = logits.device
    if out is None:
        cand_id = torch.empty((B, L, K), dtype=torch.int32, device=dev)
        cand_u = torch.empty((B, L, K), dtype=torch.float32, device=dev)
    else:
        cand_id, cand_u = out
        _need(cand_id, "cand_id", torch.int32, (B, L, K))
        _need(cand_u, "cand_u", torch.float32, (B, L, K))
    need = int(_load().dsel_topk_workspace_bytes(B * L, V, dt))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().dsel_select_topk(_ptr(logits), dt, B, L, _lens(block_len, B), V, ld, _ptr(cand_id), _ptr(cand_u),
                                  _ptr(workspace), wsb, _stream(stream))
    _check(st, "dsel_select_topk")
    return cand_id, cand_u


@_on_stream
def project(E, W_A, W_B, W_H, h, cand_id, verified, out=None, stream=None, block_len=None):
    """``A_prev [B,L,16,r]``, ``B_cur [B,L,16,r]``, ``G [B,L,r]`` (fp32) from bf16
    ``E [V,d]``, ``W_* [r,d]``, ``h [B,L,d]``, int32 ``cand_id``, ``verified [B]``."""
    V, d = E.shape
    r = W_A.shape[0]
    B, L = cand_id.shape[:2]
    for t, n, shp in ((E, "E", (V, d)), (W_A, "W_A", (r, d)), (W_B, "W_B", (r, d)),
                      (W_H, "W_H", (r, d)), (h, "h", (B, L, d))):
        _need(t, n, torch.bfloat16, shp)
    _need(cand_id, "cand_id", torch.int32, (B, L, K))
    _need(verified, "verified", torch.int32, (B,))
    dev = E.device
    if out is None:
        A_prev = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
        B_cur = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
        G = torch.empty((B, L, r), dtype=torch.float32, device=dev)
    else:
        A_prev, B_cur, G = out
        _need(A_prev, "A_prev", torch.float32, (B, L, K, r))
        _need(B_cur, "B_cur", torch.float32, (B, L, K, r))
        _need(G, "G", torch.float32, (B, L, r))
    ws = _project_workspace(B, L, d, r, dev)
    wsb = 0 if ws is None else ws.numel()
    st = _load().dsel_project(_ptr(E), V, d, _ptr(W_A), _ptr(W_B), _ptr(W_H), r, _ptr(h),
                              _ptr(cand_id), _ptr(verified), B, L, _lens(block_len, B), _ptr(A_prev), _ptr(B_cur),
                              _ptr(G), _ptr(ws), wsb, _stream(stream))
    _check(st, "dsel_project")
    return A_prev, B_cur, G


def project_workspace_bytes(batch: int, block: int, d: int, r: int) -> int:
    return int(_load().dsel_project_workspace_bytes(batch, block, d, r))


def _project_workspace(B, L, d, r, dev):
    n = project_workspace_bytes(B, L, d, r)
    return torch.empty(n, dtype=torch.uint8, device=dev) if n else None


@_on_stream
def project_gate(E, W_A, W_H, h, verified, A_prev, G, workspace=None, stream=None, block_len=None):
    """G and the position-0 predecessor rows of A_prev (needs no candidates)."""
    V, d = E.shape
    r = W_A.shape[0]
    B, L = h.shape[:2]
    for t, n, shp in ((E, "E", (V, d)), (W_A, "W_A", (r, d)), (W_H, "W_H", (r, d)), (h, "h", (B, L, d))):
        _need(t, n, torch.bfloat16, shp)
    _need(verified, "verified", torch.int32, (B,))
    _need(A_prev, "A_prev", torch.float32, (B, L, K, r))
    _need(G, "G", torch.float32, (B, L, r))
    if workspace is None:
        workspace = _project_workspace(B, L, d, r, E.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().dsel_project_gate(_ptr(E), V, d, _ptr(W_A), _ptr(W_H), r, _ptr(h), _ptr(verified),
                                   B, L, _lens(block_len, B), _ptr(A_prev), _ptr(G), _ptr(workspace), wsb,
                                   _stream(stream))
    _check(st, "dsel_project_gate")


@_on_stream
def project_gate_overlap(E, W_A, W_H, h, verified, A_prev, G, stream=None, block_len=None):
    """project_gate with one workgroup per output tile and no workspace, for
    running beside select_topk on another stream."""
    V, d = E.shape
    r = W_A.shape[0]
    B, L = h.shape[:2]
    for t, n, shp in ((E, "E", (V, d)), (W_A, "W_A", (r, d)), (W_H, "W_H", (r, d)), (h, "h", (B, L, d))):
        _need(t, n, torch.bfloat16, shp)
    _need(verified, "verified", torch.int32, (B,))
    _need(A_prev, "A_prev", torch.float32, (B, L, K, r))
    _need(G, "G", torch.float32, (B, L, r))
    st = _load().dsel_project_gate_overlap(_ptr(E), V, d, _ptr(W_A), _ptr(W_H), r, _ptr(h), _ptr(verified),
                                           B, L, _lens(block_len, B), _ptr(A_prev), _ptr(G), _stream(stream))
    _check(st, "dsel_project_gate_overlap")


@_on_stream
def project_cand(E, W_A, W_B, cand_id, A_prev, B_cur, workspace=None, stream=None, block_len=None):
    """B_cur and the predecessor rows of A_prev for positions >= 1."""
    V, d = E.shape
    r = W_A.shape[0]
    B, L = cand_id.shape[:2]
    for t, n, shp in ((E, "E", (V, d)), (W_A, "W_A", (r, d)), (W_B, "W_B", (r, d))):
        _need(t, n, torch.bfloat16, shp)
    _need(cand_id, "cand_id", torch.int32, (B, L, K))
    _need(A_prev, "A_prev", torch.float32, (B, L, K, r))
    _need(B_cur, "B_cur", torch.float32, (B, L, K, r))
    if workspace is None:
        workspace = _project_workspace(B, L, d, r, E.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().dsel_project_cand(_ptr(E), V, d, _ptr(W_A), _ptr(W_B), r, _ptr(cand_id), B, L,
                                   _lens(block_len, B), _ptr(A_prev), _ptr(B_cur), _ptr(workspace), wsb, _stream(stream))
    _check(st, "dsel_project_cand")


_side = {}


def side_stream(device) -> "torch.cuda.Stream":
    """A second stream (default priority) per device for work that overlaps."""
    idx = torch.device(device).index or 0
    if idx not in _side:
        _side[idx] = torch.cuda.Stream(device=idx)
    return _side[idx]


def _walk_args(cand_id, mode, temperature, uniforms, want_q, want_s):
    B, L = cand_id.shape[:2]
    dev = cand_id.device
    res = dict(path_tok=torch.empty((B, L), dtype=torch.int32, device=dev),
               path_slot=torch.empty((B, L), dtype=torch.int32, device=dev))
    if want_s:
        res["path_s"] = torch.empty((B, L), dtype=torch.float32, device=dev)
    if want_q:
        res["q"] = torch.empty((B, L, K), dtype=torch.float32, device=dev)
    if mode == SAMPLED:
        if uniforms is None:
            raise ValueError("the sampled walk needs uniforms [batch, block]")
        _need(uniforms, "uniforms", torch.float32, (B, L))
    a = WalkArgs(int(mode), float(temperature),
                 uniforms.data_ptr() if (uniforms is not None and mode == SAMPLED) else None,
                 cand_id.data_ptr(), res["path_tok"].data_ptr(), res["path_slot"].data_ptr(),
                 res["path_s"].data_ptr() if want_s else None,
                 res["q"].data_ptr() if want_q else None)
    return a, res


@_on_stream
def score_pairs(cand_u, A_prev, B_cur, G, want_S: bool = True, walk_mode: Optional[int] = None,
                cand_id=None, temperature: float = 1.0, uniforms=None, want_q: bool = False,
                stream=None, block_len=None):
    """Pair scores ``S [B,L,16,16]`` (returned if ``want_S``) and, when
    ``walk_mode`` is given, the walk over them.  Returns a dict."""
    B, L, _, r = A_prev.shape
    _need(cand_u, "cand_u", torch.float32, (B, L, K))
    _need(A_prev, "A_prev", torch.float32, (B, L, K, r))
    _need(B_cur, "B_cur", torch.float32, (B, L, K, r))
    _need(G, "G", torch.float32, (B, L, r))
    res = {}
    S = torch.empty((B, L, K, K), dtype=torch.float32, device=A_prev.device)
    wa = None
    if walk_mode is not None:
        if cand_id is None:
            raise ValueError("the walk needs cand_id")
        _need(cand_id, "cand_id", torch.int32, (B, L, K))
        wa, res = _walk_args(cand_id, walk_mode, temperature, uniforms, want_q, True)
    st = _load().dsel_score_pairs(_ptr(cand_u), _ptr(A_prev), _ptr(B_cur), _ptr(G), B, L, _lens(block_len, B), r,
                                  _ptr(S), C.byref(wa) if wa is not None else None, _stream(stream))
    _check(st, "dsel_score_pairs")
    if want_S:
        res["S"] = S
    return res


def pair_groups(r: int) -> int:
    """Column groups of the rank in the pair partials of project_pairs."""
    return int(_load().dsel_pair_groups(r))


@_on_stream
def project_pairs(E, W_A, W_B, cand_id, G, A_ver, ver_stride: Optional[int] = None, want_AB: bool = False,
                  stream=None, block_len=None):
    """Candidate projections and the pair term in one kernel (blocks of at most
    16 positions): returns ``partials [B, L, nq, 16, 16]`` fp32 (and ``A_prev``,
    ``B_cur`` with ``want_AB``).  ``A_ver``: A of each block's verified token,
    ``[B, r]`` (``ver_stride`` r) or the ``A_prev`` written by project_gate
    (``ver_stride`` = L * 16 * r)."""
    V, d = E.shape
    r = W_A.shape[0]
    B, L = cand_id.shape[:2]
    for t, n, shp in ((E, "E", (V, d)), (W_A, "W_A", (r, d)), (W_B, "W_B", (r, d))):
        _need(t, n, torch.bfloat16, shp)
    _need(cand_id, "cand_id", torch.int32, (B, L, K))
    _need(G, "G", torch.float32, (B, L, r))
    _need(A_ver, "A_ver", torch.float32)
    vs = r if ver_stride is None else int(ver_stride)
    if B and A_ver.numel() < (B - 1) * vs + r:
        raise ValueError("A_ver is too small for its stride")
    nq = pair_groups(r)
    dev = E.device
    partials = torch.empty((B, L, nq, K, K), dtype=torch.float32, device=dev)
    A_prev = B_cur = None
    if want_AB:
        A_prev = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
        B_cur = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
    st = _load().dsel_project_pairs(_ptr(E), V, d, _ptr(W_A), _ptr(W_B), r, _ptr(cand_id), _ptr(G), _ptr(A_ver), vs,
                                    B, L, _lens(block_len, B), _ptr(partials), _ptr(A_prev), _ptr(B_cur),
                                    _stream(stream))
    _check(st, "dsel_project_pairs")
    res = {"partials": partials}
    if want_AB:
        res.update(A_prev=A_prev, B_cur=B_cur)
    return res


@_on_stream
def walk_pairs(cand_u, partials, cand_id, mode: int = GREEDY, temperature: float = 1.0, uniforms=None,
               want_S: bool = False, want_q: bool = False, stream=None, block_len=None):
    """The scores from project_pairs' partial tables and the walk over them."""
    B, L, nq = partials.shape[:3]
    _need(partials, "partials", torch.float32, (B, L, nq, K, K))
    _need(cand_u, "cand_u", torch.float32, (B, L, K))
    _need(cand_id, "cand_id", torch.int32, (B, L, K))
    S = torch.empty((B, L, K, K), dtype=torch.float32, device=partials.device) if want_S else None
    wa, res = _walk_args(cand_id, mode, temperature, uniforms, want_q, True)
    _check(_load().dsel_walk_pairs(_ptr(cand_u), _ptr(partials), B, L, _lens(block_len, B), nq, _ptr(S), C.byref(wa),
                                   _stream(stream)), "dsel_walk_pairs")
    if want_S:
        res["S"] = S
    return res


@_on_stream
def walk(S, cand_id, mode: int = GREEDY, temperature: float = 1.0, uniforms=None,
         want_q: bool = False, stream=None, block_len=None):
    """The walk alone over ``S [B,L,16,16]`` fp32."""
    B, L = S.shape[:2]
    _need(S, "S", torch.float32, (B, L, K, K))
    _need(cand_id, "cand_id", torch.int32, (B, L, K))
    wa, res = _walk_args(cand_id, mode, temperature, uniforms, want_q, True)
    _check(_load().dsel_walk(_ptr(S), B, L, _lens(block_len, B), C.byref(wa), _stream(stream)), "dsel_walk")
    return res


@_on_stream
def gather_probe(E, cand_id, out=None, stream=None):
    """Measurement aid: the candidate GEMM's gather of ``E[cand_id]`` rows into
    LDS, alone (dsel_gather_probe).  Returns the scratch words it folds its loads
    into (meaningless apart from keeping the loads alive)."""
    V, d = E.shape
    B, L = cand_id.shape[:2]
    _need(E, "E", torch.bfloat16, (V, d))
    _need(cand_id, "cand_id", torch.int32, (B, L, K))
    n = int(_load().dsel_gather_probe_words(B, L, d))
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.int32, device=E.device)
    _check(_load().dsel_gather_probe(_ptr(E), V, d, _ptr(cand_id), B, L, _ptr(out), out.numel(), _stream(stream)),
           "dsel_gather_probe")
    return out


def device_error(stream=None) -> int:
    """Synchronise, then read and clear the device error word."""
    v = C.c_int32(0)
    _check(_load().dsel_device_error(C.byref(v), _stream(stream)), "dsel_device_error")
    return int(v.value)


@_on_stream
def lmhead_topk(h, W, stream=None):
    """The LM head and its top-16 in one pass (logits never written):
    ``h [..., d]`` and ``W [vocab, d]`` bf16; returns ``cand_id [..., 16]``
    int32 and ``cand_u [..., 16]`` fp32 (the fp32 logits)."""
    d = h.shape[-1]
    V = W.shape[0]
    _need(h, "h", torch.bfloat16)
    _need(W, "W", torch.bfloat16, (V, d))
    rows = h.numel() // d
    cid = torch.empty(h.shape[:-1] + (K,), dtype=torch.int32, device=h.device)
    cu = torch.empty(h.shape[:-1] + (K,), dtype=torch.float32, device=h.device)
    wsb = int(_load().dsel_lmhead_topk_workspace_bytes(rows, V)) if rows else 0
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=h.device)
    st = _load().dsel_lmhead_topk(_ptr(h), _ptr(W), rows, V, d, _ptr(cid), _ptr(cu), _ptr(ws), wsb,
                                  _stream(stream))
    _check(st, "dsel_lmhead_topk")
    return cid, cu


def dyn_conv_workspace_bytes(batch: int, block: int, d: int) -> int:
    return int(_load().dsel_dyn_conv_workspace_bytes(batch, block, d))


@_on_stream
def dyn_conv(x, x_prev, base, W_c, y=None, workspace=None, stream=None, block_len=None):
    """Dynamic two-tap short convolution of the drafter over each block's
    positions: ``x [B, L, d]``, ``x_prev [B, d]``, ``base [2, d]``,
    ``W_c [2 d / 16, d]``, all bf16; returns ``y [B, L, d]`` bf16."""
    B, L, d = x.shape
    _need(x, "x", torch.bfloat16, (B, L, d))
    _need(x_prev, "x_prev", torch.bfloat16, (B, d))
    _need(base, "base", torch.bfloat16, (2, d))
    _need(W_c, "W_c", torch.bfloat16, (2 * (d // 16), d))
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", torch.bfloat16, (B, L, d))
    if workspace is None:
        wsb = dyn_conv_workspace_bytes(B, L, d)
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() * workspace.element_size()
    st = _load().dsel_dyn_conv(_ptr(x), _ptr(x_prev), _ptr(base), _ptr(W_c), B, L, _lens(block_len, B), d,
                               _ptr(y), _ptr(workspace),
                               wsb, _stream(stream))
    _check(st, "dsel_dyn_conv")
    return y


def verify_workspace_bytes(batch: int, block: int, vocab: int) -> int:
    return int(_load().dsel_verify_workspace_bytes(batch, block, vocab))


@_on_stream
def verify(target_logits, cand_id, path_slot, q=None, mode: int = GREEDY, temperature: float = 1.0,
           u_acc=None, u_res=None, vocab: Optional[int] = None, workspace=None, stream=None,
           block_len=None):
    """Verify drafted blocks against target logits ``[B, L+1, ld]`` (fp32 or
    bf16): returns ``(n_accepted [B] int32, out_tok [B, L+1] int32)``."""
    B, L1, ld = target_logits.shape
    L = L1 - 1
    V = ld if vocab is None else int(vocab)
    dt = F32 if target_logits.dtype == torch.float32 else BF16
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    if target_logits.stride(2) != 1 or target_logits.stride(1) != target_logits.stride(2) * ld \
            or target_logits.stride(0) != L1 * ld:
        raise ValueError("target_logits must be contiguous")
    _need(cand_id, "cand_id", torch.int32, (B, L, K))
    _need(path_slot, "path_slot", torch.int32, (B, L))
    if mode == SAMPLED:
        _need(q, "q", torch.float32, (B, L, K))
        _need(u_acc, "u_acc", torch.float32, (B, L))
        _need(u_res, "u_res", torch.float32, (B,))
    dev = target_logits.device
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty((B, L + 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(verify_workspace_bytes(B, L, V), 1), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    st = _load().dsel_verify(_ptr(target_logits), dt, B, L, _lens(block_len, B), V, ld, _ptr(cand_id),
                             _ptr(path_slot),
                             _ptr(q) if mode == SAMPLED else None, int(mode), float(temperature),
                             _ptr(u_acc) if mode == SAMPLED else None,
                             _ptr(u_res) if mode == SAMPLED else None, _ptr(n_acc), _ptr(out_tok),
                             _ptr(workspace), wsb, _stream(stream))
    _check(st, "dsel_verify")
    return n_acc, out_tok


def select_path_workspace_bytes(batch: int, block: int, vocab: int, dtype: torch.dtype, d: int, r: int) -> int:
    dt = BF16 if dtype == torch.bfloat16 else F32
    return int(_load().dsel_select_path_workspace_bytes(batch, block, vocab, dt, d, r))


@_on_stream
def select_path(logits, E, W_A, W_B, W_H, h, verified, mode: int = GREEDY,
                temperature: float = 1.0, uniforms=None, vocab: Optional[int] = None,
                want_S: bool = False, want_q: bool = False, want_AB: bool = False, overlap: bool = False,
                stream=None, block_len=None, workspace=None):
    """The whole selector: top-16, projections, pair scores and the walk.

    By default one call of dsel_select_path.  The intermediates are returned
    only when asked for: ``S`` with ``want_S``, ``A_prev``, ``B_cur`` and ``G``
    with ``want_AB`` (not asking lets the library keep the projections on
    chip).  With ``overlap`` the steps are separate calls and the gate GEMM
    (which needs no candidates) runs on a side stream, one workgroup per output
    tile (dsel_project_gate_overlap), beside the top-16."""
    main = torch.cuda.current_stream() if stream is None else stream
    B, L = h.shape[:2]
    r = W_A.shape[0]
    dev = E.device
    if overlap:
        A_prev = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
        B_cur = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
        G = torch.empty((B, L, r), dtype=torch.float32, device=dev)
        ws = _project_workspace(B, L, E.shape[1], r, dev)  # one workspace serves both halves
        side = side_stream(dev)
        side.wait_stream(main)
        project_gate_overlap(E, W_A, W_H, h, verified, A_prev, G, stream=side, block_len=block_len)
        G.record_stream(side)
        A_prev.record_stream(side)
        cand_id, cand_u = select_topk(logits, vocab, stream=main, block_len=block_len)
        main.wait_stream(side)
        project_cand(E, W_A, W_B, cand_id, A_prev, B_cur, workspace=ws, stream=main, block_len=block_len)
        res = score_pairs(cand_u, A_prev, B_cur, G, want_S=want_S, walk_mode=mode, cand_id=cand_id,
                          temperature=temperature, uniforms=uniforms, want_q=want_q, stream=main,
                          block_len=block_len)
        res.update(cand_id=cand_id, cand_u=cand_u)
        if want_AB:
            res.update(A_prev=A_prev, B_cur=B_cur, G=G)
        return res
    Bl, Ll, ld, V = _logits_geometry(logits, vocab)
    if (Bl, Ll) != (B, L):
        raise ValueError("logits and h disagree on [batch, block]")
    VE, d = E.shape
    if VE < V:
        raise ValueError("E needs a row for every token id below vocab")
    for t, n, shp in ((E, "E", (VE, d)), (W_A, "W_A", (r, d)), (W_B, "W_B", (r, d)), (W_H, "W_H", (r, d)),
                      (h, "h", (B, L, d))):
        _need(t, n, torch.bfloat16, shp)
    _need(verified, "verified", torch.int32, (B,))
    cand_id = torch.empty((B, L, K), dtype=torch.int32, device=dev)
    cand_u = torch.empty((B, L, K), dtype=torch.float32, device=dev)
    S = torch.empty((B, L, K, K), dtype=torch.float32, device=dev) if want_S else None
    if want_AB:
        A_prev = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
        B_cur = torch.empty((B, L, K, r), dtype=torch.float32, device=dev)
        G = torch.empty((B, L, r), dtype=torch.float32, device=dev)
    else:
        A_prev = B_cur = G = None
    wa, res = _walk_args(cand_id, mode, temperature, uniforms, want_q, True)
    dt = BF16 if logits.dtype == torch.bfloat16 else F32
    need = select_path_workspace_bytes(B, L, V, logits.dtype, d, r)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()

    def addr(t):
        return None if t is None else t.data_ptr()

    pa = PathArgs(logits.data_ptr(), dt, V, ld, E.data_ptr(), d, W_A.data_ptr(), W_B.data_ptr(), W_H.data_ptr(),
                  r, h.data_ptr(), verified.data_ptr(), B, L,
                  _lens(block_len, B).value if block_len is not None else None,
                  cand_id.data_ptr(), cand_u.data_ptr(), addr(A_prev), addr(B_cur), addr(G), addr(S))
    _check(_load().dsel_select_path(C.byref(pa), C.byref(wa), _ptr(workspace), wsb, _stream(main)),
           "dsel_select_path")
    if want_S:
        res["S"] = S
    res.update(cand_id=cand_id, cand_u=cand_u)
    if want_AB:
        res.update(A_prev=A_prev, B_cur=B_cur, G=G)
    return res


ROUTE_SEPARATE, ROUTE_FUSED, ROUTE_SMALL = 0, 1, 2


def select_path_route(batch: int, block: int, vocab: int, dtype, d: int, r: int, want_AB: bool = False) -> int:
    """The route dsel_select_path takes for this shape (dsel_select_path_route):
    ROUTE_FUSED, ROUTE_SMALL or ROUTE_SEPARATE (-1: empty or invalid)."""
    dt = BF16 if dtype == torch.bfloat16 else F32
    mark = 16 if want_AB else None  # only whether the outputs are given is read
    pa = PathArgs(None, dt, vocab, vocab, None, d, None, None, None, r, None, None, batch, block, None, None, None,
                  mark, mark, mark, None)
    return int(_load().dsel_select_path_route(C.byref(pa)))
