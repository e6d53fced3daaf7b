"""CPU oracle of the DFlash 2 path selector -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
fp64, OpenMP; see ``oracle.h``) with numpy in / numpy out, and shares no code
with the HIP path.

Every function below is pinned by the ``-m "not gpu"`` tests against brute
force, library routines, closed forms and invariants (``tests/test_oracle_*``).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
K = 16
GREEDY, SAMPLED = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
               "-o", _SO, os.path.join(_HERE, "oracle.c"), "-lm"]
        subprocess.run(cmd, check=True)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = C.CDLL(_SO)
        P, I64, I32, D = C.c_void_p, C.c_int64, C.c_int, C.c_double
        sig = {
            "ora_select_topk": [P, I32, I64, I64, I64, P, P],
            "ora_project": [P, I64, I64, P, P, P, I64, P, P, P, I64, I64, P, P, P],
            "ora_score_pairs": [P, P, P, P, I64, I64, I64, P],
            "ora_step": [P, I32, I32, D, D, P, P, P],
            "ora_walk": [P, P, P, D, I32, I64, I64, P, P, P, P, P],
            "ora_step_table": [P, P, D, I32, I64, I64, P, P],
            "ora_verify": [P, I32, I64, I64, I64, I64, P, P, P, I32, D, P, P, P, P, P, P],
            "ora_verify_draw": [P, I32, I64, I64, I64, I64, P, P, I32, D, P, I64, I64, I32, P, P],
            "ora_dyn_conv": [P, P, P, P, I64, I64, I64, P, P],
            "ora_lmhead_topk": [P, P, I64, I64, I64, P, P],
            "ora_time_selector": [P, I32, I64, P, I64, P, P, P, I64, P, P, P, D, I32, I64, I64, P, P, P],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = C.c_int
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def select_topk(logits: np.ndarray, vocab: Optional[int] = None):
    """Top-16 of every row.  ``logits[..., ld]``: float32, or uint16 bf16 bits.

    Returns ``cand_id`` int32 and ``cand_u`` float32, shape ``[..., 16]``.
    """
    x = np.ascontiguousarray(logits)
    if x.dtype == np.float32:
        dt = 0
    elif x.dtype == np.uint16:
        dt = 1
    else:
        raise TypeError("logits must be float32 or uint16 (bf16 bits)")
    ld = x.shape[-1]
    V = ld if vocab is None else int(vocab)
    rows = int(np.prod(x.shape[:-1]))
    cid = np.empty(x.shape[:-1] + (K,), np.int32)
    cu = np.empty(x.shape[:-1] + (K,), np.float32)
    _check(_load().ora_select_topk(_p(x), dt, rows, V, ld, _p(cid), _p(cu)), "select_topk")
    return cid, cu


def project(E, W_A, W_B, W_H, h, cand_id, verified):
    """fp64 ``A_prev [B,L,16,r]``, ``B_cur [B,L,16,r]``, ``G [B,L,r]``."""
    E = np.ascontiguousarray(E, np.uint16)
    W_A, W_B, W_H = (np.ascontiguousarray(w, np.uint16) for w in (W_A, W_B, W_H))
    h = np.ascontiguousarray(h, np.uint16)
    cand_id = np.ascontiguousarray(cand_id, np.int32)
    verified = np.ascontiguousarray(verified, np.int32)
    V, d = E.shape
    r = W_A.shape[0]
    B, L = cand_id.shape[:2]
    assert W_A.shape == W_B.shape == W_H.shape == (r, d) and h.shape == (B, L, d)
    assert cand_id.shape == (B, L, K) and verified.shape == (B,)
    A = np.empty((B, L, K, r), np.float64)
    Bm = np.empty((B, L, K, r), np.float64)
    G = np.empty((B, L, r), np.float64)
    rc = _load().ora_project(_p(E), V, d, _p(W_A), _p(W_B), _p(W_H), r, _p(h), _p(cand_id),
                             _p(verified), B, L, _p(A), _p(Bm), _p(G))
    _check(rc, "project")
    return A, Bm, G


def score_pairs(cand_u, A_prev, B_cur, G):
    """fp64 ``S [B,L,16,16]``."""
    cand_u = np.ascontiguousarray(cand_u, np.float32)
    A_prev = np.ascontiguousarray(A_prev, np.float64)
    B_cur = np.ascontiguousarray(B_cur, np.float64)
    G = np.ascontiguousarray(G, np.float64)
    B, L, _, r = A_prev.shape
    S = np.empty((B, L, K, K), np.float64)
    _check(_load().ora_score_pairs(_p(cand_u), _p(A_prev), _p(B_cur), _p(G), B, L, r, _p(S)),
           "score_pairs")
    return S


def step(S_bt, row: int, mode: int = GREEDY, u: float = 0.0, T: float = 1.0):
    """One walk step from predecessor ``row`` of a 16x16 score table.

    Returns ``(choice, aux, q)``: aux is the top-2 gap (greedy) or the CDF margin
    over Z (sampled)."""
    S_bt = np.ascontiguousarray(S_bt, np.float64)
    assert S_bt.shape == (K, K)
    ch = C.c_int(0)
    aux = C.c_double(0)
    q = np.empty(K, np.float64)
    _check(_load().ora_step(_p(S_bt), int(row), int(mode), float(u), float(T), C.byref(ch),
                            C.byref(aux), _p(q)), "step")
    return ch.value, aux.value, q


def walk(S, cand_id, mode: int = GREEDY, uniforms=None, T: float = 1.0):
    """Walk every block from the verified token.

    Returns dict with ``path_tok``, ``path_slot`` int32 ``[B,L]``, ``path_s``,
    ``aux`` float64 ``[B,L]`` and ``q`` float64 ``[B,L,16]``."""
    S = np.ascontiguousarray(S, np.float64)
    cand_id = np.ascontiguousarray(cand_id, np.int32)
    B, L = S.shape[:2]
    u = None if uniforms is None else np.ascontiguousarray(uniforms, np.float32)
    out = dict(path_tok=np.empty((B, L), np.int32), path_slot=np.empty((B, L), np.int32),
               path_s=np.empty((B, L), np.float64), aux=np.empty((B, L), np.float64),
               q=np.empty((B, L, K), np.float64))
    rc = _load().ora_walk(_p(S), _p(cand_id), _p(u), float(T), int(mode), B, L,
                          _p(out["path_tok"]), _p(out["path_slot"]), _p(out["path_s"]),
                          _p(out["aux"]), _p(out["q"]))
    _check(rc, "walk")
    return out


def step_table(S, mode: int = GREEDY, uniforms=None, T: float = 1.0):
    """Choice and aux of the step from every predecessor row: ``[B,L,16]`` each."""
    S = np.ascontiguousarray(S, np.float64)
    B, L = S.shape[:2]
    u = None if uniforms is None else np.ascontiguousarray(uniforms, np.float32)
    choice = np.empty((B, L, K), np.int32)
    aux = np.empty((B, L, K), np.float64)
    _check(_load().ora_step_table(_p(S), _p(u), float(T), int(mode), B, L, _p(choice), _p(aux)),
           "step_table")
    return choice, aux


def run(inp: Dict[str, np.ndarray], mode: int = GREEDY, T: float = 1.0, vocab: Optional[int] = None):
    """The whole selector on one set of inputs (as drawn by ``synth.make``)."""
    cand_id, cand_u = select_topk(inp["logits"], vocab)
    A, Bm, G = project(inp["E"], inp["W_A"], inp["W_B"], inp["W_H"], inp["h"], cand_id,
                       inp["verified"])
    S = score_pairs(cand_u, A, Bm, G)
    w = walk(S, cand_id, mode, inp.get("uniforms"), T)
    return dict(cand_id=cand_id, cand_u=cand_u, A_prev=A, B_cur=Bm, G=G, S=S, **w)


def _tlogits(tlogits, vocab):
    tl = np.ascontiguousarray(tlogits)
    dtype = 0 if tl.dtype == np.float32 else 1
    assert tl.dtype in (np.float32, np.uint16)
    B, L1, ld = tl.shape
    return tl, dtype, B, L1 - 1, (ld if vocab is None else int(vocab)), ld


def verify(tlogits, cand_id, path_slot, q=None, mode: int = GREEDY, T: float = 1.0, u_acc=None,
           u_res=None, vocab: Optional[int] = None):
    """Lossless verification of drafted blocks against target logits
    ``[B, L+1, ld]`` (see ``ora_verify``).  Returns dict with ``n_acc`` [B],
    ``out_tok`` [B, L+1] and the margins ``m_acc`` [B, L], ``m_draw`` [B]."""
    tl, dt, B, L, V, ld = _tlogits(tlogits, vocab)
    cand_id = np.ascontiguousarray(cand_id, np.int32)
    path_slot = np.ascontiguousarray(path_slot, np.int32)
    q = None if q is None else np.ascontiguousarray(q, np.float64)
    ua = None if u_acc is None else np.ascontiguousarray(u_acc, np.float32)
    ur = None if u_res is None else np.ascontiguousarray(u_res, np.float32)
    out = dict(n_acc=np.empty(B, np.int32), out_tok=np.empty((B, L + 1), np.int32),
               m_acc=np.empty((B, L), np.float64), m_draw=np.empty(B, np.float64))
    _check(_load().ora_verify(_p(tl), dt, B, L, V, ld, _p(cand_id), _p(path_slot), _p(q), int(mode),
                              float(T), _p(ua), _p(ur), _p(out["n_acc"]), _p(out["out_tok"]),
                              _p(out["m_acc"]), _p(out["m_draw"])), "verify")
    return out


def verify_draw(tlogits, b: int, t: int, residual: bool, cand_id=None, q=None, mode: int = SAMPLED,
                T: float = 1.0, u_res=None, vocab: Optional[int] = None):
    """The extra token of block ``b`` drawn at position ``t`` (see
    ``ora_verify_draw``): returns ``(token, margin)``."""
    tl, dt, B, L, V, ld = _tlogits(tlogits, vocab)
    cand_id = None if cand_id is None else np.ascontiguousarray(cand_id, np.int32)
    q = None if q is None else np.ascontiguousarray(q, np.float64)
    ur = None if u_res is None else np.ascontiguousarray(u_res, np.float32)
    tok = C.c_int(0)
    mg = C.c_double(0)
    _check(_load().ora_verify_draw(_p(tl), dt, B, L, V, ld, _p(cand_id), _p(q), int(mode), float(T),
                                   _p(ur), int(b), int(t), int(bool(residual)), C.byref(tok), C.byref(mg)),
           "verify_draw")
    return tok.value, mg.value


def dyn_conv(x, x_prev, base, W_c):
    """Dynamic two-tap short convolution (see ``ora_dyn_conv``): bf16 bits in
    (``x [B,L,d]``, ``x_prev [B,d]``, ``base [2,d]``, ``W_c [2d/16, d]``);
    returns fp64 ``y [B,L,d]`` and the corrections ``corr [B,L,2d/16]``."""
    x = np.ascontiguousarray(x, np.uint16)
    x_prev = np.ascontiguousarray(x_prev, np.uint16)
    base = np.ascontiguousarray(base, np.uint16)
    W_c = np.ascontiguousarray(W_c, np.uint16)
    B, L, d = x.shape
    assert x_prev.shape == (B, d) and base.shape == (2, d) and W_c.shape == (2 * (d // 16), d)
    y = np.empty((B, L, d), np.float64)
    corr = np.empty((B, L, 2 * (d // 16)), np.float64)
    _check(_load().ora_dyn_conv(_p(x), _p(x_prev), _p(base), _p(W_c), B, L, d, _p(y), _p(corr)), "dyn_conv")
    return y, corr


def lmhead_topk(h, W):
    """LM head and top-16 (see ``ora_lmhead_topk``): ``h [rows, d]``,
    ``W [V, d]`` as bf16 bits; returns ``cand_id [rows, 16]`` int32 and the
    fp64 values of the 17 best, ``cand_z [rows, 17]``."""
    h = np.ascontiguousarray(h, np.uint16)
    W = np.ascontiguousarray(W, np.uint16)
    rows, d = h.shape
    V = W.shape[0]
    assert W.shape == (V, d)
    cid = np.empty((rows, K), np.int32)
    cz = np.empty((rows, K + 1), np.float64)
    _check(_load().ora_lmhead_topk(_p(h), _p(W), rows, V, d, _p(cid), _p(cz)), "lmhead_topk")
    return cid, cz


# ------------------------------------------------------------ ragged batches --
# Block size is a per-request knob ("DFlash 2: Keep Drafting Parallel",
# supplementary deployment notes: oMLX runs blocks of 5, the release tables use
# 8 and 16; "DFlash 2: The Drafter Stopped Guessing Alone", "What to check on
# your own serving": the block size is a knob).  A ragged batch keeps the
# padded [batch, block] layout and gives each block its own length
# block_len[b] in 0..block; block b is then exactly the selector (or
# verification) run on that block alone at that length.  Padding positions
# have no result: NaN (floats) and -1 (ids) here.


def _lens(block_len, B: int, L: int) -> np.ndarray:
    lens = np.asarray(block_len, np.int64).reshape(-1)
    if lens.shape != (B,) or (lens < 0).any() or (lens > L).any():
        raise ValueError(f"block_len must be [{B}] with entries in 0..{L}")
    return lens


def run_ragged(inp: Dict[str, np.ndarray], block_len, mode: int = GREEDY, T: float = 1.0,
               vocab: Optional[int] = None):
    """The whole selector on a ragged batch: block ``b`` is ``run`` on its
    first ``block_len[b]`` positions alone; padding is NaN / -1."""
    B, L = inp["logits"].shape[:2]
    lens = _lens(block_len, B, L)
    r = inp["W_A"].shape[0]
    out = dict(cand_id=np.full((B, L, K), -1, np.int32), cand_u=np.full((B, L, K), np.nan, np.float32),
               A_prev=np.full((B, L, K, r), np.nan), B_cur=np.full((B, L, K, r), np.nan),
               G=np.full((B, L, r), np.nan), S=np.full((B, L, K, K), np.nan),
               path_tok=np.full((B, L), -1, np.int32), path_slot=np.full((B, L), -1, np.int32),
               path_s=np.full((B, L), np.nan), aux=np.full((B, L), np.nan), q=np.full((B, L, K), np.nan))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        sub = dict(inp)
        for k in ("logits", "h", "uniforms"):
            if k in inp and inp[k] is not None:
                sub[k] = np.ascontiguousarray(inp[k][b:b + 1, :n])
        sub["verified"] = np.ascontiguousarray(inp["verified"][b:b + 1])
        o = run(sub, mode, T, vocab)
        for k in out:
            out[k][b, :n] = o[k][0]
    return out


def verify_ragged(tlogits, block_len, cand_id, path_slot, q=None, mode: int = GREEDY, T: float = 1.0,
                  u_acc=None, u_res=None, vocab: Optional[int] = None):
    """Verification of a ragged batch: target rows ``[B, L+1, ld]``, block
    ``b`` verified on its rows ``0 .. block_len[b]`` alone (row ``block_len[b]``
    follows its last drafted token).  ``out_tok [B, L+1]`` holds the accepted
    tokens, the extra token, then -1."""
    tl = np.ascontiguousarray(tlogits)
    B, L1 = tl.shape[:2]
    L = L1 - 1
    lens = _lens(block_len, B, L)
    out = dict(n_acc=np.zeros(B, np.int32), out_tok=np.full((B, L + 1), -1, np.int32),
               m_acc=np.full((B, L), np.nan), m_draw=np.full(B, np.nan))
    for b in range(B):
        n = int(lens[b])
        sl = lambda a: None if a is None else np.ascontiguousarray(a[b:b + 1, :n])
        o = verify(tl[b:b + 1, :n + 1], sl(cand_id), sl(path_slot), sl(q), mode, T, sl(u_acc),
                   None if u_res is None else np.ascontiguousarray(u_res[b:b + 1]), vocab)
        out["n_acc"][b] = o["n_acc"][0]
        out["out_tok"][b, :n + 1] = o["out_tok"][0]
        out["m_acc"][b, :n] = o["m_acc"][0]
        out["m_draw"][b] = o["m_draw"][0]
    return out


def dyn_conv_ragged(x, x_prev, base, W_c, block_len):
    """Dynamic convolution of a ragged batch: block ``b`` is ``dyn_conv`` on
    its first ``block_len[b]`` positions alone; padding is NaN."""
    B, L, d = x.shape
    lens = _lens(block_len, B, L)
    y = np.full((B, L, d), np.nan)
    corr = np.full((B, L, 2 * (d // 16)), np.nan)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        yb, cb = dyn_conv(x[b:b + 1, :n], x_prev[b:b + 1], base, W_c)
        y[b, :n] = yb[0]
        corr[b, :n] = cb[0]
    return y, corr


def time_selector(inp: Dict[str, np.ndarray], mode: int = GREEDY, T: float = 1.0):
    """The whole selector on ``inp`` with each stage timed inside the C library
    on the monotonic clock.  Returns ``(path_slot, seconds per stage, OpenMP
    threads)``; the stages are top-16, projections, scores, walk."""
    logits = np.ascontiguousarray(inp["logits"])
    B, L, V = logits.shape
    dt = 1 if logits.dtype == np.uint16 else 0
    E, W_A, W_B, W_H, h = (np.ascontiguousarray(inp[k]) for k in ("E", "W_A", "W_B", "W_H", "h"))
    ver = np.ascontiguousarray(inp["verified"], np.int32)
    u = np.ascontiguousarray(inp["uniforms"], np.float32) if mode == SAMPLED else None
    slot = np.empty((B, L), np.int32)
    sec = np.zeros(4, np.float64)
    nt = C.c_int(0)
    rc = _load().ora_time_selector(_p(logits), dt, V, _p(E), E.shape[1], _p(W_A), _p(W_B), _p(W_H), W_A.shape[0],
                                   _p(h), _p(ver), _p(u), float(T), int(mode), B, L, _p(slot), _p(sec), C.byref(nt))
    _check(rc, "time_selector")
    return slot, dict(zip(("select_topk", "project", "score_pairs", "walk"), sec.tolist())), int(nt.value)
