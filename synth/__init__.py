"""Seeded synthetic inputs for the DFlash 2 path selector.

This module only *draws* inputs: logits, the token-embedding table, the three
selector weights, drafter hidden states, the last verified token of every block
and the caller-side uniforms of the sampled walk.  It holds none of the
selector's arithmetic, and both the CPU oracle (``oracle/``) and the HIP path
consume exactly the arrays it returns.

Shapes and distributions follow the five workloads the selector is measured on
(drafter shapes from "DFlash 2: Keep Drafting Parallel", Setup section: block 16
for the 4B/30B-class drafters and block 8 for the 27B-class one; the vocab and
width of each class are fixed by the workload descriptions below).  The pages
publish no dataset-free workload, so these stand in for the GSM8K / MATH-500 /
HumanEval / MBPP / MT-Bench runs the pages measure on.

Readings of the workload text:
  * ``W ~ N(0, 1/d)`` (tiny) and ``W ~ N(0, 1/sqrt d)`` (others) both mean a
    standard deviation of ``1/sqrt(d)``.
  * "Gumbel(0,1)*3 plus a Zipf-ranked prior" is ``x_v = 3 g_v - ln(v + 1)``
    with ``g`` standard Gumbel, exponent 1 and rank = token id + 1.
  * The tiny workload's "+4 to one random token" and "repeat of the previous
    position's top token at 30 % of positions" are applied in that order, the
    repeat setting the previous position's arg-max token to the row max + 1.

Randomness: every tensor (and, for the big ones, every row or row chunk) has its
own ``numpy.random.SeedSequence`` child keyed by ``(seed, tensor, index)``, so a
subset of blocks or table rows can be regenerated on its own and the result
never depends on the number of worker threads.

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even
from float32).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, Optional

import numpy as np

K = 16  # candidates kept per draft position

# tensor tags for SeedSequence spawn keys
_T_LOGITS, _T_E, _T_WA, _T_WB, _T_WH, _T_H, _T_VER, _T_U, _T_INJ = range(1, 10)
_T_TGT, _T_UACC, _T_URES = range(10, 13)
_T_CX, _T_CXP, _T_CB, _T_CW = range(13, 17)  # dynamic convolution inputs
_T_LEN = 17  # per-block lengths of a ragged batch
_E_CHUNK = 256  # rows of E per seed child


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    block: int
    vocab: int
    d: int
    r: int
    logits_dtype: str  # "f32" or "bf16"
    logit_kind: str  # "tiny" or "gumbel_zipf"
    e_std: float
    walk: str  # "greedy", "sampled" or "both"
    temperature: float = 1.0

    @property
    def rows(self) -> int:
        return self.batch * self.block

    @property
    def w_std(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    # 4 blocks x 8 positions, vocab 1024, d=64, r=32, fp32 logits, greedy.
    "c0": Config("c0", 4, 8, 1024, 64, 32, "f32", "tiny", 1.0, "greedy"),
    # Qwen3-4B-like drafter, latency shape (one block of 16).
    "c1": Config("c1", 1, 16, 151936, 2560, 256, "bf16", "gumbel_zipf", 0.02, "greedy"),
    # Same shapes, 64 blocks: batched throughput.
    "c2": Config("c2", 64, 16, 151936, 2560, 256, "bf16", "gumbel_zipf", 0.02, "greedy"),
    # 27B-class drafter: 128 blocks of 8, d=5120, sampled walk at T=1.
    "c3": Config("c3", 128, 8, 152064, 5120, 256, "bf16", "gumbel_zipf", 0.02, "sampled"),
    # 30B-class drafter: 256 blocks of 16, d=6144, fp32 logits, both walks.
    "c4": Config("c4", 256, 16, 202048, 6144, 256, "f32", "gumbel_zipf", 0.02, "both"),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are always finite, so no NaN special case is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def _gumbel_zipf_row(rng: np.random.Generator, prior: np.ndarray) -> np.ndarray:
    u = rng.random(prior.shape[0], dtype=np.float32)
    u[u == 0.0] = np.float32(2.0 ** -25)  # keep -log(-log u) finite
    g = -np.log(-np.log(u))
    return np.float32(3.0) * g + prior


def _logits_block(cfg: Config, seed: int, b: int, prior: Optional[np.ndarray]) -> np.ndarray:
    """Float32 logits of one block, shape [block, vocab]."""
    L, V = cfg.block, cfg.vocab
    out = np.empty((L, V), dtype=np.float32)
    for t in range(L):
        rng = _rng(seed, _T_LOGITS, b * L + t)
        if cfg.logit_kind == "tiny":
            out[t] = rng.standard_normal(V, dtype=np.float32)
        else:
            out[t] = _gumbel_zipf_row(rng, prior)
    if cfg.logit_kind == "tiny":
        inj = _rng(seed, _T_INJ, b)
        spike = inj.integers(0, V, size=L)
        coin = inj.random(L)
        for t in range(L):
            out[t, spike[t]] += np.float32(4.0)
            if t >= 1 and coin[t] < 0.3:
                tau = int(np.argmax(out[t - 1]))  # previous position's top token
                out[t, tau] = out[t].max() + np.float32(1.0)
    return out


def make_logits(cfg: Config, seed: int = 0, blocks: Optional[Iterable[int]] = None) -> np.ndarray:
    """Logits ``[nb, block, vocab]`` (float32, or uint16 bf16 bits)."""
    blocks = list(range(cfg.batch)) if blocks is None else list(blocks)
    prior = None
    if cfg.logit_kind == "gumbel_zipf":
        prior = (-np.log(np.arange(1, cfg.vocab + 1, dtype=np.float64))).astype(np.float32)
    dt = np.float32 if cfg.logits_dtype == "f32" else np.uint16
    out = np.empty((len(blocks), cfg.block, cfg.vocab), dtype=dt)

    def one(i):
        x = _logits_block(cfg, seed, blocks[i], prior)
        out[i] = x if cfg.logits_dtype == "f32" else f32_to_bf16_bits(x)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(blocks))))
    return out


def make_E(cfg: Config, seed: int = 0) -> np.ndarray:
    """Token-embedding table ``E[vocab, d]`` as bf16 bits."""
    V, d = cfg.vocab, cfg.d
    E = np.empty((V, d), dtype=np.uint16)
    nchunk = (V + _E_CHUNK - 1) // _E_CHUNK

    def one(c):
        lo, hi = c * _E_CHUNK, min(V, (c + 1) * _E_CHUNK)
        E[lo:hi] = _normal_bf16(_rng(seed, _T_E, c), (hi - lo, d), cfg.e_std)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(nchunk)))
    return E


def make_weights(cfg: Config, seed: int = 0):
    """``W_A, W_B, W_H``, each ``[r, d]`` bf16 bits (linear-layer layout)."""
    return tuple(_normal_bf16(_rng(seed, tag), (cfg.r, cfg.d), cfg.w_std) for tag in (_T_WA, _T_WB, _T_WH))


def make_h(cfg: Config, seed: int = 0, blocks: Optional[Iterable[int]] = None) -> np.ndarray:
    """Drafter hidden states ``h[nb, block, d]`` as bf16 bits."""
    blocks = list(range(cfg.batch)) if blocks is None else list(blocks)
    return np.stack([_normal_bf16(_rng(seed, _T_H, b), (cfg.block, cfg.d), 1.0) for b in blocks]) \
        if blocks else np.empty((0, cfg.block, cfg.d), np.uint16)


def make_verified(cfg: Config, seed: int = 0) -> np.ndarray:
    """Last verified token of each block, uniform over the vocab: ``[batch]`` int32."""
    return _rng(seed, _T_VER).integers(0, cfg.vocab, size=cfg.batch).astype(np.int32)


def make_uniforms(cfg: Config, seed: int = 0) -> np.ndarray:
    """Caller-side uniforms of the sampled walk, ``U[0,1)`` float32 ``[batch, block]``."""
    return _rng(seed, _T_U).random((cfg.batch, cfg.block), dtype=np.float32)


def make_target_logits(cfg: Config, seed: int = 0, blocks: Optional[Iterable[int]] = None,
                       noise: float = 1.0) -> np.ndarray:
    """Target-model logits for verifying each block: ``[nb, block + 1, vocab]``
    in the draft logits' dtype.  Row t < block is the draft's row t plus
    N(0, noise^2) per token (a target that mostly agrees with the drafter);
    row ``block`` (the token after the block) is a fresh draw of the same
    kind."""
    blocks = list(range(cfg.batch)) if blocks is None else list(blocks)
    prior = None
    if cfg.logit_kind == "gumbel_zipf":
        prior = (-np.log(np.arange(1, cfg.vocab + 1, dtype=np.float64))).astype(np.float32)
    dt = np.float32 if cfg.logits_dtype == "f32" else np.uint16
    L, V = cfg.block, cfg.vocab
    out = np.empty((len(blocks), L + 1, V), dtype=dt)

    def one(i):
        b = blocks[i]
        x = np.empty((L + 1, V), np.float32)
        x[:L] = _logits_block(cfg, seed, b, prior)
        for t in range(L):
            x[t] += np.float32(noise) * _rng(seed, _T_TGT, b * (L + 1) + t).standard_normal(V, dtype=np.float32)
        rng = _rng(seed, _T_TGT, b * (L + 1) + L)
        x[L] = _gumbel_zipf_row(rng, prior) if prior is not None else rng.standard_normal(V, dtype=np.float32)
        out[i] = x if cfg.logits_dtype == "f32" else f32_to_bf16_bits(x)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(blocks))))
    return out


def make_verify_uniforms(cfg: Config, seed: int = 0):
    """Caller-side uniforms of the sampled verification: ``u_acc [batch, block]``
    (one per acceptance test) and ``u_res [batch]`` (the extra token's draw)."""
    return (_rng(seed, _T_UACC).random((cfg.batch, cfg.block), dtype=np.float32),
            _rng(seed, _T_URES).random(cfg.batch, dtype=np.float32))


def make_conv(cfg: Config, seed: int = 0, blocks: Optional[Iterable[int]] = None) -> Dict[str, np.ndarray]:
    """Inputs of one dynamic two-tap convolution unit at the drafter's width d,
    as bf16 bits: ``x [nb, block, d]`` ~ N(0, 1) (the hidden state entering
    the unit), ``x_prev [nb, d]`` ~ N(0, 1) (the last verified token's),
    ``base [2, d]`` with tap 0 ~ 1 + N(0, 0.1^2) and tap 1 ~ N(0, 0.1^2) (a
    near-identity learned kernel), ``W_c [2 d / 16, d]`` ~ N(0, (0.1/sqrt d)^2)
    (a small correction)."""
    blocks = list(range(cfg.batch)) if blocks is None else list(blocks)
    d = cfg.d
    x = np.stack([_normal_bf16(_rng(seed, _T_CX, b), (cfg.block, d), 1.0) for b in blocks]) \
        if blocks else np.empty((0, cfg.block, d), np.uint16)
    xp = np.stack([_normal_bf16(_rng(seed, _T_CXP, b), (d,), 1.0) for b in blocks]) \
        if blocks else np.empty((0, d), np.uint16)
    rb = _rng(seed, _T_CB)
    base = np.empty((2, d), np.float32)
    base[0] = 1.0 + 0.1 * rb.standard_normal(d, dtype=np.float32)
    base[1] = 0.1 * rb.standard_normal(d, dtype=np.float32)
    W_c = _normal_bf16(_rng(seed, _T_CW), (2 * (d // 16), d), 0.1 / np.sqrt(d))
    return dict(x=x, x_prev=xp, base=f32_to_bf16_bits(base), W_c=W_c)


def make_block_len(cfg: Config, seed: int = 0, choices: Optional[Iterable[int]] = None) -> np.ndarray:
    """Per-block lengths of a ragged batch, ``[batch]`` int32 in ``0..block``,
    each drawn uniformly from ``choices``.  The default mix is the block sizes
    the pages run (5 on oMLX, 8 and 16 in the release tables) that fit
    ``cfg.block``, plus ``cfg.block`` itself."""
    if choices is None:
        choices = sorted({c for c in (5, 8, 16) if c <= cfg.block} | {cfg.block})
    choices = np.asarray(list(choices), np.int64)
    if choices.size == 0 or (choices < 0).any() or (choices > cfg.block).any():
        raise ValueError("block lengths must lie in 0..block")
    return choices[_rng(seed, _T_LEN).integers(0, choices.size, size=cfg.batch)].astype(np.int32)


def make(cfg: Config, seed: int = 0) -> Dict[str, np.ndarray]:
    """All inputs of one selector call for workload ``cfg``."""
    W_A, W_B, W_H = make_weights(cfg, seed)
    return dict(
        logits=make_logits(cfg, seed),
        E=make_E(cfg, seed),
        W_A=W_A, W_B=W_B, W_H=W_H,
        h=make_h(cfg, seed),
        verified=make_verified(cfg, seed),
        uniforms=make_uniforms(cfg, seed),
    )


def sub_blocks(inp: Dict[str, np.ndarray], blocks) -> Dict[str, np.ndarray]:
    """The inputs of a subset of blocks (blocks are independent of each other)."""
    blocks = np.asarray(blocks)
    out = dict(inp)
    for k in ("logits", "h", "verified", "uniforms"):
        out[k] = np.ascontiguousarray(inp[k][blocks])
    return out


def to_device(inp: Dict[str, np.ndarray], dev):
    """Upload drawn inputs as torch tensors: bf16 bit patterns become bfloat16."""
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    lg = inp["logits"]
    out = dict(logits=bf(lg) if lg.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(lg)).to(dev))
    for k in ("E", "W_A", "W_B", "W_H", "h"):
        out[k] = bf(inp[k])
    out["verified"] = torch.from_numpy(np.ascontiguousarray(inp["verified"], np.int32)).to(dev)
    out["uniforms"] = torch.from_numpy(np.ascontiguousarray(inp["uniforms"], np.float32)).to(dev)
    return out
