"""dyn_conv on the GPU against the oracle.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Local Convolution,
eq. Conv_k; "DFlash 2: The Drafter Stopped Guessing Alone", section "The decay
at the end of the block".)

Tolerance, derived from the arithmetic.  The GPU forms each correction as an
fp32 sum of exact bf16 x bf16 products, so it is within gamma_d * sum |w x|
of the fp64 value in any summation order (gamma_d = d u / (1 - d u),
u = 2^-24).  Each coefficient adds one rounding of base + corr, and the two
taps two more roundings of products and one of their sum; the result is then
rounded to bf16, at most half a bf16 ulp = 2^-8 |y| relative.  The test
applies that bound element by element (first order in u, with 1% slack)."""
import numpy as np
import pytest
import torch

import draft_selection_amd as ds
import synth

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def _f(u):
    return synth.bf16_bits_to_f32(u).astype(np.float64)


def _rand(seed, B, L, d, x_std=1.0, w_scale=1.0):
    rng = np.random.default_rng(seed)
    G = d // 16
    return dict(
        x=synth.f32_to_bf16_bits((rng.standard_normal((B, L, d)) * x_std).astype(np.float32)),
        x_prev=synth.f32_to_bf16_bits(rng.standard_normal((B, d)).astype(np.float32)),
        base=synth.f32_to_bf16_bits(np.stack([1 + 0.1 * rng.standard_normal(d), 0.1 * rng.standard_normal(d)])
                                    .astype(np.float32)),
        W_c=synth.f32_to_bf16_bits((rng.standard_normal((2 * G, d)) * w_scale / np.sqrt(d)).astype(np.float32)),
    )


def _run(inp, dev):
    t = {k: _dev(v, dev) for k, v in inp.items()}
    y = ds.dyn_conv(t["x"], t["x_prev"], t["base"], t["W_c"])
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def _bound(inp, y, corr):
    """Element-wise error bound of the GPU result (module doc)."""
    x, xp, base, W = (_f(inp[k]) for k in ("x", "x_prev", "base", "W_c"))
    B, L, d = x.shape
    G = d // 16
    prev = np.concatenate([xp[:, None], x[:, :-1]], axis=1)
    cabs = np.abs(x) @ np.abs(W).T                       # sum |w x| per correction
    gam = d * U / (1 - d * U)
    ec = gam * cabs                                      # [B, L, 2G]
    grp = np.arange(d) // 16
    k0 = base[0] + corr[..., grp]
    k1 = base[1] + corr[..., G + grp]
    ek0 = ec[..., grp] + U * np.abs(k0)
    ek1 = ec[..., G + grp] + U * np.abs(k1)
    e32 = np.abs(x) * ek0 + np.abs(prev) * ek1 + 2 * U * (np.abs(k0 * x) + np.abs(k1 * prev))
    return 2.0 ** -8 * np.abs(y) + 1.01 * e32 + 1e-30


def _check(ora, inp, dev):
    got = _f(_run(inp, dev))
    y, corr = ora.dyn_conv(inp["x"], inp["x_prev"], inp["base"], inp["W_c"])
    err = np.abs(got - y)
    bnd = _bound(inp, y, corr)
    worst = np.unravel_index(np.argmax(err - bnd), err.shape)
    assert np.all(err <= bnd), f"y off by {err[worst]} > {bnd[worst]} at {worst}"
    return got, y


@pytest.mark.parametrize("B,L,d", [
    (1, 1, 512),      # one position: only the verified token as predecessor
    (3, 5, 512),      # ragged row tile
    (4, 16, 1024),
    (2, 8, 2560),     # the 4B drafter's width, several splits
    (7, 3, 1536),
    (64, 16, 2560),   # 64 blocks x 16 positions at d 2560 (full)
    (128, 8, 5120),   # 128 blocks x 8 positions at d 5120 (full)
])
def test_dyn_conv_matches_oracle(ora, dev, B, L, d):
    _check(ora, _rand(B * 100 + L + d, B, L, d), dev)


def test_dyn_conv_large_workload_sampled_blocks(ora, dev):
    """256 blocks x 16 positions at d 6144 on the GPU; the oracle checks a
    sample of blocks (blocks are independent)."""
    cfg = synth.CONFIGS["c4"]
    inp = synth.make_conv(cfg)
    got = _f(_run(inp, dev))
    blocks = [0, 1, 127, 255]
    sub = dict(x=inp["x"][blocks], x_prev=inp["x_prev"][blocks], base=inp["base"], W_c=inp["W_c"])
    y, corr = ora.dyn_conv(sub["x"], sub["x_prev"], sub["base"], sub["W_c"])
    err = np.abs(got[blocks] - y)
    assert np.all(err <= _bound(sub, y, corr))


def test_dyn_conv_exact_integer_case(ora, dev):
    """Small integers, W_c = 0: every value is exact in fp32 and in bf16, so
    the GPU must match the oracle bit for bit."""
    rng = np.random.default_rng(11)
    B, L, d = 3, 6, 512
    inp = dict(
        x=synth.f32_to_bf16_bits(rng.integers(-4, 5, (B, L, d)).astype(np.float32)),
        x_prev=synth.f32_to_bf16_bits(rng.integers(-4, 5, (B, d)).astype(np.float32)),
        base=synth.f32_to_bf16_bits(rng.integers(-3, 4, (2, d)).astype(np.float32)),
        W_c=np.zeros((2 * d // 16, d), np.uint16),
    )
    got = _f(_run(inp, dev))
    y, _ = ora.dyn_conv(inp["x"], inp["x_prev"], inp["base"], inp["W_c"])
    assert np.array_equal(got, y)


def test_dyn_conv_deterministic_and_empty(dev):
    inp = _rand(5, 6, 16, 1024)
    a, b = _run(inp, dev), _run(inp, dev)
    assert np.array_equal(a, b)
    e = {k: _dev(v[:0] if k in ("x", "x_prev") else v, dev) for k, v in inp.items()}
    y = ds.dyn_conv(e["x"], e["x_prev"], e["base"], e["W_c"])
    assert y.shape == (0, 16, 1024)


def test_dyn_conv_rejects_bad_width(dev):
    x = torch.zeros((1, 2, 640), dtype=torch.bfloat16, device=dev)
    xp = torch.zeros((1, 640), dtype=torch.bfloat16, device=dev)
    base = torch.zeros((2, 640), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((80, 640), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError):
        ds.dyn_conv(x, xp, base, W, workspace=torch.empty(1 << 20, dtype=torch.uint8, device=dev))
