"""Pins of the oracle's dynamic two-tap short convolution.

("DFlash 2: Keep Drafting Parallel", Method > Lightweight Local Convolution,
eq. Conv_k: y_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1}, every coefficient a
learned base kernel plus a correction from the current hidden state shared by
16 channels, the first position reading the last verified token; "DFlash 2:
The Drafter Stopped Guessing Alone", section "The decay at the end of the block".)

The pages print no worked example.  The form of the correction map is pinned by
the published parameter count (golden file); the arithmetic by a library
convolution, a library matrix product, exact small-integer cases and the
locality and sharing properties the pages state."""
import numpy as np
import pytest

import oracle
import synth
from helpers import load_golden


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def _f(u):
    return synth.bf16_bits_to_f32(u).astype(np.float64)


def _rand(seed, B, L, d, w_std=None):
    rng = np.random.default_rng(seed)
    G = d // 16
    x = _bits(rng.standard_normal((B, L, d)))
    xp = _bits(rng.standard_normal((B, d)))
    base = _bits(rng.standard_normal((2, d)) * 0.5)
    W = _bits(rng.standard_normal((2 * G, d)) / np.sqrt(d) if w_std is None else rng.standard_normal((2 * G, d)) * w_std)
    return x, xp, base, W


def test_parameter_count_pins_the_correction_map():
    g = load_golden("conv_params.json")
    d, units, group, taps = g["drafter_width_d"], g["layers"] * g["units_per_layer"], g["channels_per_correction"], g["taps"]
    per_unit = taps * d + d * (taps * d // group)  # base kernel + bias-free d -> 2 d/16 map
    assert abs(units * per_unit - g["published_params"]) <= g["published_rounding"]
    shared = taps * d + d * (d // group)  # one correction for both taps
    assert abs(units * shared - g["published_params"]) > 10 * g["published_rounding"]


def test_zero_correction_is_a_plain_two_tap_convolution():
    """W_c = 0: every channel is the library convolution of the sequence
    [x_prev, x_0, ..., x_{L-1}] with the kernel (base_0, base_1)."""
    B, L, d = 3, 7, 32
    x, xp, base, W = _rand(1, B, L, d)
    W[:] = 0
    y, corr = oracle.dyn_conv(x, xp, base, W)
    assert np.all(corr == 0.0)
    X, XP, BS = _f(x), _f(xp), _f(base)
    for b in range(B):
        for c in range(d):
            seq = np.concatenate([[XP[b, c]], X[b, :, c]])
            want = np.convolve(seq, [BS[0, c], BS[1, c]])[1:L + 1]
            np.testing.assert_allclose(y[b, :, c], want, rtol=1e-15, atol=1e-15)


def test_correction_is_the_matrix_product_and_is_shared_by_16_channels():
    B, L, d = 2, 5, 64
    x, xp, base, W = _rand(2, B, L, d)
    y, corr = oracle.dyn_conv(x, xp, base, W)
    np.testing.assert_allclose(corr, _f(x) @ _f(W).T, rtol=1e-12, atol=1e-12)
    # with x_{t-1} = 0 (t = 0, x_prev = 0): y_t / x_t - base_0 is the tap-0
    # correction, constant over each group of 16 channels
    xp0 = np.zeros_like(xp)
    y0, corr0 = oracle.dyn_conv(x, xp0, base, W)
    X = _f(x)
    k0 = y0[:, 0] / X[:, 0] - _f(base)[0]
    G = d // 16
    for g in range(G):
        np.testing.assert_allclose(k0[:, 16 * g:16 * g + 16], corr0[:, 0, g:g + 1] * np.ones((1, 16)),
                                   rtol=1e-9, atol=1e-12)


def test_small_integers_are_exact():
    """Integer-valued inputs: every product and sum is exact, so y equals the
    integer arithmetic of the definition."""
    rng = np.random.default_rng(3)
    B, L, d = 2, 4, 32
    G = d // 16
    xi = rng.integers(-3, 4, size=(B, L, d))
    pi = rng.integers(-3, 4, size=(B, d))
    bi = rng.integers(-2, 3, size=(2, d))
    wi = rng.integers(-1, 2, size=(2 * G, d))
    y, corr = oracle.dyn_conv(_bits(xi), _bits(pi), _bits(bi), _bits(wi))
    for b in range(B):
        for t in range(L):
            prev = pi[b] if t == 0 else xi[b, t - 1]
            c = [int(sum(int(wi[n, k]) * int(xi[b, t, k]) for k in range(d))) for n in range(2 * G)]
            for ch in range(d):
                want = (int(bi[0, ch]) + c[ch // 16]) * int(xi[b, t, ch]) + (int(bi[1, ch]) + c[G + ch // 16]) * int(prev[ch])
                assert y[b, t, ch] == want


def test_reaches_exactly_one_position_back():
    """An impulse at position s (x_prev = 0) reaches positions s and s + 1 only."""
    B, L, d = 1, 8, 32
    _, _, base, W = _rand(4, B, L, d)
    rng = np.random.default_rng(5)
    for s in range(L):
        x = np.zeros((B, L, d), np.float32)
        x[0, s] = rng.standard_normal(d)
        y, _ = oracle.dyn_conv(_bits(x), _bits(np.zeros((B, d))), base, W)
        nz = np.flatnonzero(np.any(y[0] != 0.0, axis=1))
        assert set(nz) <= {s, s + 1} and s in nz


def test_first_position_reads_the_last_verified_token():
    B, L, d = 2, 6, 48
    x, xp, base, W = _rand(6, B, L, d)
    y1, _ = oracle.dyn_conv(x, xp, base, W)
    xp2 = _bits(np.random.default_rng(7).standard_normal((B, d)))
    y2, _ = oracle.dyn_conv(x, xp2, base, W)
    assert np.any(y1[:, 0] != y2[:, 0])
    assert np.array_equal(y1[:, 1:], y2[:, 1:])


def test_rejects_bad_shapes():
    x, xp, base, W = _rand(8, 1, 2, 32)
    with pytest.raises(AssertionError):
        oracle.dyn_conv(x, xp, base, W[:-1])
