"""Pins of the oracle's DFlash 2 grouped dynamic two-tap conv.

Sources: [Code] sections 13 (the two-tap formula, the base + correction
coefficients with one correction per 16 channels, the block's first position,
the parameter figure) and 14 (the base kernel and projection shapes).
"""
import numpy as np
import pytest
from scipy.signal import lfilter

from oracle import dflash_oracle as O


def _rand(seed, D=64, gs=16, n_seqs=2, bl=4):
    r = np.random.default_rng(seed)
    G = D // gs
    x = r.standard_normal((n_seqs * bl, D))
    prev = r.standard_normal((n_seqs, D))
    base = r.standard_normal((2, 2, D)) * 0.5
    proj = r.standard_normal((4 * G, D)) * 0.1
    return x, prev, base, proj


def test_parameter_count_matches_the_pages_figure():
    # [Code] section 13 gives +16.5M parameters for the conv modules of the
    # 5-layer drafter of Qwen3-4B (hidden width 2560), one correction per 16
    # channels. The (2, taps, hidden) base and the 2 * taps * groups outputs
    # of the projection reproduce it; readings with one call's outputs, or
    # with a correction per channel, do not.
    n = O.dynamic_conv_param_count(2560, 16, 5)
    assert round(n / 1e6, 1) == 16.5
    one_call = 5 * 2 * (2 * 2 * 2560 + 2560 * 2 * (2560 // 16))
    per_channel = 5 * 2 * (2 * 2 * 2560 + 2560 * 2 * 2 * 2560)
    assert round(one_call / 1e6, 1) != 16.5 and round(per_channel / 1e6, 1) != 16.5


def test_zero_projection_is_a_causal_fir_filter_per_channel():
    # with no correction each channel is a fixed two-tap causal filter over
    # the sequence [prev, x_0 .. x_{Bl-1}] (scipy's lfilter)
    x, prev, base, proj = _rand(1)
    y, corr = O.dynamic_conv_prepare(x, prev, 4, base, np.zeros_like(proj), 16)
    assert np.all(corr == 0)
    for s in range(2):
        for c in range(x.shape[1]):
            seq = np.concatenate([[prev[s, c]], x[s * 4:(s + 1) * 4, c]])
            want = lfilter([base[0, 0, c], base[0, 1, c]], [1.0], seq)[1:]
            np.testing.assert_allclose(y[s * 4:(s + 1) * 4, c], want, rtol=1e-13, atol=1e-13)


def test_identity_and_shift_kernels():
    x, prev, base, proj = _rand(2)
    z = np.zeros_like(proj)
    ident = np.zeros_like(base); ident[0, 0] = 1.0
    y, _ = O.dynamic_conv_prepare(x, prev, 4, ident, z, 16)
    np.testing.assert_array_equal(y, x)
    shift = np.zeros_like(base); shift[0, 1] = 1.0
    y, _ = O.dynamic_conv_prepare(x, prev, 4, shift, z, 16)
    for s in range(2):
        np.testing.assert_array_equal(y[s * 4], prev[s])
        np.testing.assert_array_equal(y[s * 4 + 1:(s + 1) * 4], x[s * 4:(s + 1) * 4 - 1])


def test_brute_force_tiny():
    # element by element in plain Python: coefficient of channel c, tap j at
    # row m = base[call][j][c] + sum_i proj[(call * 2 + j) * G + c // gs][i] * x[m][i]
    D, gs, bl = 32, 16, 3
    x, prev, base, proj = _rand(3, D=D, gs=gs, n_seqs=2, bl=bl)
    G = D // gs
    y, corr = O.dynamic_conv_prepare(x, prev, bl, base, proj, gs)
    z = np.random.default_rng(33).standard_normal(x.shape)
    zprev = np.random.default_rng(34).standard_normal(prev.shape)
    y2 = O.dynamic_conv_finish(z, zprev, bl, base, corr, gs)
    for m in range(x.shape[0]):
        s, t = divmod(m, bl)
        for c in range(D):
            g = c // gs
            def coef(call, j):
                acc = 0.0
                for i in range(D):
                    acc += proj[(call * 2 + j) * G + g][i] * x[m][i]
                return base[call][j][c] + acc
            before = prev[s][c] if t == 0 else x[m - 1][c]
            want = coef(0, 0) * x[m][c] + coef(0, 1) * before
            assert abs(y[m][c] - want) <= 1e-12 * (1 + abs(want))
            zb = zprev[s][c] if t == 0 else z[m - 1][c]
            want2 = coef(1, 0) * z[m][c] + coef(1, 1) * zb
            assert abs(y2[m][c] - want2) <= 1e-12 * (1 + abs(want2))


def test_one_correction_per_group():
    # a projection that only feeds group g's tap-0 correction of the prepare
    # call changes exactly that group's channels, by the same factor times x
    x, prev, base, proj = _rand(4, D=64, gs=16)
    G = 4
    only = np.zeros_like(proj)
    only[0 * G + 2] = proj[2]       # call 0, tap 0, group 2
    y0, _ = O.dynamic_conv_prepare(x, prev, 4, base, np.zeros_like(proj), 16)
    y1, _ = O.dynamic_conv_prepare(x, prev, 4, base, only, 16)
    d = y1 - y0
    assert np.all(d[:, :32] == 0) and np.all(d[:, 48:] == 0)
    factor = x @ proj[2]
    np.testing.assert_allclose(d[:, 32:48], factor[:, None] * x[:, 32:48], rtol=1e-12, atol=1e-12)


def test_blocks_do_not_read_each_other():
    x, prev, base, proj = _rand(5, n_seqs=3, bl=4)
    y, _ = O.dynamic_conv_prepare(x, prev, 4, base, proj, 16)
    x2 = x.copy(); x2[4:8] += 1.0
    y2, _ = O.dynamic_conv_prepare(x2, prev, 4, base, proj, 16)
    np.testing.assert_array_equal(y[:4], y2[:4])
    np.testing.assert_array_equal(y[8:], y2[8:])


def test_finish_takes_the_second_half():
    # zeroing the call-0 rows of the projection leaves the prepare call a
    # fixed filter, while its finish half is unchanged
    x, prev, base, proj = _rand(6)
    G = 4
    p2 = proj.copy(); p2[:2 * G] = 0
    y_a, c_a = O.dynamic_conv_prepare(x, prev, 4, base, p2, 16)
    y_b, _ = O.dynamic_conv_prepare(x, prev, 4, base, np.zeros_like(proj), 16)
    _, c_full = O.dynamic_conv_prepare(x, prev, 4, base, proj, 16)
    np.testing.assert_array_equal(y_a, y_b)
    np.testing.assert_allclose(c_a, c_full, rtol=1e-14, atol=0)
    np.testing.assert_allclose(c_full, x @ proj[2 * G:].T, rtol=1e-12, atol=1e-12)
    # a mistaken half (call 0's corrections) would differ
    assert not np.allclose(c_full, x @ proj[:2 * G].T)


def test_block_length_one():
    x, prev, base, proj = _rand(7, n_seqs=3, bl=1)
    y, _ = O.dynamic_conv_prepare(x, prev, 1, base, proj, 16)
    for m in range(3):
        k = O.dynamic_conv_coefficients(x[m], base[0], proj, 16, 0)
        np.testing.assert_allclose(y[m], k[0] * x[m] + k[1] * prev[m], rtol=1e-13, atol=1e-13)
