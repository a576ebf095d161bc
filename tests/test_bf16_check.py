"""The rounding-exactness check used by the GPU tests of the bf16 outputs
(fused context, injected K/V): it accepts one rounding of a value close to the
exact one, and rejects the mistakes it is there to catch - a double rounding
(the projection rounded to bf16 before the norm, then again after it) and a
one-step error. Mistakes are planted in copies of the oracle's result, on the
CPU."""
import numpy as np

import oracle as O
from bf16_check import bf16_neighbours, check_bf16_rounding, midpoint_distance, row_rms

# the band the GPU tests use for the fusion at D = 4096 (8 sigma of an fp32
# accumulation of 5D products), wider than this D = 512 case needs
BAND = 5e-5


def _fused(D=512, T=64, seed=0):
    rng = np.random.default_rng(seed)
    feats = [rng.standard_normal((T, D)) for _ in range(5)]
    w_c = O.round_bf16(0.02 * rng.standard_normal((D, 5 * D)))
    gain = np.ones(D)
    c = np.concatenate(feats, axis=-1)
    y = O.linear(c, w_c)
    return y, gain, O.rms_norm(y, gain, 1e-6)


def test_midpoints_and_neighbours():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -9, -3.0 - 2 ** -7])
    lo, hi = bf16_neighbours(x)
    np.testing.assert_array_equal(lo, [1.0, 1.0, 1.0, -3.0])
    np.testing.assert_array_equal(hi, [1.0 + 2 ** -7, 1.0 + 2 ** -7, 1.0 + 2 ** -7, -3.0 - 2 ** -6])
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7
    # (the bf16 step at 3 is 2^-6, so -3 - 2^-7 is a midpoint too)
    np.testing.assert_allclose(midpoint_distance(x), [2 ** -8, 0.0, 2 ** -9, 0.0], atol=0)


def test_single_rounding_passes_with_few_banded_values():
    _, _, H = _fused()
    # a perturbation well inside the band (as an fp32 evaluation would leave)
    pert = H * (1.0 + 1e-7 * np.random.default_rng(1).standard_normal(H.shape))
    bad, banded, n = check_bf16_rounding(O.round_bf16(pert), H, BAND * row_rms(H))
    assert bad == 0
    assert banded < 0.15 * n


def test_double_rounding_fails():
    y, gain, H = _fused()
    twice = O.round_bf16(O.rms_norm(O.round_bf16(y), gain, 1e-6))
    bad, _, n = check_bf16_rounding(twice, H, BAND * row_rms(H))
    assert bad > 0.1 * n, (bad, n)


def test_tiny_values_accept_the_band_not_more():
    # below the band a bf16 step is finer than the fp32 error: every bf16
    # value within the band is accepted, one just outside it is not
    ref = np.array([1.4365e-5, -2.84e-5, 0.75])
    band = np.array([3e-6, 3e-6, 3e-6])
    ok = O.round_bf16(ref + np.array([2.5e-6, -2.0e-6, 0.0]))
    assert check_bf16_rounding(ok, ref, band)[0] == 0
    off = O.round_bf16(ref + np.array([4e-6, 0.0, 0.0]))
    assert check_bf16_rounding(off, ref, band)[0] == 1


def test_one_step_error_fails():
    _, _, H = _fused()
    out = O.round_bf16(H)
    flat = out.reshape(-1).copy()
    lo, hi = bf16_neighbours(flat[17:18])
    flat[17] = hi[0] if flat[17] == lo[0] else lo[0]
    bad, _, _ = check_bf16_rounding(flat.reshape(H.shape), H, BAND * row_rms(H))
    assert bad == (0 if midpoint_distance(H.reshape(-1)[17]) <= BAND * row_rms(H).reshape(-1)[17 // 512] else 1)
