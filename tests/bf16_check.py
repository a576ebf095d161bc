"""Rounding-exact comparison of a bf16 output with an fp64 oracle value.

A kernel that computes a value in fp32 and rounds it to bf16 once returns
round_bf16(v) for some v within its own fp32 error of the exact value. The
check therefore accepts exactly the bf16 values in
[round_bf16(exact - band), round_bf16(exact + band)], band being a stated
bound on that fp32 error. Where no rounding midpoint lies within the band
that interval is the single value round_bf16(exact): the output must be the
correctly rounded one. Near a midpoint both neighbours are accepted, and for
values so small that a bf16 step is below the band, every bf16 value within
the band is. Each caller states the band from the arithmetic of the kernel
it checks.
"""
import numpy as np

import oracle as O


def _bits(x):
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    return f.view(np.uint32).astype(np.uint64)


def _from_bits(u):
    return np.asarray(u, np.uint64).astype(np.uint32).view(np.float32).astype(np.float64)


def midpoint_distance(ref):
    """|ref - m|, m the rounding midpoint above |ref| (truncated bf16 + half a
    bf16 step, same sign); the midpoint below lies at least half a step away
    and cannot be reached by an fp32 error far smaller than a bf16 step."""
    u = _bits(ref)
    mid = _from_bits((u & 0xFFFF0000) | 0x8000)
    return np.abs(np.asarray(ref, np.float64) - mid)


def bf16_neighbours(ref):
    """The two bf16 values around ref: truncated toward zero and one step away."""
    u = _bits(ref)
    t = u & 0xFFFF0000
    return _from_bits(t), _from_bits(t + 0x10000)


def _accepted(ref, band):
    ref = np.asarray(ref, np.float64)
    band = np.broadcast_to(np.asarray(band, np.float64), ref.shape)
    return O.round_bf16(ref - band), O.round_bf16(ref + band)


def bad_bf16_rounding(out, ref, band):
    """Flat indices of the values check_bf16_rounding counts as wrong."""
    lo, hi = _accepted(ref, band)
    out = np.asarray(out, np.float64)
    return np.nonzero(((out < lo) | (out > hi)).reshape(-1))[0]


def check_bf16_rounding(out, ref, band):
    """Returns (n_bad, n_banded, n_total): n_bad counts outputs outside
    [round_bf16(ref - band), round_bf16(ref + band)]; n_banded counts the
    values where that interval holds more than one bf16 value (a rounding
    midpoint lies within the band)."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    lo, hi = _accepted(ref, band)
    return int(((out < lo) | (out > hi)).sum()), int((lo != hi).sum()), int(out.size)


def row_rms(x):
    x = np.asarray(x, np.float64)
    return np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
