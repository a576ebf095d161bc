"""Pins of the oracle's block attention."""
import math

import numpy as np

import oracle as O


def _brute(q, k, v):
    B, Hq, hd = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for r in range(B):
        for a in range(Hq):
            g = a // G
            s = [sum(q[r, a, d] * k[j, g, d] for d in range(hd)) / math.sqrt(hd)
                 for j in range(k.shape[0])]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for d in range(hd):
                out[r, a, d] = sum(e[j] * v[j, g, d] for j in range(k.shape[0])) / z
    return out


def test_matches_brute_force_gqa():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((4, 4, 8)); k = rng.standard_normal((9, 2, 8))
    v = rng.standard_normal((9, 2, 8))
    np.testing.assert_allclose(O.block_attention(q, k, v), _brute(q, k, v), atol=1e-12)


def test_head_grouping_is_contiguous():
    # head a reads kv head a // G: make kv head 1's values a constant 7
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 4, 4)); k = rng.standard_normal((5, 2, 4))
    v = rng.standard_normal((5, 2, 4)); v[:, 1, :] = 7.0
    o = O.block_attention(q, k, v)
    np.testing.assert_allclose(o[:, 2:, :], 7.0, atol=1e-12)
    assert np.abs(o[:, :2, :] - 7.0).min() > 1e-3


def test_special_cases():
    rng = np.random.default_rng(12)
    hd = 8
    q = rng.standard_normal((3, 2, hd))
    # all keys equal -> mean of V
    k = np.tile(rng.standard_normal((1, 1, hd)), (6, 1, 1))
    v = rng.standard_normal((6, 1, hd))
    np.testing.assert_allclose(O.block_attention(q, k, v), np.broadcast_to(v.mean(0), (3, 2, hd)), atol=1e-12)
    # one key -> that value
    k1 = rng.standard_normal((1, 1, hd)); v1 = rng.standard_normal((1, 1, hd))
    np.testing.assert_allclose(O.block_attention(q, k1, v1), np.broadcast_to(v1[0], (3, 2, hd)), atol=1e-12)


def test_no_mask_key_order_invariance():
    # bidirectional: permuting the keys (with their values) changes nothing, so
    # no key is hidden from any block row
    rng = np.random.default_rng(13)
    q = rng.standard_normal((4, 2, 8)); k = rng.standard_normal((10, 1, 8))
    v = rng.standard_normal((10, 1, 8))
    perm = rng.permutation(10)
    np.testing.assert_allclose(O.block_attention(q, k, v), O.block_attention(q, k[perm], v[perm]), atol=1e-12)
    # the first block row (the anchor) is influenced by the last key
    v2 = v.copy(); v2[-1] += 10.0
    assert np.abs(O.block_attention(q, k, v2)[0] - O.block_attention(q, k, v)[0]).max() > 1e-3


def test_scale_is_inverse_sqrt_head_dim():
    # two keys with scores differing by exactly sqrt(hd)*ln(3): weights 3/4, 1/4
    hd = 16
    q = np.zeros((1, 1, hd)); q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, hd)); k[0, 0, 0] = math.sqrt(hd) * math.log(3.0)
    v = np.zeros((2, 1, hd)); v[0, 0, 1] = 1.0; v[1, 0, 2] = 1.0
    o = O.block_attention(q, k, v)[0, 0]
    np.testing.assert_allclose([o[1], o[2]], [0.75, 0.25], atol=1e-13)
