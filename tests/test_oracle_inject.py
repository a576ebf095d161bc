"""Pins of the oracle's RoPE, KV injection and trim/append."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS


def _brute_rope(vec, pos, theta):
    hd = len(vec)
    half = hd // 2
    out = [0.0] * hd
    for d in range(half):
        ang = pos * theta ** (-2.0 * d / hd)
        c, s = math.cos(ang), math.sin(ang)
        # a 2-D rotation by +ang of the point (x_d, x_{d+half})
        out[d] = vec[d] * c - vec[d + half] * s
        out[d + half] = vec[d] * s + vec[d + half] * c
    return out


def test_rope_unit_vector_rotation():
    # hd = 4, theta = 100: frequencies 1 and 1/10; e_0 at position p -> (cos p, 0, sin p, 0)
    x = np.zeros((1, 1, 4)); x[0, 0, 0] = 1.0
    for p in [0, 1, 3, 17]:
        y = O.apply_rope(x, [p], 100.0)[0, 0]
        np.testing.assert_allclose(y, [math.cos(p), 0, math.sin(p), 0], atol=1e-14)
    x = np.zeros((1, 1, 4)); x[0, 0, 1] = 1.0
    y = O.apply_rope(x, [5], 100.0)[0, 0]
    np.testing.assert_allclose(y, [0, math.cos(0.5), 0, math.sin(0.5)], atol=1e-14)


def test_rope_matches_brute_force_and_invariants():
    rng = np.random.default_rng(3)
    hd, theta = 16, 1e6
    x = rng.standard_normal((6, 3, hd))
    pos = np.array([0, 1, 7, 100, 2048, 8191])
    y = O.apply_rope(x, pos, theta)
    for t in range(6):
        for h in range(3):
            np.testing.assert_allclose(y[t, h], _brute_rope(list(x[t, h]), pos[t], theta),
                                       atol=1e-12)
    # position 0 is the identity; per-pair norms are preserved
    np.testing.assert_array_equal(y[0], x[0])
    half = hd // 2
    n_in = x[..., :half] ** 2 + x[..., half:] ** 2
    n_out = y[..., :half] ** 2 + y[..., half:] ** 2
    np.testing.assert_allclose(n_in, n_out, rtol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(4)
    hd, theta = 32, 1e6
    q = rng.standard_normal((1, 1, hd)); k = rng.standard_normal((1, 1, hd))
    for m, n, delta in [(5, 2, 11), (100, 37, 1000), (0, 0, 4096)]:
        a = (O.apply_rope(q, [m], theta) * O.apply_rope(k, [n], theta)).sum()
        b = (O.apply_rope(q, [m + delta], theta) * O.apply_rope(k, [n + delta], theta)).sum()
        assert abs(a - b) < 1e-9
    # composition: rotating by a then by b is rotating by a+b
    x = rng.standard_normal((1, 2, hd))
    ab = O.apply_rope(O.apply_rope(x, [13], theta), [29], theta)
    np.testing.assert_allclose(ab, O.apply_rope(x, [42], theta), atol=1e-12)


def test_inject_matches_brute_force_loops():
    rng = np.random.default_rng(5)
    T, D, Hkv, hd, theta, pos0 = 3, 8, 2, 4, 1e6, 6
    ctx = rng.standard_normal((T, D))
    wk = rng.standard_normal((Hkv * hd, D)); wv = rng.standard_normal((Hkv * hd, D))
    K, V = O.inject_kv(ctx, wk, wv, pos0, Hkv, hd, theta)
    for t in range(T):
        krow = [sum(wk[n, d] * ctx[t, d] for d in range(D)) for n in range(Hkv * hd)]
        vrow = [sum(wv[n, d] * ctx[t, d] for d in range(D)) for n in range(Hkv * hd)]
        for h in range(Hkv):
            np.testing.assert_allclose(
                K[t, h], _brute_rope(krow[h * hd:(h + 1) * hd], pos0 + t, theta), atol=1e-12)
            np.testing.assert_allclose(V[t, h], vrow[h * hd:(h + 1) * hd], atol=1e-12)


def _tiny_layers(cfg, rng):
    return [{"wk": rng.standard_normal((cfg.kv_dim, cfg.hidden)) * 0.02,
             "wv": rng.standard_normal((cfg.kv_dim, cfg.hidden)) * 0.02}
            for _ in range(cfg.n_layers)]


def test_incremental_append_equals_one_shot():
    cfg = CONFIGS[0].shrink(n_layers=2)
    rng = np.random.default_rng(6)
    layers = _tiny_layers(cfg, rng)
    ctx = rng.standard_normal((23, cfg.hidden))
    one = O.DraftCache(cfg.n_layers)
    O.cache_inject(one, ctx, layers, cfg, 0)
    inc = O.DraftCache(cfg.n_layers)
    O.cache_inject(inc, ctx[:10], layers, cfg, 0)
    O.cache_inject(inc, ctx[10:17], layers, cfg, 10)
    O.cache_inject(inc, ctx[17:], layers, cfg, 17)
    assert inc.len == one.len == 23
    for i in range(cfg.n_layers):
        np.testing.assert_array_equal(inc.k[i], one.k[i])
        np.testing.assert_array_equal(inc.v[i], one.v[i])


def test_trim_then_append_rounds():
    # round r: the cache is cut back to the accepted prefix, then the accepted
    # rows' features are appended (txtmix article section 9)
    cfg = CONFIGS[0]
    rng = np.random.default_rng(7)
    layers = _tiny_layers(cfg, rng)
    rows = rng.standard_normal((40, cfg.hidden))
    c = O.DraftCache(cfg.n_layers)
    O.cache_inject(c, rows[:10], layers, cfg, 0)
    S = 10
    for tau in [3, 1, 4, 4]:
        # garbage rows beyond S must not survive the trim
        O.cache_inject(c, rng.standard_normal((4, cfg.hidden)), layers, cfg, S)
        c.trim(S)
        O.cache_inject(c, rows[S:S + tau], layers, cfg, S)
        S += tau
    assert c.len == 10 + 3 + 1 + 4 + 4
    ref = O.DraftCache(cfg.n_layers)
    O.cache_inject(ref, rows[:S], layers, cfg, 0)
    np.testing.assert_allclose(c.k[0], ref.k[0], atol=1e-14)
    np.testing.assert_allclose(c.v[0], ref.v[0], atol=1e-14)
    with pytest.raises(ValueError):
        c.trim(S + 1)


def test_round_bf16_matches_library_conversion():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(50000) * 10.0 ** rng.uniform(-30, 30, 50000)
    # exact ties: the 16 dropped bits are 0x8000, upper halves odd and even
    hi = rng.integers(0x0080, 0x7F00, 20000, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32).astype(np.float64)
    ties = np.concatenate([ties, -ties, [0.0, -0.0, 1.0]])
    for v in (x, ties):
        ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(O.round_bf16(v), ref)


def test_bf16_cache_stores_rounded_rows():
    cfg = CONFIGS[0].shrink(n_layers=2)
    rng = np.random.default_rng(13)
    layers = _tiny_layers(cfg, rng)
    ctx = rng.standard_normal((9, cfg.hidden))
    exact = O.DraftCache(cfg.n_layers)
    O.cache_inject(exact, ctx, layers, cfg, 0)
    low = O.DraftCache(cfg.n_layers, bf16_kv=True)
    O.cache_inject(low, ctx[:4], layers, cfg, 0)
    O.cache_inject(low, ctx[4:], layers, cfg, 4)
    for i in range(cfg.n_layers):
        kk = torch.from_numpy(exact.k[i].astype(np.float32)).to(torch.bfloat16).double().numpy()
        vv = torch.from_numpy(exact.v[i].astype(np.float32)).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(low.k[i], kk)
        np.testing.assert_array_equal(low.v[i], vv)
        assert not np.array_equal(low.k[i], exact.k[i])
