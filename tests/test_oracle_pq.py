"""Pins of the oracle's p/q rejection-sampling verification and its RNG."""
import math

import numpy as np
import pytest

import oracle as O


def test_philox_known_answers_against_numpy():
    # numpy.random.Philox is Philox4x64-10; it bumps the counter before each
    # block, so the block at counter c comes from a generator set to c - 1.
    cases = [((1, 0, 0, 0), (0, 0)), ((6, 0, 0, 0), (7, 3)),
             ((2 ** 64 - 1, 5, 0, 9), (123456789, 987654321)),
             ((17, 3, 1, 0), (0, 0)), ((0, 0, 0, 1), (2 ** 63, 1))]
    for ctr, key in cases:
        c = list(ctr)
        # c - 1 in 256-bit arithmetic
        i = 0
        while c[i] == 0:
            c[i] = 2 ** 64 - 1; i += 1
        c[i] -= 1
        bg = np.random.Philox(counter=np.array(c, dtype=np.uint64),
                              key=np.array(key, dtype=np.uint64))
        ref = [int(x) for x in bg.random_raw(4)]
        assert list(O.philox4x64_10(ctr, key)) == ref


def test_uniform_mapping():
    # the 53-bit mapping of word 0 equals numpy's double from the same word
    bg = np.random.Philox(counter=[4, 2, 1, 0], key=[9, 0])
    w = int(bg.random_raw(1)[0])
    assert O.philox_uniform(9, 5, 2, 1) == (w >> 11) * 2.0 ** -53
    us = [O.philox_uniform(0, j, s, p) for j in range(50) for s in range(4) for p in range(3)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert abs(np.mean(us) - 0.5) < 0.05


def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(30)
    for _ in range(500):
        w = rng.random(int(rng.integers(1, 9))) * (rng.random() < 0.9)
        w[rng.integers(0, len(w))] += 0.1
        u = rng.random()
        tot = 0.0
        for x in w:
            tot += x
        acc, tok = 0.0, len(w) - 1
        for v, x in enumerate(w):
            acc += x
            if acc > u * tot:
                tok = v
                break
        assert O.sample_inverse_cdf(w, u)[0] == tok
    # zero-weight entries are never drawn
    for u in np.linspace(0, 0.999, 101):
        assert O.sample_inverse_cdf([0.0, 0.3, 0.0, 0.7, 0.0], u)[0] in (1, 3)


def _grid(n):
    return (np.arange(n) + 0.5) / n


def test_lossless_by_quadrature_tiny_vocab():
    # P(first emitted token = v) = p_0(v) whatever q is: the drafted token x is
    # drawn from q_0, the accept test integrates over u, the replacement over u'.
    rng = np.random.default_rng(31)
    V, N = 4, 160
    T = rng.standard_normal((2, V)) * 1.5
    Q = rng.standard_normal((1, V)) * 1.5
    p0, q0 = O.softmax(T[0]), O.softmax(Q[0])
    prob = np.zeros(V)
    acc_prob = 0.0
    for x in range(V):
        for u in _grid(N):
            for u2 in _grid(N):
                tau, tok, _ = O.verify_pq_with_uniforms([0, x], T, Q, 1.0, [u], [u2, u2])
                first = x if tau == 2 else tok
                prob[first] += q0[x] / (N * N)
                acc_prob += q0[x] * (tau == 2) / (N * N)
    np.testing.assert_allclose(prob, p0, atol=4.0 / N)
    # row acceptance probability = sum_v min(p, q)
    assert abs(acc_prob - np.minimum(p0, q0).sum()) < 2.0 / N
    # a verifier that resampled from p (not the residual) would be visibly off
    biased = np.zeros(V)
    for x in range(V):
        a = min(1.0, p0[x] / q0[x])
        biased += q0[x] * (a * (np.arange(V) == x) + (1 - a) * p0)
    assert np.abs(biased - p0).max() > 10.0 / N


def test_temperature_scales_logits():
    rng = np.random.default_rng(32)
    T = rng.standard_normal((3, 6)); Q = rng.standard_normal((2, 6))
    ua, ur = [0.3, 0.6], [0.2, 0.7, 0.9]
    a = O.verify_pq_with_uniforms([0, 2, 4], T, Q, 0.5, ua, ur)
    b = O.verify_pq_with_uniforms([0, 2, 4], 2 * T, 2 * Q, 1.0, ua, ur)
    assert a[:2] == b[:2]


def test_identical_distributions_always_accept():
    rng = np.random.default_rng(33)
    for _ in range(50):
        L = rng.standard_normal((5, 30))
        ids = rng.integers(0, 30, size=5)
        tau, _, _ = O.verify_pq(ids, L, L[:4], 1.0, int(rng.integers(0, 1000)))
        assert tau == 5


def test_rejection_draws_from_residual_support():
    # the target puts its mass on token 0; the draft proposes token 1 where
    # p << q, so it is rejected and the replacement must be token 0
    T = np.array([[10.0, -10, -10, -10], [0, 0, 0, 0]])
    Q = np.array([[-10.0, 10, -10, -10]])
    for seed in range(20):
        tau, tok, _ = O.verify_pq([2, 1], T, Q, 1.0, seed)
        assert tau == 1 and tok == 0


def test_acceptance_rate_iid_logits_large_vocab():
    # iid N(0,1) target and draft logits at large V: sum_v min(p, q) tends to
    # E[min(e^x, e^y)] / E[e^x] = 2 Phi(-1/sqrt 2)
    rng = np.random.default_rng(34)
    V = 151936
    beta = []
    for _ in range(6):
        p = O.softmax(rng.standard_normal(V)); q = O.softmax(rng.standard_normal(V))
        beta.append(np.minimum(p, q).sum())
    expect = 2 * 0.5 * math.erfc(1 / math.sqrt(2) / math.sqrt(2))
    assert abs(expect - 0.4795) < 1e-3
    assert abs(np.mean(beta) - expect) < 0.01


def test_bonus_after_full_acceptance_comes_from_last_target_row():
    # when every draft is kept, the extra token is drawn from the target's
    # distribution at the last block row (txtmix article section 8)
    rng = np.random.default_rng(35)
    L = rng.standard_normal((4, 12))
    T = L.copy(); T[3] = -30.0; T[3, 5] = 30.0
    for seed in range(20):
        tau, tok, _ = O.verify_pq([1, 2, 3, 4], T, L[:3], 1.0, seed)
        assert tau == 4 and tok == 5
