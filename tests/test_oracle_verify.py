"""Pins of the oracle's greedy verification."""
import numpy as np
import torch

import oracle as O
import synth
from synth import CONFIGS


def _brute(block, logits):
    post = [max(range(len(r)), key=lambda v: (r[v], -v)) for r in logits]
    a = 0
    while a < len(block) - 1 and block[a + 1] == post[a]:
        a += 1
    return a + 1, post[a]


def _logits_with_posterior(post, V, rng):
    x = rng.standard_normal((len(post), V))
    for j, p in enumerate(post):
        x[j, p] = x[j].max() + 0.5
    return x


def test_walkthrough_ninth_candidate_breaks():
    # txtmix article section 9: block of 16, the 9th candidate is wrong:
    # 8 drafts accepted, the bonus makes the round advance 9 tokens
    rng = np.random.default_rng(20)
    V = 50
    post = rng.integers(0, V, size=16)
    block = np.empty(16, dtype=np.int64)
    block[0] = 3
    block[1:] = post[:-1]
    block[9] = (post[8] + 1) % V
    tau, bonus = O.verify_greedy(block, _logits_with_posterior(post, V, rng))
    assert tau == 9 and bonus == post[8]


def test_all_reject_and_all_accept():
    rng = np.random.default_rng(21)
    V = 40
    post = rng.integers(0, V, size=8)
    lg = _logits_with_posterior(post, V, rng)
    block = np.concatenate([[1], post[:-1]])
    assert O.verify_greedy(block, lg) == (8, post[7])
    block[1] = (post[0] + 1) % V
    assert O.verify_greedy(block, lg) == (1, post[0])
    # a later match after a mismatch does not count (prefix rule)
    block2 = np.concatenate([[1], post[:-1]]); block2[3] = (post[2] + 1) % V
    assert O.verify_greedy(block2, lg) == (3, post[2])


def test_matches_brute_force_and_range():
    rng = np.random.default_rng(22)
    for trial in range(3000):
        B = int(rng.integers(1, 17))
        V = int(rng.integers(2, 6))
        lg = rng.integers(0, 3, size=(B, V)).astype(np.float32)  # many ties
        block = rng.integers(0, V, size=B)
        tau, bonus = O.verify_greedy(block, lg)
        assert 1 <= tau <= B
        assert (tau, bonus) == _brute(list(block), lg.tolist())


def test_planted_agreement_reproduced():
    cfg = CONFIGS[1].shrink(vocab=1000, index=92)
    taus = synth.planted_taus(cfg, 200)
    rng = np.random.default_rng(23)
    for i, tau in enumerate(taus):
        lg = synth.make_target_logits(cfg, cfg.block_size, round_index=i)
        block = rng.integers(0, cfg.vocab - 1, size=cfg.block_size)
        synth.plant_agreement(lg, block, int(tau) - 1)
        assert O.verify_greedy(block, lg.numpy())[0] == tau


def test_expected_tau_capped_geometric():
    # E[tau] = sum_{t=0}^{15} 0.75^t = 3.95991 for tau = min(G, 16), G ~ Geom(0.25)
    cfg = CONFIGS[1]
    exact = sum(0.75 ** t for t in range(16))
    assert abs(exact - 3.959909) < 1e-6
    taus = synth.planted_taus(cfg, 100000)
    sd = taus.std() / np.sqrt(len(taus))
    assert abs(taus.mean() - exact) < 5 * sd


def test_acceptance_identity_with_independent_hits():
    # E[a] = sum_k P(x_1..k all hit) = sum_k prod_{i<=k} h_i when position i hits
    # independently with probability h_i ([Note] section 1, acceptance length);
    # a per-position (non-prefix) count would give sum_k h_k instead.
    rng = np.random.default_rng(24)
    h = np.array([0.9, 0.8, 0.7, 0.9, 0.5, 0.6, 0.8])
    B, V, n = len(h) + 1, 7, 20000
    tot = 0
    counts = np.zeros(B, dtype=np.int64)   # counts[k] = #{rounds with a >= k}
    post = np.arange(B) % V
    lg = _logits_with_posterior(post, V, rng)
    for _ in range(n):
        hit = rng.random(len(h)) < h
        block = np.empty(B, dtype=np.int64); block[0] = 0
        block[1:] = np.where(hit, post[:-1], (post[:-1] + 1) % V)
        a = O.verify_greedy(block, lg)[0] - 1
        tot += a
        counts[1:a + 1] += 1
    assert tot == counts.sum()              # sum_i a_i = sum_k #{a_i >= k}, exactly
    expect = np.cumprod(h).sum()
    assert abs(tot / n - expect) < 0.05
    assert abs(tot / n - h.sum()) > 0.5
