"""Pins of the oracle's DFlash 2 candidate selector: the top-k order, the
cases where the walk reduces to plain argmax drafting, a planted chain that
only the right predecessor/successor tables recover, the zero-temperature
limit of the sampled walk, and the sampled walk's frequencies."""
import numpy as np

import oracle as O


def test_top_k_order_fixture_and_numpy_stable_sort():
    z = np.array([0.5, 3.0, -1.0, 3.0, 2.0, 3.0, 0.0])
    idx, val = O.top_k_candidates(z, 4)
    assert idx.tolist() == [1, 3, 5, 4]
    assert val.tolist() == [3.0, 3.0, 3.0, 2.0]
    rng = np.random.default_rng(5)
    for _ in range(20):
        z = rng.integers(-3, 4, size=40).astype(float)  # many ties
        idx, _ = O.top_k_candidates(z, 7)
        assert idx.tolist() == np.argsort(-z, kind="stable")[:7].tolist()


def _inputs(rng, P=5, V=60, D=12, r=8):
    return (rng.standard_normal((P, V)), rng.standard_normal((P, D)),
            rng.standard_normal((r, D)), rng.standard_normal((V, r)), rng.standard_normal((V, r)))


def test_zero_gate_and_k1_reduce_to_argmax_drafting():
    rng = np.random.default_rng(1)
    Z, H, W, A, B = _inputs(rng)
    want = np.argmax(Z, axis=-1)
    out = O.select_candidates(Z, H, 3, np.zeros_like(W), A, B, k=6)
    assert out["path"].tolist() == want.tolist()
    out = O.select_candidates(Z, H, 3, W, A, B, k=1)
    assert out["path"].tolist() == want.tolist()
    # the pair term is zero when either table is zero
    out = O.select_candidates(Z, H, 3, W, np.zeros_like(A), B, k=6)
    assert out["path"].tolist() == want.tolist()


def test_planted_chain_is_followed():
    # codes that reward exactly the planted pairs (anchor -> t0 -> t1 ...):
    # predecessor code of t_{j-1} and successor code of t_j share unit vector
    # e_j; swapped tables, a fixed predecessor or position-indexed codes would
    # not recover the chain
    rng = np.random.default_rng(2)
    P, V, r, k = 4, 80, 8, 6
    Z = rng.standard_normal((P, V))
    anchor = 79
    chain = []
    for t in range(P):
        cand, _ = O.top_k_candidates(Z[t], k)
        pick = next(int(c) for c in cand[2:] if int(c) not in chain and int(c) != anchor)
        chain.append(pick)
    A = np.zeros((V, r))
    B = np.zeros((V, r))
    prev = anchor
    for t, tok in enumerate(chain):
        A[prev, t] = 10.0
        B[tok, t] = 10.0
        prev = tok
    H = np.ones((P, r))
    out = O.select_candidates(Z, H, anchor, np.eye(r), A, B, k=k)
    assert out["path"].tolist() == chain
    assert out["path"].tolist() != np.argmax(Z, axis=-1).tolist()
    # the same codes with the tables exchanged do not reward the chain
    out = O.select_candidates(Z, H, anchor, np.eye(r), B, A, k=k)
    assert out["path"].tolist() == np.argmax(Z, axis=-1).tolist()


def test_sampled_walk_at_low_temperature_is_the_greedy_walk():
    rng = np.random.default_rng(3)
    Z, H, W, A, B = _inputs(rng)
    g = O.select_candidates(Z, H, 7, W, A, B, k=8)
    assert np.all(g["gap"] > 1e-3)
    s = O.select_candidates(Z, H, 7, W, A, B, k=8, temperature=1e-5,
                            uniforms=rng.random(Z.shape[0]))
    assert s["path"].tolist() == g["path"].tolist()


def test_sampled_step_frequencies_follow_q():
    rng = np.random.default_rng(4)
    Z, H, W, A, B = _inputs(rng, P=1)
    n = 4000
    counts = {}
    q = None
    for i in range(n):
        out = O.select_candidates(Z, H, 0, W, A, B, k=5, temperature=1.5,
                                  uniforms=[(i + 0.5) / n])
        counts[int(out["path"][0])] = counts.get(int(out["path"][0]), 0) + 1
        q = out["q"][0]
        cand = out["cand"][0]
    assert abs(q.sum() - 1.0) < 1e-12
    for c, p in zip(cand, q):
        assert abs(counts.get(int(c), 0) / n - p) <= 1.0 / n + 1e-12


def test_candidate_q_verify_with_the_whole_vocabulary_is_dense_verify():
    # candidates = every token, q = softmax(draft / T): the dense p/q rule
    rng = np.random.default_rng(6)
    V, gamma, T = 9, 4, 0.7
    tl = rng.standard_normal((gamma + 1, V))
    dl = rng.standard_normal((gamma, V))
    for trial in range(30):
        block = [3] + rng.integers(0, V, gamma).tolist()
        ua, ur = rng.random(gamma), rng.random(gamma + 1)
        cand = np.array([rng.permutation(V) for _ in range(gamma)])
        q = np.array([O.softmax(dl[j] / T)[cand[j]] for j in range(gamma)])
        a = O.verify_pq_candidates_with_uniforms(block, tl, cand, q, T, ua, ur)
        b = O.verify_pq_with_uniforms(block, tl, dl, T, ua, ur)
        assert a[:2] == b[:2]


def test_candidate_q_verify_is_lossless():
    # speculative sampling keeps the target distribution: with x ~ q on a
    # candidate set, the first emitted token (x if kept, else the
    # replacement) is distributed as p
    rng = np.random.default_rng(7)
    V, k, T = 7, 3, 1.0
    tl = rng.standard_normal((2, V))
    p = O.softmax(tl[0] / T)
    cand = np.array([[5, 1, 2]])
    q = np.array([[0.5, 0.3, 0.2]])
    n = 40000
    counts = np.zeros(V)
    for i in range(n):
        x = int(cand[0][np.searchsorted(np.cumsum(q[0]), rng.random(), side="right")])
        tau, bonus, _ = O.verify_pq_candidates_with_uniforms([0, x], tl, cand, q, T,
                                                             [rng.random()], [rng.random(), rng.random()])
        counts[x if tau == 2 else bonus] += 1
    assert np.abs(counts / n - p).max() < 0.01


def test_candidate_q_verify_accepts_tokens_outside_the_candidates_and_bounds_tau():
    rng = np.random.default_rng(8)
    V, gamma, T = 12, 5, 1.3
    for _ in range(40):
        tl = rng.standard_normal((gamma + 1, V))
        cand = np.array([rng.choice(V, 4, replace=False) for _ in range(gamma)])
        q = rng.dirichlet(np.ones(4), size=gamma)
        block = [1] + rng.integers(0, V, gamma).tolist()
        tau, bonus, _ = O.verify_pq_candidates_with_uniforms(block, tl, cand, q, T,
                                                             rng.random(gamma), rng.random(gamma + 1))
        assert 1 <= tau <= gamma + 1 and 0 <= bonus < V
        # a row whose token is no candidate is always kept, so it is never
        # the rejected row
        outside = [j for j in range(gamma) if block[j + 1] not in cand[j]]
        if tau <= gamma:
            assert (tau - 1) not in outside
