"""GPU parity of verification (greedy and p/q) and of sampling-mode drafting
against the oracle.

tau and bonus must be bit-exact; for p/q, rows whose accept test has
|p/q - u| < 1e-4 or whose final draw lies within 1e-12 (relative) of a CDF
boundary are excluded, as those decisions may flip under rounding order."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import DEV, make, say
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _greedy_case(dc, n_seqs, bl, rng, agreements):
    ids = rng.integers(0, dc.vocab - 1, size=(n_seqs, bl)).astype(np.int32)
    lg = torch.randn(n_seqs, bl, dc.vocab, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
    for s in range(n_seqs):
        synth.plant_agreement(lg[s], ids[s], agreements[s])
    return ids, lg


@pytest.mark.parametrize("ci,n_seqs,bl", [(0, 1, 4), (0, 3, 2), (1, 1, 16), (1, 4, 16), (1, 2, 9),
                                          (0, 2, 1), (4, 1, 8)])
def test_greedy_matches_oracle(ci, n_seqs, bl):
    dc = CONFIGS[ci]
    say(f"greedy verify: config {dc.name} n_seqs={n_seqs} block_len={bl}")
    d, _ = make(dc, max_seqs=n_seqs)
    rng = np.random.default_rng(100 + ci * 10 + bl)
    for trial in range(6):
        agree = [int(rng.integers(0, bl)) for _ in range(n_seqs)]
        if trial == 0:
            agree = [0] * n_seqs
        if trial == 1:
            agree = [bl - 1] * n_seqs
        ids, lg = _greedy_case(dc, n_seqs, bl, rng, agree)
        tau, bonus = d.verify(torch.from_numpy(ids).to(DEV), lg.to(DEV))
        tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
        for s in range(n_seqs):
            t, b = O.verify_greedy(ids[s], lg[s].numpy())
            assert (tau[s], bonus[s]) == (t, b), (trial, s)
            assert t == agree[s] + 1


def test_greedy_ties_take_lowest_index():
    dc = CONFIGS[0]
    d, _ = make(dc, max_seqs=1)
    lg = torch.zeros(1, 4, dc.vocab)
    lg[0, :, 7] = 1.0
    lg[0, :, 3] = 1.0
    lg[0, :, 900] = 1.0
    ids = torch.tensor([[5, 3, 3, 7]], dtype=torch.int32)
    tau, bonus = d.verify(ids.to(DEV), lg.to(DEV))
    assert O.verify_greedy(ids[0].numpy(), lg[0].numpy()) == (3, 3)
    assert (int(tau[0]), int(bonus[0])) == (3, 3)


def _pq_case(dc, bl, seed, rng):
    V = dc.vocab
    g = torch.Generator().manual_seed(seed)
    T = torch.randn(bl, V, generator=g)
    Q = torch.randn(bl - 1, V, generator=g)
    return T, Q


@pytest.mark.parametrize("ci,bl,temp", [(4, 8, 1.0), (0, 4, 1.0), (0, 4, 0.7), (4, 3, 1.5), (0, 1, 1.0)])
def test_pq_matches_oracle(ci, bl, temp):
    dc = CONFIGS[ci]
    say(f"p/q verify: config {dc.name} block_len={bl} temperature={temp}")
    d, _ = make(dc, max_seqs=2)
    rng = np.random.default_rng(7)
    checked = 0
    for trial in range(8):
        T, Q = [], []
        ids = []
        for s in range(2):
            t, q = _pq_case(dc, bl, 1000 * trial + s, rng)
            # drafted tokens x_j ~ q_j (the rule assumes drafts come from q)
            x, _ = O.sample_draft_tokens(q.numpy(), temp, seed=trial, seq=s) if bl > 1 else (np.zeros(0, np.int64), None)
            ids.append(np.concatenate([[int(rng.integers(0, dc.vocab))], x]).astype(np.int32))
            T.append(t); Q.append(q)
        ids = np.stack(ids)
        Tt = torch.stack(T).to(DEV)
        Qt = torch.stack(Q).to(DEV) if bl > 1 else None
        seed, off = 11 + trial, 3 * trial
        tau, bonus = d.verify(torch.from_numpy(ids).to(DEV), Tt, Qt, temperature=temp, seed=seed,
                              philox_offset=off)
        tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
        for s in range(2):
            t, b, diag = O.verify_pq(ids[s], T[s].numpy(), Q[s].numpy() if bl > 1 else np.zeros((0, dc.vocab)),
                                     temp, seed, off, s)
            if min(diag["ratio_margin"] or [1.0]) < 1e-4 or diag["cdf_margin"] < 1e-12:
                continue
            assert (tau[s], bonus[s]) == (t, b), (trial, s, diag)
            checked += 1
    assert checked >= 12


def _sampled_rows_match(got, logits, temp, seed, off, n_seqs, bl):
    """Compare sampled block columns 1.. with the oracle's draws; rows whose draw
    lies within 1e-12 of a CDF boundary are skipped. Returns rows compared."""
    checked = 0
    for s in range(n_seqs):
        x, margin = O.sample_draft_tokens(logits[s], temp, seed, off, s)
        for j in range(bl - 1):
            if margin[j] < 1e-12:
                continue
            assert int(got[s, 1 + j]) == int(x[j]), (s, j, margin[j])
            checked += 1
    return checked


@pytest.mark.parametrize("ci,n_seqs,bl,temp", [(0, 2, 4, 1.0), (0, 1, 4, 0.5), (4, 2, 8, 1.0),
                                               (1, 1, 16, 1.0), (1, 3, 5, 2.0)])
def test_sample_draft_matches_oracle(ci, n_seqs, bl, temp):
    dc = CONFIGS[ci]
    say(f"sample_draft: config {dc.name} n_seqs={n_seqs} block_len={bl} temperature={temp}")
    d, _ = make(dc, max_seqs=n_seqs)
    checked = 0
    for trial in range(3):
        g = torch.Generator().manual_seed(500 + 17 * trial + ci)
        lg = torch.randn(n_seqs, bl - 1, dc.vocab, generator=g) * (1.0 + trial)
        anchors = torch.arange(n_seqs, dtype=torch.int32) * 7 + 1
        blk = torch.full((n_seqs, bl), -1, dtype=torch.int32)
        blk[:, 0] = anchors
        blk = blk.to(DEV)
        seed, off = 3 + trial, 5 * trial
        d.sample_draft(blk, lg.to(DEV), temp, seed=seed, philox_offset=off)
        got = blk.cpu().numpy()
        assert (got[:, 0] == anchors.numpy()).all()
        assert ((got[:, 1:] >= 0) & (got[:, 1:] < dc.vocab)).all()
        checked += _sampled_rows_match(got, lg.numpy(), temp, seed, off, n_seqs, bl)
    assert checked >= 3 * n_seqs * (bl - 1) - 2


def test_sampling_round_from_draft_logits():
    """A whole sampling-mode round at the tiny shape: draft forward with logits,
    tokens sampled from them, p/q verification against target logits; the
    oracle takes the same logits and uniforms at every step."""
    from gpu_helpers import fill_context
    dc = CONFIGS[0]
    d, w = make(dc, max_seqs=2)
    g = torch.Generator().manual_seed(77)
    kvs = []
    for s in range(2):
        kv = d.new_kv(64)
        fill_context(kv, [(torch.randn(10 + s, dc.n_kv_heads, dc.head_dim, generator=g).to(torch.bfloat16).to(DEV),
                           torch.randn(10 + s, dc.n_kv_heads, dc.head_dim, generator=g).to(torch.bfloat16).to(DEV))
                          for _ in range(dc.n_layers)])
        kvs.append(kv)
    anchors = torch.tensor([5, 9], dtype=torch.int32, device=DEV)
    temp, seed = 1.0, 21
    checked = 0
    for rnd in range(4):
        blk, _, dl = d.draft_block(kvs, anchors, logits=True)
        d.sample_draft(blk, dl, temp, seed=seed, philox_offset=4 * rnd)
        tl = torch.randn(2, dc.block_size, dc.vocab, generator=g)
        tau, bonus = d.verify(blk, tl.to(DEV), dl, temperature=temp, seed=seed, philox_offset=4 * rnd)
        got, dln = blk.cpu().numpy(), dl.cpu().numpy()
        n = _sampled_rows_match(got, dln, temp, seed, 4 * rnd, 2, dc.block_size)
        for s in range(2):
            t, b, diag = O.verify_pq(got[s], tl[s].numpy(), dln[s], temp, seed, 4 * rnd, s)
            if min(diag["ratio_margin"] or [1.0]) < 1e-4 or diag["cdf_margin"] < 1e-12:
                continue
            assert (int(tau[s]), int(bonus[s])) == (t, b), (rnd, s, diag)
            checked += 1
        checked += n
    assert checked >= 20


def test_greedy_32_sequences_in_one_call():
    # the 32-sequence workload: every sequence's block verified in one call,
    # planted agreement lengths k ~ Geometric(0.25) capped at the block
    dc = CONFIGS[3]
    n, bl = 32, dc.block_size
    say(f"greedy verify: config {dc.name} n_seqs={n} in one call")
    d, _ = make(dc, max_seqs=n)
    rng = np.random.default_rng(31)
    taus = synth.planted_taus(dc, n, salt=3)
    ids, lg = _greedy_case(dc, n, bl, rng, [int(t) - 1 for t in taus])
    tau, bonus = d.verify(torch.from_numpy(ids).to(DEV), lg.to(DEV))
    tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
    for s in range(n):
        t, b = O.verify_greedy(ids[s], lg[s].numpy())
        assert (tau[s], bonus[s]) == (t, b), s
        assert t == taus[s]


def test_pq_d2048_block8_philox_seed0():
    # the D=2048 workload's verification: temperature 1, target and draft
    # logits N(0, 1) per row, draft tokens drawn from q, uniforms from Philox
    # with seed 0; decisions with |p/q - u| < 1e-4 (or a draw within 1e-12 of
    # a CDF boundary) are excluded and counted
    dc = CONFIGS[4]
    bl, temp, seed = dc.block_size, dc.temperature, 0
    n = 4
    say(f"p/q verify: config {dc.name} block_len={bl} seed={seed}")
    d, _ = make(dc, max_seqs=n)
    checked = excluded = 0
    for trial in range(6):
        g = torch.Generator().manual_seed(900 + trial)
        T = torch.randn(n, bl, dc.vocab, generator=g)
        Q = torch.randn(n, bl - 1, dc.vocab, generator=g)
        off = bl * trial
        ids = []
        for s in range(n):
            x, _ = O.sample_draft_tokens(Q[s].numpy(), temp, seed, off, s)
            ids.append(np.concatenate([[7 + s], x]).astype(np.int32))
        ids = np.stack(ids)
        tau, bonus = d.verify(torch.from_numpy(ids).to(DEV), T.to(DEV), Q.to(DEV), temperature=temp,
                              seed=seed, philox_offset=off)
        tau, bonus = tau.cpu().numpy(), bonus.cpu().numpy()
        for s in range(n):
            t, b, diag = O.verify_pq(ids[s], T[s].numpy(), Q[s].numpy(), temp, seed, off, s)
            assert 1 <= tau[s] <= bl
            if min(diag["ratio_margin"] or [1.0]) < 1e-4 or diag["cdf_margin"] < 1e-12:
                excluded += 1
                continue
            assert (tau[s], bonus[s]) == (t, b), (trial, s, diag)
            checked += 1
    say(f"  {checked} rounds compared, {excluded} excluded by the bands")
    assert checked >= 20
