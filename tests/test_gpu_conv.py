"""GPU parity of the DFlash 2 grouped dynamic two-tap conv against the oracle
([Code] sections 13-14), on the same seeded bf16 tables and fp32 rows.

Tolerance: the GPU forms each correction as an fp32 sum of bf16 weights
times the row split into bf16 high and low halves (relative representation
error 2^-17 per element), so a correction c = sum_i w_i x_i is off by about
2^-17 * sqrt(sum_i (w_i x_i)^2) plus fp32 rounding of the sum: ~1e-5 for
the N(0, 1/D) projection. An output element k0 x_t + k1 x_{t-1} then
differs by at most ~1e-5 (|x_t| + |x_{t-1}|); the test allows
2e-4 (|x_t| + |x_{t-1}|) + 1e-5 elementwise."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import DEV, make, np32, say
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _check(got, ref, a, a_prev, bl):
    rows = a.shape[0]
    before = np.empty_like(a)
    for m in range(rows):
        s, t = divmod(m, bl)
        before[m] = a_prev[s] if t == 0 else a[m - 1]
    tol = 2e-4 * (np.abs(a) + np.abs(before)) + 1e-5
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max excess {np.max(err - tol):.3e}"


def _run(dc, n_seqs, bl, gs=16, max_seqs=None):
    say(f"conv: config {dc.name} seqs={n_seqs} block_len={bl} group={gs}")
    d, _ = make(dc, max_seqs=max_seqs or n_seqs)
    cv = synth.make_conv(dc, n_seqs, bl, gs, device=DEV)
    y, corr = d.conv_prepare(cv["x"], cv["prev"], cv["base"], cv["proj"], bl, gs)
    y2 = d.conv_finish(cv["z"], cv["zprev"], cv["base"], corr, bl, gs)
    torch.cuda.synchronize()
    n = {k: np32(v).astype(np.float64) for k, v in cv.items()}
    ry, rc = O.dynamic_conv_prepare(n["x"], n["prev"], bl, n["base"], n["proj"], gs)
    _check(np32(y), ry, n["x"], n["prev"], bl)
    G = dc.hidden // gs
    np.testing.assert_allclose(np32(corr), rc, rtol=0, atol=2e-5 * np.sqrt(dc.hidden / 64))
    # the finish call on the GPU's own corrections (the oracle reads the same fp32 values)
    ry2 = O.dynamic_conv_finish(n["z"], n["zprev"], bl, n["base"], np32(corr), gs)
    _check(np32(y2), ry2, n["z"], n["zprev"], bl)
    assert corr.shape == (n_seqs * bl, 2 * G)


def test_tiny_config():
    # hidden 64: groups of 4 channels (hidden must hold 16 whole groups)
    _run(CONFIGS[0], 1, 4, gs=4)


def test_tiny_block_one_and_single_channel_groups():
    _run(CONFIGS[0], 2, 1, gs=4)
    _run(CONFIGS[0], 1, 3, gs=1)


def test_qwen_shape_one_block():
    # hidden 4096, 256 groups: the LDS-staged streaming GEMM (16 rows)
    _run(CONFIGS[1], 1, 16)


def test_qwen_shape_ragged_rows_and_many_sequences():
    # 2 x 7 rows (the streaming GEMM's ragged tile), 3 x 7 rows and 32 x 16
    # rows (the register-streaming kernel, one 32-row block / 64-row blocks)
    _run(CONFIGS[1], 2, 7, max_seqs=32)
    _run(CONFIGS[1], 3, 7, max_seqs=32)
    _run(CONFIGS[3], 32, 16)


def test_qwen_shape_single_row_blocks():
    # one row per block: every row reads its sequence's prev row
    _run(CONFIGS[1], 1, 1, max_seqs=16)
    _run(CONFIGS[1], 16, 1)


def test_d2048_group_32():
    _run(CONFIGS[4], 2, 8, gs=32)


# ---------------------------------------------------------------------------
# the convs inside every draft layer (dflash_set_conv)
# ---------------------------------------------------------------------------

def _conv_np(conv):
    return {"group_size": conv["group_size"],
            "layers": [{k: np32(v).astype(np.float64) for k, v in l.items()} for l in conv["layers"]]}


def _draft_with_convs(dc, lens, gs, bl=None, gains="random"):
    from gpu_helpers import (TIGHT_TOL, assert_hidden, assert_tokens, fill_context, hidden_errs,
                             oracle_cache, poisoned_kv, synthetic_context, weights_np)
    bl = dc.block_size if bl is None else bl
    lens = [lens] if isinstance(lens, int) else list(lens)
    n = len(lens)
    say(f"draft with convs: config {dc.name} contexts {lens} group_size={gs} block_len={bl}")
    d, w = make(dc, max_seqs=n, gains=gains)
    conv = synth.make_conv_layers(dc, gs, device=DEV)
    d.set_conv(conv)
    kvs, ctxs = [], []
    for s_, S in enumerate(lens):
        kv = poisoned_kv(d, S + 8)
        ctx = synthetic_context(dc, S, seq=s_)
        if S:
            fill_context(kv, ctx)
        kvs.append(kv)
        ctxs.append(ctx)
    anchors = synth.make_anchor(dc, n=n)
    block, hid, _ = d.draft_block(kvs, torch.from_numpy(anchors).to(DEV), bl, hidden=True)
    torch.cuda.synchronize()
    wn = weights_np(w)
    cn = _conv_np(conv)
    orc = O.draft_block(dc, wn, [oracle_cache(dc, c) for c in ctxs], [int(a) for a in anchors], bl,
                        conv=cn)
    g = np32(hid).reshape(dc.n_layers, n * bl, -1)
    say("  plain: " + " ".join(f"{e:.2e}" for e in hidden_errs(g, orc["hidden"])))
    assert_hidden(g, orc["hidden"], what="conv draft")
    assert_hidden(g, orc["hidden"], what="conv draft", tol=TIGHT_TOL)
    if bl > 1:
        assert_tokens(block.cpu().numpy(), orc, what="conv draft")
    # removing the convs gives the plain draft back
    d.set_conv(None)
    block2, hid2, _ = d.draft_block(kvs, torch.from_numpy(anchors).to(DEV), bl, hidden=True)
    torch.cuda.synchronize()
    orc2 = O.draft_block(dc, wn, [oracle_cache(dc, c) for c in ctxs], [int(a) for a in anchors], bl)
    assert_hidden(np32(hid2).reshape(dc.n_layers, n * bl, -1), orc2["hidden"], what="plain draft",
                  tol=TIGHT_TOL)
    d.close()


def test_draft_with_convs_tiny():
    # hidden 64: four channels per correction group
    _draft_with_convs(CONFIGS[0].shrink(n_layers=2, index=94), 10, 4)


def test_draft_with_convs_tiny_empty_context_short_block():
    _draft_with_convs(CONFIGS[0].shrink(n_layers=2, index=94), 0, 4, bl=3)


def test_draft_with_convs_mid_shape_one_sequence():
    # 16 rows: the convs fused into the GEMMs' finishers
    dc = CONFIGS[1].shrink(hidden=512, n_layers=2, n_heads=8, n_kv_heads=2, ffn=1024, vocab=4096,
                           index=93)
    _draft_with_convs(dc, 300, 16)


def test_draft_with_convs_mid_shape_two_sequences():
    # 32 rows: the convs as separate kernels
    dc = CONFIGS[1].shrink(hidden=512, n_layers=2, n_heads=8, n_kv_heads=2, ffn=1024, vocab=4096,
                           index=93)
    _draft_with_convs(dc, [300, 45], 16)


def test_draft_with_convs_mid_shape_tall_batch():
    # 6 sequences x 16 = 96 rows: the projections, the plain products before
    # the finish calls and the layer products on the tiled (tall) GEMM
    dc = CONFIGS[1].shrink(hidden=512, n_layers=2, n_heads=8, n_kv_heads=2, ffn=1024, vocab=4096,
                           index=93)
    _draft_with_convs(dc, [300, 45, 0, 129, 7, 64], 16)


def test_draft_with_convs_mid_shape_short_block_fused():
    # 5 rows in one tile; group size 32
    dc = CONFIGS[1].shrink(hidden=512, n_layers=2, n_heads=8, n_kv_heads=2, ffn=1024, vocab=4096,
                           index=93)
    _draft_with_convs(dc, 77, 32, bl=5)


def test_draft_with_convs_qwen_shape_full_size():
    dc = CONFIGS[1]
    _draft_with_convs(dc, dc.ctx_len, 16, gains="ones")
