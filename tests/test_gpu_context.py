"""GPU parity of context fusion, KV injection and trim/append of the draft KV cache.

Fusion and injection compute in fp32 and round to bf16 once, so their outputs
are checked at rounding exactness: equal to round_bf16 of the fp64 oracle
except within a stated band around the bf16 rounding midpoints (the bands and
their derivation are in gpu_helpers), where either bf16 neighbour is accepted;
the number of banded values is printed."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import (DEV, fuse_band, inject_band, assert_bf16_rounding, assert_close_rms, make,
                         np32, poisoned_kv, say)
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _fuse_check(dc, T, rows=None, gains="random", ld_pad=0):
    say(f"fuse: config {dc.name} T={T} ld_pad={ld_pad}")
    d, w = make(dc, max_tokens=T, gains=gains)
    feats = synth.make_feats(dc, T, device=DEV)
    if ld_pad:
        feats = [torch.nn.functional.pad(f, (0, ld_pad))[:, :dc.hidden] for f in feats]
    out = d.fuse_context(feats)
    torch.cuda.synchronize()
    rows = np.arange(T) if rows is None else rows
    ref = O.fuse_context([np32(f)[rows] for f in feats], np32(w["w_c"]), np32(w["ctx_norm"]), dc.rms_eps)
    assert_close_rms(np32(out)[rows], ref, what="fused context")
    return assert_bf16_rounding(np32(out)[rows], ref, fuse_band(dc), "fused context")


def test_fuse_tiny():
    _fuse_check(CONFIGS[0], 10)


def test_fuse_ragged_tiles_and_row_stride():
    # 300 rows: three 128-row tiles, the last one ragged; padded row stride
    dc = CONFIGS[0].shrink(hidden=192, index=93)
    _fuse_check(dc, 300, ld_pad=24)


def test_fuse_d2048_sampled_rows():
    dc = CONFIGS[4]
    rng = np.random.default_rng(0)
    _fuse_check(dc, 2048, rows=np.sort(rng.choice(2048, 96, replace=False)), gains="ones")


@pytest.mark.slow
def test_fuse_qwen_shape_sampled_rows():
    dc = CONFIGS[1]
    rng = np.random.default_rng(1)
    _fuse_check(dc, 2048, rows=np.sort(rng.choice(2048, 64, replace=False)), gains="ones")


@pytest.mark.slow
def test_fuse_qwen_shape_8192_rows_sampled():
    # 256-row tiles: 32 x 32 of them
    dc = CONFIGS[2]
    rng = np.random.default_rng(3)
    rows = np.sort(np.concatenate([rng.choice(8192, 40, replace=False), [0, 8191]]))
    _fuse_check(dc, 8192, rows=np.unique(rows), gains="random")


def test_fuse_qwen_shape_ragged_rows():
    # 2148 rows: 17 row tiles of 128, the last one ragged
    dc = CONFIGS[1]
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.choice(2048, 24, replace=False), np.arange(2040, 2148, 9), [2147]]))
    _fuse_check(dc, 2148, rows=rows, gains="random")


def test_fuse_many_rows_narrow_hidden():
    # 16484 rows of a 640-wide hidden state (5 column tiles, ragged last row tile)
    dc = CONFIGS[1].shrink(hidden=640, index=95)
    T = 16384 + 100
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(T, 40, replace=False), [T - 1, T - 100]]))
    _fuse_check(dc, T, rows=rows, gains="random")


def _inject_check(dc, T, pos0_chunks, rows=None, gains="ones", seq=0):
    say(f"inject: config {dc.name} T={T} chunks={pos0_chunks} seq={seq}")
    d, w = make(dc, max_tokens=max(pos0_chunks) if pos0_chunks else T, gains=gains)
    # any bf16 [T, D] context feature (the sequence index picks another draw)
    ctx = synth.make_feats(dc, T, round_index=seq, device=DEV)[0]
    kv = poisoned_kv(d, T + 32)
    p = 0
    for n in pos0_chunks:
        d.inject_kv(kv, ctx[p:p + n], p)
        p += n
    assert kv.len == T
    torch.cuda.synchronize()
    rows = np.arange(T) if rows is None else np.asarray(rows)
    ctx_np = np32(ctx)
    gk_all, gv_all, ok_all, ov_all = [], [], [], []
    for i, lw in enumerate(w["layers"]):
        for t in rows:
            k, v = O.inject_kv(ctx_np[t:t + 1], np32(lw["wk"]), np32(lw["wv"]), int(t),
                               dc.n_kv_heads, dc.head_dim, dc.rope_theta)
            gk_all.append(np32(kv.k_view(i)[:, t, :]))
            gv_all.append(np32(kv.v_view(i)[:, :, t]))
            ok_all.append(k[0])
            ov_all.append(v[0])
    gk, gv, ok, ov = (np.stack(x) for x in (gk_all, gv_all, ok_all, ov_all))
    assert_close_rms(gk, ok, what="K")
    assert_close_rms(gv, ov, what="V")
    return (assert_bf16_rounding(gk, ok, inject_band(dc), f"K ({len(rows)} rows x {dc.n_layers} layers)") +
            assert_bf16_rounding(gv, ov, inject_band(dc), f"V ({len(rows)} rows x {dc.n_layers} layers)"))


def test_inject_tiny_incremental():
    _inject_check(CONFIGS[0], 10, [4, 3, 3])


def test_inject_ragged_tiles():
    dc = CONFIGS[1].shrink(hidden=256, n_layers=2, n_heads=4, n_kv_heads=2, ffn=512, vocab=512, index=94)
    _inject_check(dc, 300, [300])


def test_inject_qwen_shape_sampled_rows():
    dc = CONFIGS[1]
    rng = np.random.default_rng(2)
    _inject_check(dc, 2048, [2048], rows=np.sort(rng.choice(2048, 24, replace=False)))


def test_inject_qwen_shape_ragged_rows():
    # 2148 rows: a ragged last row tile
    dc = CONFIGS[1]
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([rng.choice(2048, 10, replace=False), [2047, 2048, 2100, 2147]]))
    _inject_check(dc, 2148, [2148], rows=rows)


def test_inject_d2048_full_shape():
    # D = 2048, 4 KV heads, 5 layers: N = 5 x 2 x 512 columns (16 tiles of 320)
    dc = CONFIGS[4]
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([rng.choice(2048, 20, replace=False), [0, 2047]]))
    _inject_check(dc, 2048, [2048], rows=rows)


@pytest.mark.slow
def test_inject_long_context_prefill_8192_sampled_rows():
    # the long-context workload's prefill: 8192 rows in one call (32 row
    # tiles of 256), sampled rows including the first and the last tile's
    dc = CONFIGS[2]
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.choice(8192, 16, replace=False), [0, 7936, 8191]]))
    _inject_check(dc, 8192, [8192], rows=rows)


def test_inject_ragged_batch_two_of_32_sequences():
    # the 32-sequence workload: each sequence's context is injected into its
    # own cache at its ragged length; checked on the first sequence and the
    # longest one
    dc = CONFIGS[3]
    lens = synth.ragged_lengths(32)
    for s in (0, int(np.argmax(lens))):
        T = int(lens[s])
        rng = np.random.default_rng(10 + s)
        rows = np.unique(np.concatenate([rng.choice(T, 8, replace=False), [T - 1]]))
        _inject_check(dc, T, [T], rows=rows, seq=s)


def test_trim_then_append_overwrites_rejected_rows():
    dc = CONFIGS[0]
    d, w = make(dc, max_tokens=32)
    ctx = synth.make_feats(dc, 30, device=DEV)[1]
    junk = synth.make_feats(dc, 16, device=DEV)[2]
    kv = poisoned_kv(d, 40)
    d.inject_kv(kv, ctx[:10], 0)
    S = 10
    for tau in (3, 1, 5):
        d.inject_kv(kv, junk[:6], S)      # a later-rejected write past S
        d.kv_trim(kv, S)
        d.inject_kv(kv, ctx[S:S + tau], S)
        S += tau
    assert kv.len == S == 19
    ref = poisoned_kv(d, 40)
    d.inject_kv(ref, ctx[:S], 0)
    torch.cuda.synchronize()
    for i in range(dc.n_layers):
        assert_close_rms(np32(kv.k_view(i)[:, :S]), np32(ref.k_view(i)[:, :S]), tol=1e-2)
        assert_close_rms(np32(kv.v_view(i)[:, :, :S]), np32(ref.v_view(i)[:, :, :S]), tol=1e-2)
