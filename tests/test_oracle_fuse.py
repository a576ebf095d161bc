"""Pins of the oracle's context fusion against the pages and mathematics."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, target_layer_ids_rule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fusion_worked_example.txt")


def _worked_example_inputs():
    # Input generation of the tutorial's example (torch is used only to draw).
    torch.manual_seed(42)
    hs = [torch.randn(10, 64) for _ in [2, 5, 8, 11, 14]]
    lin = torch.nn.Linear(5 * 64, 64, bias=False)
    return [h.double().numpy() for h in hs], lin.weight.detach().double().numpy()


def _golden():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    return np.array(rows, dtype=np.float64)


def test_worked_example_printed_values():
    feats, w_c = _worked_example_inputs()
    out = O.fuse_context(feats, w_c, np.ones(64), 1e-6)
    assert out.shape == (10, 64)
    np.testing.assert_allclose(out[:3, :8], _golden(), atol=5.001e-5, rtol=0)


def test_worked_example_catches_transposed_or_reordered_inputs():
    feats, w_c = _worked_example_inputs()
    g = _golden()
    # concat in reverse layer order must not reproduce the print
    bad = O.fuse_context(feats[::-1], w_c, np.ones(64), 1e-6)
    assert np.abs(bad[:3, :8] - g).max() > 1e-2
    # eps outside the square root changes nothing visible at 4 dp, but a norm
    # over the wrong axis does
    c = np.concatenate(feats, -1)
    y = c @ w_c.T
    wrong_axis = y / np.sqrt((y * y).mean(0, keepdims=True) + 1e-6)
    assert np.abs(wrong_axis[:3, :8] - g).max() > 1e-2


def test_concat_shape_and_output_shape():
    rng = np.random.default_rng(0)
    feats = [rng.standard_normal((10, 64)) for _ in range(5)]
    assert np.concatenate(feats, -1).shape == (10, 320)
    out = O.fuse_context(feats, rng.standard_normal((64, 320)) * 0.02, np.ones(64))
    assert out.shape == (10, 64)


def test_row_rms_invariant_with_gain():
    rng = np.random.default_rng(1)
    D = 48
    feats = [rng.standard_normal((7, D)) for _ in range(5)]
    w_c = rng.standard_normal((D, 5 * D)) * 0.02
    gain = 1 + 0.3 * rng.standard_normal(D)
    eps = 1e-6
    out = O.fuse_context(feats, w_c, gain, eps)
    y = np.concatenate(feats, -1) @ w_c.T
    m = (y * y).mean(-1)
    rms_unit = np.sqrt(((out / gain) ** 2).mean(-1))
    np.testing.assert_allclose(rms_unit, np.sqrt(m / (m + eps)), rtol=1e-12)


def test_selector_weights_pick_one_layer():
    rng = np.random.default_rng(2)
    D = 32
    feats = [rng.standard_normal((5, D)) for _ in range(5)]
    for k in range(5):
        w_c = np.zeros((D, 5 * D))
        w_c[:, k * D:(k + 1) * D] = np.eye(D)
        out = O.fuse_context(feats, w_c, np.ones(D), 1e-6)
        h = feats[k]
        ref = h / np.sqrt((h * h).mean(-1, keepdims=True) + 1e-6)
        np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_w_c_size_closed_form():
    # "about 42 MB" for D=2048 in bf16 (A3-dflash tutorial section 2.1.2;
    # txtmix article section 5): 5 * D * D * 2 bytes
    assert 5 * 2048 * 2048 * 2 == 41_943_040
    assert abs(5 * 2048 * 2048 * 2 / 1e6 - 42) < 0.5
    c5 = CONFIGS[4]
    assert c5.n_feat * c5.hidden * c5.hidden * 2 == 41_943_040
    c2 = CONFIGS[1]
    assert c2.n_feat * c2.hidden * c2.hidden * 2 == 167_772_160
    # activations at batch 1, 2048 tokens, D=2048: ~40 MB in, ~8 MB out (bf16)
    assert 2048 * 5 * 2048 * 2 == 40 * 2 ** 20
    assert 2048 * 2048 * 2 == 8 * 2 ** 20
    # a 16-row append buffer stays under 400 KB
    assert 16 * 5 * 2048 * 2 + 16 * 2048 * 2 < 400_000


def test_target_layer_rule():
    # txtmix article section 5: from index 1 to num_target_layers-3
    assert O.target_layer_ids(36, 5) == [1, 9, 17, 25, 33]
    assert O.target_layer_ids(48, 5) == [1, 12, 23, 34, 45]
    assert O.target_layer_ids(16, 5) == [1, 4, 7, 10, 13]
    assert O.target_layer_ids(36, 1) == [18]
    for n in range(8, 80):
        ids = O.target_layer_ids(n, 5)
        assert ids[0] == 1 and ids[-1] == n - 3 and ids == sorted(set(ids))
        assert ids == target_layer_ids_rule(n, 5)
