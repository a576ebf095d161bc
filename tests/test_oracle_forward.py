"""Pins of the oracle's full draft forward.

The pages print no values for a draft forward (no trained weights exist), so
the forward is pinned by an independent fp64 composition written with torch
CPU operators (torch's rms_norm, complex-number RoPE, scaled_dot_product_attention,
silu), by constructed argmax ties, and by degenerate cases.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth
from synth import CONFIGS


def _np_weights(w):
    f = lambda t: t.float().numpy()  # noqa: E731
    out = {k: f(v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: f(v) for k, v in lw.items()} for lw in w["layers"]]
    return out


def _torch_rope(x, pos, theta):
    # the pair (x_d, x_{d+hd/2}) as the complex number x_d + i x_{d+hd/2},
    # multiplied by exp(i * pos * theta^(-2d/hd))
    hd = x.shape[-1]
    half = hd // 2
    z = torch.complex(x[..., :half], x[..., half:])
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / hd)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    z = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def _torch_forward(cfg, w, ctx_k, ctx_v, anchor, S, bf16_block=False):
    t = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.float64)  # noqa: E731
    B, Hq, Hkv, hd = cfg.block_size, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    ids = torch.tensor([anchor] + [cfg.mask_token_id] * (B - 1))
    x = t(w["embed"])[ids]
    pos = torch.arange(S, S + B)
    hs = []
    for i, lw in enumerate(w["layers"]):
        h = F.rms_norm(x, (cfg.hidden,), t(lw["attn_norm"]), cfg.rms_eps)
        q = _torch_rope((h @ t(lw["wq"]).T).view(B, Hq, hd), pos, cfg.rope_theta)
        kb = _torch_rope((h @ t(lw["wk"]).T).view(B, Hkv, hd), pos, cfg.rope_theta)
        vb = (h @ t(lw["wv"]).T).view(B, Hkv, hd)
        if bf16_block:  # the block's rows rounded to bf16 (a deliberately different model)
            kb = kb.to(torch.float32).to(torch.bfloat16).to(torch.float64)
            vb = vb.to(torch.float32).to(torch.bfloat16).to(torch.float64)
        k = torch.cat([t(ctx_k[i]), kb]) if S else kb
        v = torch.cat([t(ctx_v[i]), vb]) if S else vb
        G = Hq // Hkv
        kk = k.transpose(0, 1).repeat_interleave(G, dim=0)
        vv = v.transpose(0, 1).repeat_interleave(G, dim=0)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), kk, vv)
        x = x + o.transpose(0, 1).reshape(B, Hq * hd) @ t(lw["wo"]).T
        h2 = F.rms_norm(x, (cfg.hidden,), t(lw["mlp_norm"]), cfg.rms_eps)
        x = x + (F.silu(h2 @ t(lw["w_gate"]).T) * (h2 @ t(lw["w_up"]).T)) @ t(lw["w_down"]).T
        hs.append(x.clone())
    z = F.rms_norm(x[1:], (cfg.hidden,), t(w["final_norm"]), cfg.rms_eps)
    logits = z @ t(w["lm_head"]).T
    return torch.stack(hs).numpy(), logits.numpy(), torch.argmax(logits, -1).numpy()


def _setup(cfg, S, gains="random"):
    w = _np_weights(synth.make_weights(cfg, gains=gains))
    ck, cv = [], []
    for i in range(cfg.n_layers):
        k, v = synth.gen.make_context_kv(cfg, i, S)
        ck.append(k.double().numpy()); cv.append(v.double().numpy())
    cache = O.DraftCache(cfg.n_layers, k=ck, v=cv) if S else O.DraftCache(cfg.n_layers)
    return w, ck, cv, cache


@pytest.mark.parametrize("n_layers,S", [(1, 10), (2, 10), (2, 0), (1, 37)])
def test_forward_matches_independent_torch_composition(n_layers, S):
    cfg = CONFIGS[0].shrink(n_layers=n_layers)
    w, ck, cv, cache = _setup(cfg, S)
    anchor = int(synth.make_anchor(cfg)[0])
    out = O.draft_block(cfg, w, [cache], [anchor])
    hs, logits, draft = _torch_forward(cfg, w, ck, cv, anchor, S)
    np.testing.assert_allclose(out["hidden"][:, 0], hs, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["logits"][0], logits, rtol=1e-10, atol=1e-10)
    np.testing.assert_array_equal(out["draft"][0], draft)
    assert (out["gap"][0] >= 0).all()


def test_forward_reduced_qwen_shape():
    # a reduced Qwen3-8B-shaped layer: GQA 32/8, head_dim 128, theta 1e6
    cfg = CONFIGS[1].shrink(hidden=256, n_layers=1, ffn=512, vocab=4096,
                            n_heads=8, n_kv_heads=2, head_dim=128, index=91)
    w, ck, cv, cache = _setup(cfg, 19)
    out = O.draft_block(cfg, w, [cache], [5])
    hs, logits, draft = _torch_forward(cfg, w, ck, cv, 5, 19)
    np.testing.assert_allclose(out["hidden"][:, 0], hs, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(out["draft"][0], draft)


def test_bf16_cache_leaves_the_block_rows_unrounded():
    # a bf16 cache rounds the context rows it stores, never the block's own
    # K/V rows (they exist only inside the forward): with context rows that
    # are bf16 values already, the bf16 cache gives exactly the plain result,
    # and the composition with the block rows rounded to bf16 differs from it
    cfg = CONFIGS[0].shrink(n_layers=2)
    w, ck, cv, _ = _setup(cfg, 10)
    anchor = int(synth.make_anchor(cfg)[0])
    cache = O.DraftCache(cfg.n_layers, k=ck, v=cv, bf16_kv=True)
    out = O.draft_block(cfg, w, [cache], [anchor])
    hs, logits, _ = _torch_forward(cfg, w, ck, cv, anchor, 10)
    np.testing.assert_allclose(out["hidden"][:, 0], hs, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["logits"][0], logits, rtol=1e-10, atol=1e-10)
    plain = O.draft_block(cfg, w, [O.DraftCache(cfg.n_layers, k=ck, v=cv)], [anchor])
    np.testing.assert_array_equal(plain["hidden"], out["hidden"])
    hs_rounded, _, _ = _torch_forward(cfg, w, ck, cv, anchor, 10, bf16_block=True)
    assert np.abs(hs_rounded - out["hidden"][:, 0]).max() > 1e-6


def test_argmax_ties_take_lowest_index():
    cfg = CONFIGS[0]
    w, ck, cv, cache = _setup(cfg, 10, gains="ones")
    out = O.draft_block(cfg, w, [cache], [3])
    top = out["draft"][0]
    # duplicate the winning LM-head row of row 0 at a lower and a higher index
    t0 = int(top[0])
    lo, hi = (0, cfg.vocab - 2) if t0 not in (0, cfg.vocab - 2) else (1, cfg.vocab - 3)
    w2 = dict(w); lm = w["lm_head"].copy()
    lm[hi] = lm[t0]
    w2["lm_head"] = lm
    assert O.draft_block(cfg, w2, [cache], [3])["draft"][0][0] == min(t0, hi)
    lm[lo] = lm[t0]
    assert O.draft_block(cfg, w2, [cache], [3])["draft"][0][0] == min(lo, t0)


def test_block_len_one_and_sequences_independent():
    cfg = CONFIGS[0]
    w, ck, cv, cache = _setup(cfg, 10)
    one = O.draft_block(cfg, w, [cache], [7], block_len=1)
    assert one["draft"].shape == (1, 0)
    # two sequences in one call give the same rows as two separate calls
    c2 = O.DraftCache(cfg.n_layers, k=[k[:6] for k in ck], v=[v[:6] for v in cv])
    both = O.draft_block(cfg, w, [cache, c2], [7, 9])
    a = O.draft_block(cfg, w, [cache], [7])
    b = O.draft_block(cfg, w, [c2], [9])
    np.testing.assert_array_equal(both["hidden"][:, 0], a["hidden"][:, 0])
    np.testing.assert_array_equal(both["hidden"][:, 1], b["hidden"][:, 0])


def test_context_changes_every_block_row():
    # the context K/V reach all block rows including the anchor (no causal mask)
    cfg = CONFIGS[0]
    w, ck, cv, cache = _setup(cfg, 10)
    base = O.draft_block(cfg, w, [cache], [7])["hidden"][0, 0]
    cv2 = [v.copy() for v in cv]; cv2[0][3] += 1.0
    alt = O.draft_block(cfg, w, [O.DraftCache(cfg.n_layers, k=ck, v=cv2)], [7])["hidden"][0, 0]
    assert (np.abs(alt - base).max(axis=-1) > 1e-6).all()


# ---------------------------------------------------------------------------
# the DFlash 2 conv inside every layer
# ---------------------------------------------------------------------------

def _conv_weights(cfg, seed, gs=16, identity=False):
    r = np.random.default_rng(seed)
    D, G = cfg.hidden, cfg.hidden // gs
    layers = []
    for _ in range(cfg.n_layers):
        lw = {}
        for inst in ("attn", "mlp"):
            if identity:
                base = np.zeros((2, 2, D))
                base[:, 0, :] = 1.0          # tap 0 passes x_t, tap 1 drops x_{t-1}
                proj = np.zeros((4 * G, D))
            else:
                base = 0.5 * r.standard_normal((2, 2, D))
                proj = r.standard_normal((4 * G, D)) / np.sqrt(D)
            lw[inst + "_base"], lw[inst + "_proj"] = base, proj
        layers.append(lw)
    return {"group_size": gs, "layers": layers}


def _brute_conv(rows, h, base_call, proj, call, gs):
    """y_t = k_{t,0} x_t + k_{t,1} x_{t-1} with element loops: k_{t,j} of
    channel c = base_call[j][c] + (proj row (call, j, c // gs)) . h_t; the
    block's first row reads a zero row."""
    T, D = len(rows), len(rows[0])
    G = D // gs
    out = []
    for t in range(T):
        y = []
        for c in range(D):
            g = c // gs
            k = []
            for j in range(2):
                row = proj[call * 2 * G + j * G + g]
                k.append(base_call[j][c] + sum(float(row[e]) * float(h[t][e]) for e in range(D)))
            before = float(rows[t - 1][c]) if t > 0 else 0.0
            y.append(k[0] * float(rows[t][c]) + k[1] * before)
        out.append(y)
    return torch.tensor(out, dtype=torch.float64)


def _torch_forward_conv(cfg, w, ctx_k, ctx_v, anchor, S, conv):
    """_torch_forward with the reading's conv placement, the conv by element loops."""
    t = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.float64)  # noqa: E731
    B, Hq, Hkv, hd = cfg.block_size, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    gs = conv["group_size"]
    ids = torch.tensor([anchor] + [cfg.mask_token_id] * (B - 1))
    x = t(w["embed"])[ids]
    pos = torch.arange(S, S + B)
    hs = []
    for i, lw in enumerate(w["layers"]):
        cw = conv["layers"][i]
        h = F.rms_norm(x, (cfg.hidden,), t(lw["attn_norm"]), cfg.rms_eps)
        hp = _brute_conv(h.tolist(), h.tolist(), cw["attn_base"][0], cw["attn_proj"], 0, gs)
        q = _torch_rope((hp @ t(lw["wq"]).T).view(B, Hq, hd), pos, cfg.rope_theta)
        kb = _torch_rope((hp @ t(lw["wk"]).T).view(B, Hkv, hd), pos, cfg.rope_theta)
        vb = (hp @ t(lw["wv"]).T).view(B, Hkv, hd)
        k = torch.cat([t(ctx_k[i]), kb]) if S else kb
        v = torch.cat([t(ctx_v[i]), vb]) if S else vb
        G = Hq // Hkv
        kk = k.transpose(0, 1).repeat_interleave(G, dim=0)
        vv = v.transpose(0, 1).repeat_interleave(G, dim=0)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), kk, vv)
        a = o.transpose(0, 1).reshape(B, Hq * hd) @ t(lw["wo"]).T
        a = _brute_conv(a.tolist(), h.tolist(), cw["attn_base"][1], cw["attn_proj"], 1, gs)
        x = x + a
        h2 = F.rms_norm(x, (cfg.hidden,), t(lw["mlp_norm"]), cfg.rms_eps)
        h2p = _brute_conv(h2.tolist(), h2.tolist(), cw["mlp_base"][0], cw["mlp_proj"], 0, gs)
        m = (F.silu(h2p @ t(lw["w_gate"]).T) * (h2p @ t(lw["w_up"]).T)) @ t(lw["w_down"]).T
        m = _brute_conv(m.tolist(), h2.tolist(), cw["mlp_base"][1], cw["mlp_proj"], 1, gs)
        x = x + m
        hs.append(x.clone())
    return torch.stack(hs).numpy()


def test_conv_identity_kernels_give_the_plain_forward():
    # base taps (1, 0) for both calls and a zero projection: every conv is the
    # identity, so the forward equals the one without convs bit for bit
    cfg = CONFIGS[0].shrink(n_layers=2)
    w, ck, cv, cache = _setup(cfg, 10)
    anchor = int(synth.make_anchor(cfg)[0])
    plain = O.draft_block(cfg, w, [cache], [anchor])
    ident = O.draft_block(cfg, w, [cache], [anchor], conv=_conv_weights(cfg, 0, identity=True))
    np.testing.assert_array_equal(plain["hidden"], ident["hidden"])
    np.testing.assert_array_equal(plain["logits"], ident["logits"])


def test_conv_forward_matches_element_by_element_brute_force():
    cfg = CONFIGS[0].shrink(n_layers=2)
    w, ck, cv, cache = _setup(cfg, 10)
    anchor = int(synth.make_anchor(cfg)[0])
    conv = _conv_weights(cfg, 3)
    out = O.draft_block(cfg, w, [cache], [anchor], conv=conv)
    hs = _torch_forward_conv(cfg, w, ck, cv, anchor, 10, conv)
    np.testing.assert_allclose(out["hidden"][:, 0], hs, rtol=1e-9, atol=1e-11)
    plain = O.draft_block(cfg, w, [cache], [anchor])
    assert np.abs(plain["hidden"] - out["hidden"]).max() > 1e-2


def test_conv_instances_are_not_interchangeable():
    # the attention instance and the MLP instance act at different places:
    # swapping their weights moves the result
    cfg = CONFIGS[0].shrink(n_layers=1)
    w, ck, cv, cache = _setup(cfg, 10)
    anchor = int(synth.make_anchor(cfg)[0])
    conv = _conv_weights(cfg, 5)
    ref = _torch_forward_conv(cfg, w, ck, cv, anchor, 10, conv)
    out = O.draft_block(cfg, w, [cache], [anchor], conv=conv)
    np.testing.assert_allclose(out["hidden"][:, 0], ref, rtol=1e-9, atol=1e-11)
    # swapping the two instances' weights moves the result
    swapped = {"group_size": 16, "layers": [{"attn_base": l["mlp_base"], "attn_proj": l["mlp_proj"],
                                             "mlp_base": l["attn_base"], "mlp_proj": l["attn_proj"]}
                                            for l in conv["layers"]]}
    other = O.draft_block(cfg, w, [cache], [anchor], conv=swapped)
    assert np.abs(other["hidden"] - out["hidden"]).max() > 1e-3
