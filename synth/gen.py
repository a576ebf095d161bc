"""Seeded draws for the workloads in ``configs``.

Every tensor has its own generator seeded with ``seed_for(workload, tensor)``
so a tensor's values do not depend on which other tensors were drawn before
it. Draws use ``torch.Generator`` on the requested device (CPU by default);
the same call on the same device returns the same values on every run.
"""
from typing import Dict, List, Optional

import numpy as np
import torch

from .configs import DraftConfig

# tensor ids inside one workload
_T_WC, _T_CTXNORM, _T_EMBED, _T_LMHEAD, _T_FINALNORM = 1, 2, 3, 4, 5
_LAYER_BASE = 10            # + 10 * layer + slot
_FEAT_BASE = 300            # + 10 * round + k
_ANCHOR_BASE = 400          # + round
_LOGIT_BASE = 500           # + round
_DLOGIT_BASE = 600          # + round
_TAU_BASE = 700
_RAGGED = 800
_CTXKV_BASE = 850           # + layer
_SEL_BASE = 900             # + 0 hidden projection, 1 predecessor, 2 successor codes
_CONV_BASE = 950            # + 0 base kernel, 1 projection, 2..5 rows
_CONV_LAYER_BASE = 200      # + 10 * layer + 2 * instance + (0 base, 1 projection)

LAYER_SLOTS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down",
               "attn_norm", "mlp_norm")


def seed_for(workload_index: int, tensor_id: int) -> int:
    return 1000 * workload_index + tensor_id


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std: float, seed: int, device, dtype=torch.bfloat16):
    g = _gen(seed, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _gain(n: int, mode: str, seed: int, device):
    if mode == "ones":
        return torch.ones(n, dtype=torch.bfloat16, device=device)
    # "random": gains near 1, used by tests so that a dropped gain shows up
    g = _gen(seed, device)
    t = 1.0 + 0.25 * torch.randn(n, generator=g, device=device)
    return t.to(torch.bfloat16)


def make_weights(cfg: DraftConfig, device="cpu", gains: str = "ones",
                 std: float = 0.02) -> Dict:
    """All draft-side parameters as bf16 tensors in nn.Linear [out, in] layout.

    w_c is [D, n_feat*D]; embed and lm_head are [V, D]; per layer wq [Hq*hd, D],
    wk/wv [Hkv*hd, D], wo [D, Hq*hd], w_gate/w_up [F, D], w_down [D, F].
    """
    D, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    s = lambda t: seed_for(cfg.index, t)  # noqa: E731
    w = {
        "w_c": _normal((D, cfg.n_feat * D), std, s(_T_WC), device),
        "ctx_norm": _gain(D, gains, s(_T_CTXNORM), device),
        "embed": _normal((V, D), std, s(_T_EMBED), device),
        "lm_head": _normal((V, D), std, s(_T_LMHEAD), device),
        "final_norm": _gain(D, gains, s(_T_FINALNORM), device),
        "layers": [],
    }
    shapes = {
        "wq": (cfg.q_dim, D), "wk": (cfg.kv_dim, D), "wv": (cfg.kv_dim, D),
        "wo": (D, cfg.q_dim), "w_gate": (F, D), "w_up": (F, D),
        "w_down": (D, F),
    }
    for i in range(cfg.n_layers):
        lw = {}
        for j, name in enumerate(LAYER_SLOTS):
            t = s(_LAYER_BASE + 10 * i + j)
            if name.endswith("norm"):
                lw[name] = _gain(D, gains, t, device)
            else:
                lw[name] = _normal(shapes[name], std, t, device)
        w["layers"].append(lw)
    return w


def make_selector(cfg: DraftConfig, rank: int = 256, device="cpu", code_std: float = 0.3) -> Dict:
    """Tables of a DFlash 2 candidate selector, bf16: hidden_proj [rank, D] with
    entries N(0, 1/D) (so the projected hidden state has entries of order 1),
    pred_codebook and succ_codebook [V, rank] with entries N(0, code_std^2)."""
    s = lambda t: seed_for(cfg.index, _SEL_BASE + t)  # noqa: E731
    return {
        "hidden_proj": _normal((rank, cfg.hidden), cfg.hidden ** -0.5, s(0), device),
        "pred_codebook": _normal((cfg.vocab, rank), code_std, s(1), device),
        "succ_codebook": _normal((cfg.vocab, rank), code_std, s(2), device),
    }


def make_conv(cfg: DraftConfig, n_seqs: int, block_len: int, group_size: int = 16,
              device="cpu") -> Dict:
    """One DFlash 2 dynamic-conv instance and its rows: base [2, 2, D] bf16 with
    entries N(0, 0.5^2), projection [4 * D / group_size, D] bf16 with entries
    N(0, 1/D) (corrections of order 1), and fp32 rows N(0, 1): x and z
    [n_seqs * block_len, D], prev and zprev [n_seqs, D]."""
    s = lambda t: seed_for(cfg.index, _CONV_BASE + t)  # noqa: E731
    D, rows = cfg.hidden, n_seqs * block_len
    f32 = torch.float32
    return {
        "base": _normal((2, 2, D), 0.5, s(0), device),
        "proj": _normal((4 * (D // group_size), D), D ** -0.5, s(1), device),
        "x": _normal((rows, D), 1.0, s(2), device, f32),
        "prev": _normal((n_seqs, D), 1.0, s(3), device, f32),
        "z": _normal((rows, D), 1.0, s(4), device, f32),
        "zprev": _normal((n_seqs, D), 1.0, s(5), device, f32),
    }


def make_conv_layers(cfg: DraftConfig, group_size: int = 16, device="cpu") -> Dict:
    """The DFlash 2 convs of every draft layer (one by attention, one by the
    MLP): per layer attn_base / mlp_base [2, 2, D] bf16 with entries
    N(0, 0.5^2) and attn_proj / mlp_proj [4 * D / group_size, D] bf16 with
    entries N(0, 1/D), as make_conv draws one instance."""
    D = cfg.hidden
    layers = []
    for i in range(cfg.n_layers):
        lw = {}
        for j, inst in enumerate(("attn", "mlp")):
            t = _CONV_LAYER_BASE + 10 * i + 2 * j
            lw[inst + "_base"] = _normal((2, 2, D), 0.5, seed_for(cfg.index, t), device)
            lw[inst + "_proj"] = _normal((4 * (D // group_size), D), D ** -0.5,
                                         seed_for(cfg.index, t + 1), device)
        layers.append(lw)
    return {"group_size": group_size, "layers": layers}


def make_feats(cfg: DraftConfig, n_tokens: int, round_index: int = 0,
               device="cpu") -> List[torch.Tensor]:
    """The fused target layers' hidden states: n_feat arrays [n_tokens, D] bf16."""
    return [
        _normal((n_tokens, cfg.hidden), 1.0,
                seed_for(cfg.index, _FEAT_BASE + 10 * round_index + k), device)
        for k in range(cfg.n_feat)
    ]


def make_context_kv(cfg: DraftConfig, layer: int, n_tokens: int, device="cpu",
                    seq: int = 0):
    """Synthetic context K/V rows [n_tokens, Hkv, hd] bf16, N(0,1).

    Used where the context is handed to the draft forward directly instead of
    being projected from fused target features.
    """
    sd = seed_for(cfg.index, _CTXKV_BASE + layer) * 100 + seq
    k = _normal((n_tokens, cfg.n_kv_heads, cfg.head_dim), 1.0, 2 * sd, device)
    v = _normal((n_tokens, cfg.n_kv_heads, cfg.head_dim), 1.0, 2 * sd + 1, device)
    return k, v


def make_anchor(cfg: DraftConfig, round_index: int = 0, n: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed_for(cfg.index, _ANCHOR_BASE + round_index))
    return rng.integers(0, cfg.vocab - 1, size=n).astype(np.int32)


def make_target_logits(cfg: DraftConfig, n_rows: int, round_index: int = 0,
                       device="cpu", draft: bool = False) -> torch.Tensor:
    base = _DLOGIT_BASE if draft else _LOGIT_BASE
    return _normal((n_rows, cfg.vocab), 1.0,
                   seed_for(cfg.index, base + round_index), device,
                   dtype=torch.float32)


def planted_taus(cfg: DraftConfig, n: int, salt: int = 0) -> np.ndarray:
    """tau = min(G, block_size), G ~ Geometric(0.25) on {1, 2, ...}."""
    rng = np.random.default_rng(seed_for(cfg.index, _TAU_BASE) + 7919 * salt)
    g = rng.geometric(0.25, size=n)
    return np.minimum(g, cfg.block_size).astype(np.int32)


def plant_agreement(logits: torch.Tensor, block_ids, a: int) -> torch.Tensor:
    """Plant an agreement length ``a`` into target logits [B, V] (in place).

    Rows j < a get block_ids[j+1] lifted to max(row)+1 so that the target's
    top token equals the drafted token there. If a < B-1, row a must not agree:
    when its top token happens to equal block_ids[a+1], that entry is dropped to
    min(row)-1. Rows after a are left as drawn.
    """
    B = logits.shape[0]
    ids = [int(x) for x in block_ids]
    for j in range(a):
        row = logits[j]
        row[ids[j + 1]] = row.max() + 1.0
    if a < B - 1:
        row = logits[a]
        if int(torch.argmax(row)) == ids[a + 1]:
            row[ids[a + 1]] = row.min() - 1.0
    return logits


def ragged_lengths(n: int, lo: int = 512, hi: int = 4096, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed_for(3, _RAGGED) + seed)
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)
