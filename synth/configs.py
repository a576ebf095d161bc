"""Workload shapes of the DFlash drafter hot path.

Each workload is a draft model plus the target-side context it is fed.
The shapes follow the pages: a Qwen3-8B-class target (hidden 4096, 36 layers)
with a 5-layer draft and block size 16 (papercache DFlash summary, A4
experimental setup; txtmix code-reading article, section 11 ``dflash_config``),
a D=2048 target whose fusion matrix is about 42 MB (A3-dflash tutorial,
section 2.1.2; txtmix article, section 5), and the tutorial's toy fusion
example (16 target layers, hidden 64, 10 tokens, layers [2,5,8,11,14];
A3-dflash tutorial, section 2.1.1).
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional


def target_layer_ids_rule(n_target_layers: int, n_feat: int) -> List[int]:
    """Uniformly spaced target layer indices from 1 to n_target_layers-3.

    The txtmix article (section 5, build_target_layer_ids) says the ids are
    spread evenly between index 1 and num_target_layers-3 (0-based), with the
    middle layer when only one is taken. Non-integer grid points are rounded
    to nearest (halves up); the pages do not say how they are rounded.
    """
    if n_feat < 1 or n_target_layers < 4:
        raise ValueError("need n_feat >= 1 and n_target_layers >= 4")
    if n_feat == 1:
        return [n_target_layers // 2]
    lo, hi = 1, n_target_layers - 3
    return [int(lo + (hi - lo) * i / (n_feat - 1) + 0.5) for i in range(n_feat)]


@dataclass(frozen=True)
class DraftConfig:
    name: str
    hidden: int            # D, shared by target and draft
    n_target_layers: int
    feat_layer_ids: tuple  # which target layers are fused (5 of them)
    n_layers: int          # draft decoder layers
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    block_size: int
    ctx_len: int           # context tokens injected before the first block
    n_seqs: int = 1
    ragged: bool = False   # ragged per-sequence context lengths
    rounds: int = 1        # speculative rounds (trim/append between them)
    verify: str = "greedy"  # "greedy" or "pq"
    temperature: float = 0.0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    dtype: str = "bf16"
    index: int = 0         # position in the workload list; seeds derive from it

    @property
    def n_feat(self) -> int:
        return len(self.feat_layer_ids)

    @property
    def mask_token_id(self) -> int:
        # The pages leave mask_token_id to the checkpoint; the last vocab id
        # is used here and anchors are drawn from the others.
        return self.vocab - 1

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def shrink(self, **kw) -> "DraftConfig":
        return replace(self, **kw)


CONFIGS = [
    DraftConfig(
        name="tiny_d64_l1_b4_ctx10", hidden=64, n_target_layers=16,
        feat_layer_ids=(2, 5, 8, 11, 14), n_layers=1, n_heads=4, n_kv_heads=2,
        head_dim=16, ffn=128, vocab=1000, block_size=4, ctx_len=10,
        dtype="fp32", index=0),
    DraftConfig(
        name="qwen3_8b_shape_b16_ctx2048", hidden=4096, n_target_layers=36,
        feat_layer_ids=tuple(target_layer_ids_rule(36, 5)), n_layers=5,
        n_heads=32, n_kv_heads=8, head_dim=128, ffn=12288, vocab=151936,
        block_size=16, ctx_len=2048, index=1),
    DraftConfig(
        name="qwen3_8b_shape_b16_ctx8192_4rounds", hidden=4096,
        n_target_layers=36, feat_layer_ids=tuple(target_layer_ids_rule(36, 5)),
        n_layers=5, n_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
        vocab=151936, block_size=16, ctx_len=8192, rounds=4, index=2),
    DraftConfig(
        name="qwen3_8b_shape_b16_32seq_ragged", hidden=4096,
        n_target_layers=36, feat_layer_ids=tuple(target_layer_ids_rule(36, 5)),
        n_layers=5, n_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
        vocab=151936, block_size=16, ctx_len=4096, n_seqs=32, ragged=True,
        index=3),
    DraftConfig(
        name="d2048_b8_ctx2048_pq", hidden=2048, n_target_layers=48,
        feat_layer_ids=tuple(target_layer_ids_rule(48, 5)), n_layers=5,
        n_heads=16, n_kv_heads=4, head_dim=128, ffn=6144, vocab=151936,
        block_size=8, ctx_len=2048, verify="pq", temperature=1.0, index=4),
]
