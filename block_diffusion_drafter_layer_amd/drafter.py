"""Torch-side convenience around the C ABI: device memory and streams only.

``Drafter`` owns a handle, its workspace tensor and helper constructors for
KV-cache buffers; each method is one ABI call. Nothing here computes any part
of the method.
"""
from typing import Dict, List, Optional, Sequence

import torch

from . import binding as B


class KVCache:
    """A dflash_kv plus the device tensor that backs it."""

    def __init__(self, cfg: B.dflash_config, max_ctx: int, device):
        nbytes = B.dflash_kv_bytes(cfg, max_ctx)
        if nbytes == 0:
            raise ValueError("invalid config or max_ctx for a KV cache")
        self.buf = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=device)
        self.kv = B.dflash_kv(self.buf.data_ptr(), max_ctx, 0)
        self.cap = B.dflash_kv_row_capacity(cfg, max_ctx)
        self.n_layers, self.n_kv_heads, self.head_dim = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim

    @property
    def len(self) -> int:
        return self.kv.len

    def planes(self):
        """View [L, 2, Hkv, cap*hd]: K planes are [cap, hd], V planes [hd, cap]."""
        return self.buf.view(self.n_layers, 2, self.n_kv_heads, self.cap * self.head_dim)

    def k_view(self, layer: int):
        """[Hkv, cap, hd] view of one layer's K (position-major)."""
        return self.planes()[layer, 0].view(self.n_kv_heads, self.cap, self.head_dim)

    def v_view(self, layer: int):
        """[Hkv, hd, cap] view of one layer's V (dim-major)."""
        return self.planes()[layer, 1].view(self.n_kv_heads, self.head_dim, self.cap)


class Drafter:
    def __init__(self, cfg: B.dflash_config, weights: Dict, max_seqs: int = 1,
                 max_tokens: int = 2048, device="cuda", stream: Optional[torch.cuda.Stream] = None):
        self.cfg = cfg
        self.device = torch.device(device)
        self.weights = B.Weights(weights)
        self.stream = stream or torch.cuda.current_stream(self.device)
        self.h = B.dflash_create(cfg, self.weights.struct, self.stream.cuda_stream)
        nbytes = B.dflash_workspace_bytes(cfg, max_seqs, max_tokens)
        if nbytes == 0:
            raise ValueError("invalid workspace request")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        B.dflash_set_workspace(self.h, self.ws.data_ptr(), nbytes, max_seqs, max_tokens)
        self.max_seqs, self.max_tokens = max_seqs, max_tokens

    def close(self):
        if self.h is not None:
            B.dflash_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def new_kv(self, max_ctx: int) -> KVCache:
        return KVCache(self.cfg, max_ctx, self.device)

    def fuse_context(self, feats: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None):
        T, ld = feats[0].shape[0], feats[0].stride(0)
        if out is None:
            out = torch.empty(T, self.cfg.hidden, dtype=torch.bfloat16, device=self.device)
        B.dflash_fuse_context(self.h, [f.data_ptr() for f in feats], ld, T, out.data_ptr())
        return out

    def inject_kv(self, kv: KVCache, ctx_feat: torch.Tensor, pos0: Optional[int] = None):
        pos0 = kv.len if pos0 is None else pos0
        B.dflash_inject_kv(self.h, kv.kv, ctx_feat.data_ptr(), ctx_feat.shape[0], pos0)

    def kv_trim(self, kv: KVCache, keep: int):
        B.dflash_kv_trim(self.h, kv.kv, keep)

    def draft_block(self, kvs: Sequence[KVCache], anchors: torch.Tensor, block_len: Optional[int] = None,
                    block_out: Optional[torch.Tensor] = None, hidden: bool = False,
                    logits: bool = False):
        bl = self.cfg.block_size if block_len is None else block_len
        n = len(kvs)
        if block_out is None:
            block_out = torch.empty(n, bl, dtype=torch.int32, device=self.device)
        hid = (torch.empty(self.cfg.n_layers, n * bl, self.cfg.hidden, dtype=torch.float32,
                           device=self.device) if hidden else None)
        lg = (torch.empty(n, max(bl - 1, 0), self.cfg.vocab, dtype=torch.float32, device=self.device)
              if logits and bl > 1 else None)
        B.dflash_draft_block(self.h, [k.kv for k in kvs], anchors.data_ptr(), bl, block_out.data_ptr(),
                             hid.data_ptr() if hid is not None else 0,
                             lg.data_ptr() if lg is not None else 0)
        return block_out, hid, lg

    # --- device-resident rounds: lengths in a device int32 tensor -------------
    def draft_block_dev(self, kvs: Sequence[KVCache], len_dev: torch.Tensor, anchors: torch.Tensor,
                        block_out: torch.Tensor, hidden: Optional[torch.Tensor] = None,
                        logits: Optional[torch.Tensor] = None):
        B.dflash_draft_block_dev(self.h, [k.kv for k in kvs], len_dev.data_ptr(), anchors.data_ptr(),
                                 block_out.shape[1], block_out.data_ptr(),
                                 hidden.data_ptr() if hidden is not None else 0,
                                 logits.data_ptr() if logits is not None else 0)
        return block_out

    def append_dev(self, kvs: Sequence[KVCache], len_dev: torch.Tensor, tau_dev: torch.Tensor,
                   feats: Sequence[torch.Tensor], rows_per_seq: int):
        B.dflash_append_dev(self.h, [k.kv for k in kvs], len_dev.data_ptr(), tau_dev.data_ptr(),
                            [f.data_ptr() for f in feats], feats[0].stride(0), rows_per_seq)

    def kv_trim_dev(self, len_dev: torch.Tensor, keep: int):
        B.dflash_kv_trim_dev(self.h, len_dev.shape[0], len_dev.data_ptr(), keep)

    def sample_draft(self, block_ids: torch.Tensor, draft_logits: torch.Tensor, temperature: float,
                     seed: int = 0, philox_offset: int = 0):
        """Overwrite block_ids[:, 1:] with tokens sampled from the draft logits."""
        n, bl = block_ids.shape
        B.dflash_sample_draft(self.h, n, bl, draft_logits.data_ptr(), temperature, seed,
                              philox_offset, block_ids.data_ptr())
        return block_ids

    # --- DFlash 2 convs inside every layer --------------------------------------
    def set_conv(self, conv: Optional[Dict]):
        """Borrow the convs' bf16 tables ({"group_size", "layers": [{attn_base,
        attn_proj, mlp_base, mlp_proj}]}, kept alive by this object); None
        removes them."""
        if conv is None:
            self._conv = None
            B.dflash_set_conv(self.h, None, 0)
            return
        self._conv = conv
        layers = [B.dflash_conv_layer(l["attn_base"].data_ptr(), l["attn_proj"].data_ptr(),
                                      l["mlp_base"].data_ptr(), l["mlp_proj"].data_ptr())
                  for l in conv["layers"]]
        B.dflash_set_conv(self.h, layers, conv["group_size"])

    # --- DFlash 2 candidate selector -------------------------------------------
    def set_selector(self, hidden_proj: torch.Tensor, pred_codebook: torch.Tensor,
                     succ_codebook: torch.Tensor, top_k: int):
        """Borrow the selector's bf16 tables (kept alive by this object)."""
        self._sel = (hidden_proj, pred_codebook, succ_codebook)
        sel = B.dflash_selector(hidden_proj.data_ptr(), pred_codebook.data_ptr(),
                                succ_codebook.data_ptr(), hidden_proj.shape[0], top_k)
        B.dflash_set_selector(self.h, sel)

    def select_block(self, block_ids: torch.Tensor, last_hidden: torch.Tensor,
                     draft_logits: torch.Tensor, anchors: torch.Tensor, temperature: float = 0.0,
                     seed: int = 0, philox_offset: int = 0, cand: Optional[torch.Tensor] = None,
                     q: Optional[torch.Tensor] = None):
        """Overwrite block_ids[:, 1:] with the selector's walk over the candidates."""
        n, bl = block_ids.shape
        B.dflash_select_block(self.h, n, bl, last_hidden.data_ptr(), draft_logits.data_ptr(),
                              anchors.data_ptr(), temperature, seed, philox_offset,
                              block_ids.data_ptr(), cand.data_ptr() if cand is not None else 0,
                              q.data_ptr() if q is not None else 0)
        return block_ids

    def conv_prepare(self, x: torch.Tensor, prev: torch.Tensor, base: torch.Tensor,
                     proj: torch.Tensor, block_len: int, group_size: int = 16):
        """DFlash 2 dynamic conv, prepare call: returns (y, the finish call's
        corrections). x fp32 [n_seqs * block_len, hidden], prev [n_seqs, hidden],
        base bf16 [2, 2, hidden], proj bf16 [4 * hidden / group_size, hidden]."""
        n = prev.shape[0]
        y = torch.empty_like(x)
        corr = torch.empty(x.shape[0], 2 * (x.shape[1] // group_size), dtype=torch.float32,
                           device=x.device)
        B.dflash_conv_prepare(self.h, n, block_len, group_size, base.data_ptr(), proj.data_ptr(),
                              x.data_ptr(), prev.data_ptr(), y.data_ptr(), corr.data_ptr())
        return y, corr

    def conv_finish(self, z: torch.Tensor, prev: torch.Tensor, base: torch.Tensor,
                    corr: torch.Tensor, block_len: int, group_size: int = 16):
        """DFlash 2 dynamic conv, finish call with the prepare call's corrections."""
        y = torch.empty_like(z)
        B.dflash_conv_finish(self.h, prev.shape[0], block_len, group_size, base.data_ptr(),
                             z.data_ptr(), prev.data_ptr(), corr.data_ptr(), y.data_ptr())
        return y

    def verify_candidates(self, block_ids: torch.Tensor, target_logits: torch.Tensor,
                          cand: torch.Tensor, q_rows: torch.Tensor, temperature: float,
                          seed: int = 0, philox_offset: int = 0):
        """p/q verification with q on the selector's candidate sets."""
        n, bl = block_ids.shape
        tau = torch.empty(n, dtype=torch.int32, device=self.device)
        bonus = torch.empty(n, dtype=torch.int32, device=self.device)
        B.dflash_verify_candidates(self.h, n, bl, block_ids.data_ptr(), target_logits.data_ptr(),
                                   cand.data_ptr(), q_rows.data_ptr(), cand.shape[-1],
                                   temperature, seed, philox_offset, tau.data_ptr(),
                                   bonus.data_ptr())
        return tau, bonus

    def verify(self, block_ids: torch.Tensor, target_logits: torch.Tensor,
               draft_logits: Optional[torch.Tensor] = None, temperature: float = 0.0,
               seed: int = 0, philox_offset: int = 0, tau: Optional[torch.Tensor] = None,
               bonus: Optional[torch.Tensor] = None):
        n, bl = block_ids.shape
        tau = torch.empty(n, dtype=torch.int32, device=self.device) if tau is None else tau
        bonus = torch.empty(n, dtype=torch.int32, device=self.device) if bonus is None else bonus
        B.dflash_verify(self.h, n, bl, block_ids.data_ptr(), target_logits.data_ptr(),
                        draft_logits.data_ptr() if draft_logits is not None else 0,
                        temperature, seed, philox_offset, tau.data_ptr(), bonus.data_ptr())
        return tau, bonus


def config_from(dc) -> B.dflash_config:
    """dflash_config from a workload description (synth.DraftConfig)."""
    return B.make_config(dc.hidden, dc.n_feat, dc.n_layers, dc.n_heads, dc.n_kv_heads,
                         dc.head_dim, dc.ffn, dc.vocab, dc.block_size, dc.mask_token_id,
                         dc.rms_eps, dc.rope_theta)
