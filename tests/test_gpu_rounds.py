"""GPU parity of speculative rounds: draft -> verify -> trim -> append, at the
long-context workload (8192 context tokens, 4 rounds, block 16).

The initial 8192 context rows are seeded synthetic K/V written into both
caches; each round's accepted rows are then fused from fresh target hidden
states and injected by the library, exactly as a host loop would do after
verification (txtmix article section 9). Verification runs on the oracle's
drafted block (so no oracle input comes from the GPU path); the GPU's own
drafted tokens are compared with the oracle's under the top-2 gap rule."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import (DEV, assert_close_rms, assert_hidden, assert_tokens, fill_context,
                         make, np32, oracle_cache, poisoned_kv, say, synthetic_context,
                         weights_np)
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _rounds(dc, S0, n_rounds):
    B = dc.block_size
    d, w = make(dc, max_tokens=B)
    wn = weights_np(w)
    kv = poisoned_kv(d, S0 + B * (n_rounds + 1))
    ctx = synthetic_context(dc, S0)
    fill_context(kv, ctx)
    ocache = oracle_cache(dc, ctx)
    taus = synth.planted_taus(dc, n_rounds, salt=5)
    anchor = int(synth.make_anchor(dc)[0])
    S = S0
    for r in range(n_rounds):
        say(f"round {r}: context {S}, planted tau {int(taus[r])}")
        block, hid, _ = d.draft_block([kv], torch.tensor([anchor], dtype=torch.int32, device=DEV),
                                      hidden=True)
        torch.cuda.synchronize()
        assert kv.len == S
        orc = O.draft_block(dc, wn, [ocache], [anchor])
        assert_hidden(np32(hid), orc["hidden"], what=f"round {r}")
        assert_tokens(block.cpu().numpy(), orc, what=f"round {r}")
        # verification of the oracle's block against planted target logits
        blk = np.concatenate([[anchor], orc["draft"][0]]).astype(np.int32)
        lg = synth.make_target_logits(dc, B, round_index=10 + r)
        synth.plant_agreement(lg, blk, int(taus[r]) - 1)
        tau_g, bonus_g = d.verify(torch.from_numpy(blk[None]).to(DEV), lg[None].to(DEV))
        tau, bonus = O.verify_greedy(blk, lg.numpy())
        assert (int(tau_g[0]), int(bonus_g[0])) == (tau, bonus) and tau == taus[r]
        # trim to the accepted prefix, append its fused features
        feats = synth.make_feats(dc, tau, round_index=20 + r, device=DEV)
        d.kv_trim(kv, S)
        H = d.fuse_context(feats)
        d.inject_kv(kv, H, S)
        Ho = O.fuse_context([np32(f) for f in feats], wn["w_c"], wn["ctx_norm"], dc.rms_eps)
        assert_close_rms(np32(H), Ho, what=f"round {r} fused rows")
        O.cache_inject(ocache, Ho, wn["layers"], dc, S)
        S += tau
        anchor = bonus
        assert kv.len == S == ocache.len
    torch.cuda.synchronize()
    # the appended rows of the cache, layer by layer
    for i in range(dc.n_layers):
        gk = np32(kv.k_view(i)[:, S0:S, :]).transpose(1, 0, 2)
        gv = np32(kv.v_view(i)[:, :, S0:S]).transpose(2, 0, 1)
        assert_close_rms(gk, ocache.k[i][S0:S], what=f"appended K layer {i}")
        assert_close_rms(gv, ocache.v[i][S0:S], what=f"appended V layer {i}")
    return S


def test_rounds_tiny():
    _rounds(CONFIGS[0].shrink(index=98), 10, 4)


def test_rounds_long_context_qwen_shape():
    dc = CONFIGS[2]
    S = _rounds(dc, dc.ctx_len, dc.rounds)
    assert S > dc.ctx_len
