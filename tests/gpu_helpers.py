"""Shared setup for the GPU parity tests: build a drafter on cuda:0 from the
seeded workload weights, hand the same bf16 values to the oracle, compare with
the stated tolerances.

Tolerances:
  * draft hidden states (every layer's residual stream): max-abs error <=
    3e-2 x the RMS of the oracle tensor;
  * drafted tokens: identical, except rows where the oracle's top-2 logit gap
    is below 1e-2;
  * fused context / K / V: max-abs error <= 3e-2 x RMS as well (bf16 outputs
    of fp32-accumulated bf16 products);
  * verification: tau and bonus bit-exact (p/q: outside the exclusion bands).

Storage precision: the library stores the fused context H_t and every K/V
cache row as bf16, as the pages' BF16 model does (the txtmix article,
section 5, sizes the projection's output and the weights at two bytes per
element). The oracle's caches here are built with bf16_kv=True and the
oracle's own H_t is rounded to bf16 before it is injected; everything else
on the oracle side stays fp64.
"""
import numpy as np
import torch

import oracle as O
import synth
from block_diffusion_drafter_layer_amd.drafter import Drafter, config_from

DEV = "cuda"
HIDDEN_TOL = 3e-2
GAP_TOL = 1e-2


def say(msg: str):
    print(msg, flush=True)


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def weights_np(w):
    out = {k: np32(v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: np32(v) for k, v in lw.items()} for lw in w["layers"]]
    return out


def make(dc, max_seqs=1, max_tokens=256, gains="ones"):
    w = synth.make_weights(dc, device=DEV, gains=gains)
    d = Drafter(config_from(dc), w, max_seqs=max_seqs, max_tokens=max_tokens, device=DEV)
    return d, w


def poisoned_kv(d: Drafter, max_ctx: int):
    kv = d.new_kv(max_ctx)
    kv.buf.fill_(float("nan"))  # rows outside the context must never be read
    return kv


def fill_context(kv, layer_kv):
    """Write context K/V rows [S, Hkv, hd] of every layer straight into the cache."""
    S = layer_kv[0][0].shape[0]
    for i, (k, v) in enumerate(layer_kv):
        kv.k_view(i)[:, :S, :] = k.transpose(0, 1)
        kv.v_view(i)[:, :, :S] = v.permute(1, 2, 0)
    kv.kv.len = S


def synthetic_context(dc, S, seq=0):
    return [tuple(t.to(DEV) for t in synth.gen.make_context_kv(dc, i, S, seq=seq))
            for i in range(dc.n_layers)]


def oracle_cache(dc, layer_kv):
    """The oracle's cache for the given bf16 context rows. It stores rows as
    bf16, as the library's cache does (the pages' model is BF16)."""
    c = O.DraftCache(dc.n_layers, bf16_kv=True)
    if layer_kv[0][0].shape[0] == 0:
        return c
    c.k = [np32(k).astype(np.float64) for k, _ in layer_kv]
    c.v = [np32(v).astype(np.float64) for _, v in layer_kv]
    return c


def rms(x):
    return float(np.sqrt(np.mean(np.asarray(x, np.float64) ** 2)))


def assert_close_rms(gpu, ref, tol=HIDDEN_TOL, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref).max()
    bound = tol * rms(ref)
    assert err <= bound, f"{what}: max-abs {err:.3e} > {bound:.3e} (rms {rms(ref):.3e})"
    return err / max(rms(ref), 1e-30)


def assert_hidden(gpu_hidden, orc_hidden, what="hidden"):
    """gpu [L, n*B, D] vs oracle [L, n, B, D]."""
    L = orc_hidden.shape[0]
    ref = orc_hidden.reshape(L, -1, orc_hidden.shape[-1])
    worst = 0.0
    for i in range(L):
        worst = max(worst, assert_close_rms(gpu_hidden[i], ref[i], what=f"{what} layer {i}"))
    return worst


def assert_tokens(gpu_block, orc, what="draft"):
    """gpu block [n, B] (anchor + drafts) vs oracle draft [n, B-1] and gap."""
    g = np.asarray(gpu_block)[:, 1:]
    o = np.asarray(orc["draft"])
    gap = np.asarray(orc["gap"])
    bad = (g != o) & (gap >= GAP_TOL)
    assert not bad.any(), f"{what}: {int(bad.sum())} tokens differ with gap >= {GAP_TOL}"
    return int((g != o).sum())
