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

Storage precision: the library stores the fused context H_t and every
context K/V cache row as bf16, as the pages' BF16 model does (the txtmix
article, section 5, sizes the projection's output and the weights at two
bytes per element); the block's own K/V rows never enter the cache and stay
fp32. The GPU results are compared with the plain oracle (fp64 rows,
unrounded H_t) at the bounds above, and - as a regression check of the
kernels' own precision - with the oracle that stores the same rows as bf16
at TIGHT_TOL x RMS.
"""
import numpy as np
import torch

import oracle as O
import synth
from bf16_check import bad_bf16_rounding, check_bf16_rounding, midpoint_distance, row_rms
from block_diffusion_drafter_layer_amd.drafter import Drafter, config_from

DEV = "cuda"
HIDDEN_TOL = 3e-2
GAP_TOL = 1e-2
# regression bound: the GPU path against an oracle with the library's storage
# roundings (bf16 hi/lo activations and fp32 accumulation leave ~1e-4)
TIGHT_TOL = 2e-3


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


def oracle_cache(dc, layer_kv, bf16_kv=False):
    """The oracle's cache for the given context rows (bf16 values). Plain by
    default (fp64 rows; the given rows are bf16 values either way);
    bf16_kv=True rounds the rows appended later as the library stores them."""
    c = O.DraftCache(dc.n_layers, bf16_kv=bf16_kv)
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


def assert_hidden(gpu_hidden, orc_hidden, what="hidden", tol=HIDDEN_TOL):
    """gpu [L, n*B, D] vs oracle [L, n, B, D]; returns the per-layer max-abs / RMS."""
    L = orc_hidden.shape[0]
    ref = orc_hidden.reshape(L, -1, orc_hidden.shape[-1])
    errs = [assert_close_rms(gpu_hidden[i], ref[i], tol=tol, what=f"{what} layer {i}")
            for i in range(L)]
    return max(errs)


def hidden_errs(gpu_hidden, orc_hidden):
    """Per-layer max-abs error / RMS of the oracle (no assertion)."""
    L = orc_hidden.shape[0]
    ref = orc_hidden.reshape(L, -1, orc_hidden.shape[-1])
    g = np.asarray(gpu_hidden, np.float64).reshape(ref.shape)
    return [float(np.abs(g[i] - ref[i]).max() / rms(ref[i])) for i in range(L)]


def assert_tokens(gpu_block, orc, what="draft"):
    """gpu block [n, B] (anchor + drafts) vs oracle draft [n, B-1] and gap."""
    g = np.asarray(gpu_block)[:, 1:]
    o = np.asarray(orc["draft"])
    gap = np.asarray(orc["gap"])
    bad = (g != o) & (gap >= GAP_TOL)
    assert not bad.any(), f"{what}: {int(bad.sum())} tokens differ with gap >= {GAP_TOL}"
    return int((g != o).sum())


# Bands around the bf16 rounding midpoints inside which either bf16 neighbour
# is accepted: 8x the fp32 error the output carries before its one rounding,
# relative to the row RMS of the exact value. A K-term fp32 accumulation of
# random-sign bf16 products rounds every partial sum, an error of about
# 2^-24 sqrt(K/2) x RMS (the partial sums grow like sqrt(k)); a bf16 hi/lo
# pair carries 2^-17 / sqrt(3) of each element. Measured tails on the GPU
# (a few values in 1e5 beyond 2.3 of these sigmas) fix the factor of 8.
_U = 2.0 ** -24


def fuse_band(dc):
    """fusion: n_feat * D products, then the norm's row scale (a few ulp)"""
    return 8 * _U * np.sqrt(dc.n_feat * dc.hidden / 2) + 16 * _U


def inject_band(dc):
    """injection: D products, then the rotation with fp32 cos/sin"""
    return 8 * _U * np.sqrt(dc.hidden / 2) + 16 * _U


def append_band(dc):
    """device-resident append: the fused rows' own error, carried through the
    projection, plus the injection's, plus the hi/lo pair of the fused rows"""
    return float(np.sqrt(fuse_band(dc) ** 2 + inject_band(dc) ** 2 + (8 * 2.0 ** -17 / np.sqrt(3)) ** 2))


def assert_bf16_rounding(gpu, ref, band_rel, what, max_banded=0.15):
    """gpu == round_bf16(ref) outside a band of band_rel x (row RMS of ref)
    around the rounding midpoints; returns the number of banded values. On
    large samples the banded share must stay small (a sanity check that the
    band did not swallow the comparison)."""
    ref = np.asarray(ref, np.float64)
    band = band_rel * row_rms(ref)
    bad, banded, n = check_bf16_rounding(gpu, ref, band)
    say(f"  {what}: {n} values, {banded} within the midpoint band ({band_rel:.1e} x rms), {bad} wrong")
    if bad:
        idx = bad_bf16_rounding(gpu, ref, np.broadcast_to(band, ref.shape))
        g, r = np.asarray(gpu, np.float64).reshape(-1), ref.reshape(-1)
        b = np.broadcast_to(band, ref.shape).reshape(-1)
        for i in idx[:8]:
            say(f"    [{np.unravel_index(i, ref.shape)}] oracle {r[i]!r} gpu {g[i]!r} "
                f"round_bf16 {O.round_bf16(r[i:i + 1])[0]!r} midpoint distance / band "
                f"{midpoint_distance(r[i:i + 1])[0] / b[i]:.2f}")
    assert bad == 0, f"{what}: {bad} of {n} values are not round_bf16(oracle)"
    assert n < 4096 or banded <= max_banded * n, f"{what}: band too wide ({banded} of {n})"
    return banded
