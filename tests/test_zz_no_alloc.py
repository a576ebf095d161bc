"""dflash_verify_noalloc (the verification for callers that cannot allocate)
against dflash_verify through the C ABI: tau and bonus identical, greedy and
p/q, two calls in a row, the second with fewer sequences and a shorter block
(the fixed scratch keeps the first call's contents). Its handle has no
workspace at all."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_drafter_layer_amd import binding as B
from gpu_helpers import DEV, make, say
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _bare_handle(dc, w):
    """A second handle on the same weights, never given a workspace."""
    from block_diffusion_drafter_layer_amd.drafter import config_from
    keep = B.Weights(w)
    h = B.dflash_create(config_from(dc), keep.struct, torch.cuda.current_stream().cuda_stream)
    return h, keep


def _case(dc, n, bl, temp, seed):
    g = torch.Generator().manual_seed(seed)
    ids = torch.randint(0, dc.vocab - 1, (n, bl), generator=g, dtype=torch.int32)
    tl = torch.randn(n, bl, dc.vocab, generator=g)
    dl = torch.randn(n, bl - 1, dc.vocab, generator=g) if temp > 0 else None
    if temp == 0:  # plant agreements so that tau varies
        for s in range(n):
            synth.plant_agreement(tl[s], ids[s].numpy(), int(seed + s) % bl)
    return ids.to(DEV), tl.to(DEV), (dl.to(DEV) if dl is not None else None)


def _both(d, h0, n, bl, ids, tl, dl, temp, seed, off):
    t1, b1 = (torch.full((n,), -7, dtype=torch.int32, device=DEV) for _ in range(2))
    t2, b2 = (torch.full((n,), -9, dtype=torch.int32, device=DEV) for _ in range(2))
    st = torch.cuda.current_stream().cuda_stream
    B.dflash_set_stream(d.h, st)
    B.dflash_verify(d.h, n, bl, ids.data_ptr(), tl.data_ptr(), dl.data_ptr() if dl is not None else 0,
                    temp, seed, off, t1.data_ptr(), b1.data_ptr())
    B.dflash_verify_noalloc(h0, n, bl, ids.data_ptr(), tl.data_ptr(),
                            dl.data_ptr() if dl is not None else 0, temp, seed, off, t2.data_ptr(),
                            b2.data_ptr())
    torch.cuda.synchronize()
    return t1.cpu(), b1.cpu(), t2.cpu(), b2.cpu()


@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_noalloc_verify_matches_verify_two_calls(temp):
    dc = CONFIGS[1] if temp == 0.0 else CONFIGS[4]
    say(f"verify_noalloc vs verify: config {dc.name} temperature {temp}")
    d, w = make(dc, max_seqs=8)
    h0, keep = _bare_handle(dc, w)
    try:
        for n, bl, seed in ((8, dc.block_size, 5), (3, dc.block_size - 3, 6)):
            ids, tl, dl = _case(dc, n, bl, temp, seed)
            t1, b1, t2, b2 = _both(d, h0, n, bl, ids, tl, dl, temp, seed, 2 * seed)
            say(f"  n_seqs={n} block_len={bl}: tau {t2.tolist()}")
            assert torch.equal(t1, t2) and torch.equal(b1, b2), (n, bl, t1, t2, b1, b2)
            assert ((t2 >= 1) & (t2 <= bl)).all()
    finally:
        B.dflash_destroy(h0)
        d.close()


def test_noalloc_verify_rejects_oversized_calls():
    # more verification rows than the fixed scratch holds: an error, nothing launched
    dc = CONFIGS[0]
    d, w = make(dc, max_seqs=1)
    h0, keep = _bare_handle(dc, w)
    try:
        ids = torch.zeros(65, dc.block_size, dtype=torch.int32, device=DEV)
        tl = torch.zeros(65, dc.block_size, dc.vocab, device=DEV)
        tau = torch.zeros(65, dtype=torch.int32, device=DEV)
        with pytest.raises(B.DflashError):
            B.dflash_verify_noalloc(h0, 65, dc.block_size, ids.data_ptr(), tl.data_ptr(), 0, 0.0, 0, 0,
                                    tau.data_ptr(), tau.data_ptr())
    finally:
        B.dflash_destroy(h0)
        d.close()
