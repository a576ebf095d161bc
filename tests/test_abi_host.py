"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before anything reaches the device.

No call here launches GPU work: every checked path returns during host-side
validation (weights are fake, never dereferenced, aligned addresses)."""
import ctypes as C
import os
import re

import pytest

import oracle as O
from block_diffusion_drafter_layer_amd import binding as B
from block_diffusion_drafter_layer_amd.drafter import config_from
from synth import CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dflash.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 14
    lib = C.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(8):
        assert B.dflash_status_str(s) and B.dflash_status_str(s) != "unknown status"


def _cfg(i=1, **kw):
    c = config_from(CONFIGS[i])
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_kv_and_workspace_sizes():
    c = _cfg(1)
    cap = B.dflash_kv_row_capacity(c, 2048)
    assert cap >= 2048 + 16 and cap % 64 == 0
    assert B.dflash_kv_bytes(c, 2048) == 5 * 2 * 8 * cap * 128 * 2
    assert B.dflash_workspace_bytes(c, 1, 2048) > 0
    assert B.dflash_workspace_bytes(c, 2, 2048) > B.dflash_workspace_bytes(c, 1, 2048)
    bad = _cfg(1, mask_token_id=-1)
    assert B.dflash_kv_bytes(bad, 2048) == 0 and B.dflash_workspace_bytes(bad, 1, 16) == 0


def test_target_layer_ids_helper_matches_rule():
    for n in (16, 28, 36, 48, 64):
        assert B.dflash_target_layer_ids(n, 5) == O.target_layer_ids(n, 5)
    assert B.dflash_target_layer_ids(36, 1) == [18]
    with pytest.raises(B.DflashError):
        B.dflash_target_layer_ids(6, 5)


FAKE = 1 << 20  # an aligned address that is never dereferenced


def _weights(n_layers, null=None, misalign=None):
    layers = (B.dflash_layer_weights * n_layers)()
    for i in range(n_layers):
        for f, _ in B.dflash_layer_weights._fields_:
            setattr(layers[i], f, FAKE)
    w = B.dflash_weights(FAKE, FAKE, FAKE, FAKE, FAKE, C.cast(layers, C.POINTER(B.dflash_layer_weights)))
    if null:
        setattr(w, null, None)
    if misalign:
        setattr(w, misalign, FAKE + 2)
    return w, layers


def test_create_rejects_bad_configs_and_weights():
    c = _cfg(1)
    w, keep = _weights(c.n_layers)
    for field, val in [("mask_token_id", -1), ("mask_token_id", c.vocab), ("head_dim", 96),
                       ("hidden", 100), ("n_kv_heads", 5), ("block_size", 17), ("ffn", 100)]:
        bad = _cfg(1, **{field: val})
        with pytest.raises(B.DflashError) as e:
            B.dflash_create(bad, w)
        assert e.value.status == 2, field
    wn, k2 = _weights(c.n_layers, null="lm_head")
    with pytest.raises(B.DflashError) as e:
        B.dflash_create(c, wn)
    assert e.value.status == 1
    wa, k3 = _weights(c.n_layers, misalign="embed")
    with pytest.raises(B.DflashError) as e:
        B.dflash_create(c, wa)
    assert e.value.status == 5


def _handle(i=1):
    c = _cfg(i)
    w, keep = _weights(c.n_layers)
    h = B.dflash_create(c, w)
    return c, h, (w, keep)


def _status(fn, *a):
    try:
        fn(*a)
        return 0
    except B.DflashError as e:
        return e.status


def test_calls_before_workspace_and_workspace_checks():
    c, h, keep = _handle()
    kv = B.dflash_kv(FAKE, 2048, 100)
    assert _status(B.dflash_draft_block, h, [kv], FAKE, 16, FAKE) == 7
    assert _status(B.dflash_fuse_context, h, [FAKE] * 5, c.hidden, 10, FAKE) == 7
    assert _status(B.dflash_sample_draft, h, 1, 16, FAKE, 1.0, 0, 0, FAKE) == 7
    need = B.dflash_workspace_bytes(c, 2, 64)
    assert _status(B.dflash_set_workspace, h, FAKE, need - 1, 2, 64) == 4
    assert _status(B.dflash_set_workspace, h, FAKE + 16, need, 2, 64) == 5
    assert _status(B.dflash_set_workspace, h, FAKE, need, 0, 64) == 3
    assert _status(B.dflash_set_workspace, h, FAKE, need, 2, 64) == 0
    B.dflash_destroy(h)


def test_argument_errors_leave_cache_lengths_unchanged():
    c, h, keep = _handle()
    B.dflash_set_workspace(h, FAKE, B.dflash_workspace_bytes(c, 2, 64), 2, 64)
    kv = B.dflash_kv(FAKE, 256, 100)
    # draft_block
    assert _status(B.dflash_draft_block, h, [], FAKE, 16, FAKE) == 3
    assert _status(B.dflash_draft_block, h, [kv, kv, kv], FAKE, 16, FAKE) == 3
    assert _status(B.dflash_draft_block, h, [kv], FAKE, 17, FAKE) == 3
    assert _status(B.dflash_draft_block, h, [kv], FAKE, 0, FAKE) == 3
    assert _status(B.dflash_draft_block, h, [B.dflash_kv(FAKE, 50, 51)], FAKE, 16, FAKE) == 3
    assert _status(B.dflash_draft_block, h, [B.dflash_kv(None, 50, 5)], FAKE, 16, FAKE) == 1
    assert _status(B.dflash_draft_block, h, [B.dflash_kv(FAKE + 64, 50, 5)], FAKE, 16, FAKE) == 5
    # inject: pos0 beyond len, capacity, too many tokens, bad pointers
    assert _status(B.dflash_inject_kv, h, kv, FAKE, 10, 101) == 3
    assert _status(B.dflash_inject_kv, h, B.dflash_kv(FAKE, 120, 100), FAKE, 64, 100) == 4
    assert _status(B.dflash_inject_kv, h, kv, FAKE, 65, 0) == 3
    assert _status(B.dflash_inject_kv, h, kv, FAKE + 2, 4, 0) == 5
    assert _status(B.dflash_inject_kv, h, kv, FAKE, 0, 0) == 3
    assert kv.len == 100
    # fuse: n_tokens and ld
    assert _status(B.dflash_fuse_context, h, [FAKE] * 5, c.hidden, 65, FAKE) == 3
    assert _status(B.dflash_fuse_context, h, [FAKE] * 5, c.hidden - 8, 10, FAKE) == 5
    assert _status(B.dflash_fuse_context, h, [FAKE] * 4 + [0], c.hidden, 10, FAKE) == 1
    # verify
    assert _status(B.dflash_verify, h, 1, 16, FAKE, FAKE, 0, -1.0, 0, 0, FAKE, FAKE) == 3
    assert _status(B.dflash_verify, h, 1, 16, FAKE, FAKE, FAKE, 0.0, 0, 0, FAKE, FAKE) == 3
    assert _status(B.dflash_verify, h, 1, 16, FAKE, FAKE, 0, 1.0, 0, 0, FAKE, FAKE) == 1
    assert _status(B.dflash_verify, h, 3, 16, FAKE, FAKE, 0, 0.0, 0, 0, FAKE, FAKE) == 3
    assert _status(B.dflash_verify, h, 1, 16, FAKE, FAKE + 4, 0, 0.0, 0, 0, FAKE, FAKE) == 5
    # sample_draft: temperature, shapes, pointers; block_len 1 draws nothing
    assert _status(B.dflash_sample_draft, h, 1, 16, FAKE, 0.0, 0, 0, FAKE) == 3
    assert _status(B.dflash_sample_draft, h, 1, 16, FAKE, float("nan"), 0, 0, FAKE) == 3
    assert _status(B.dflash_sample_draft, h, 3, 16, FAKE, 1.0, 0, 0, FAKE) == 3
    assert _status(B.dflash_sample_draft, h, 1, 17, FAKE, 1.0, 0, 0, FAKE) == 3
    assert _status(B.dflash_sample_draft, h, 1, 16, 0, 1.0, 0, 0, FAKE) == 1
    assert _status(B.dflash_sample_draft, h, 1, 16, FAKE, 1.0, 0, 0, 0) == 1
    assert _status(B.dflash_sample_draft, h, 1, 1, FAKE, 1.0, 0, 0, FAKE) == 0
    # candidate selector: state, tables, shapes, pointers
    sel = B.dflash_selector(FAKE, FAKE, FAKE, 256, 16)
    assert _status(B.dflash_select_block, h, 1, 16, FAKE, FAKE, FAKE, 0.0, 0, 0, FAKE) == 7
    assert _status(B.dflash_set_selector, h, B.dflash_selector(FAKE, FAKE, FAKE, 256, 17)) == 3
    assert _status(B.dflash_set_selector, h, B.dflash_selector(FAKE, FAKE, FAKE, 96, 16)) == 3
    assert _status(B.dflash_set_selector, h, B.dflash_selector(FAKE, FAKE, FAKE, 320, 16)) == 3
    assert _status(B.dflash_set_selector, h, B.dflash_selector(FAKE, 0, FAKE, 256, 16)) == 1
    assert _status(B.dflash_set_selector, h, B.dflash_selector(FAKE, FAKE + 8, FAKE, 256, 16)) == 5
    assert _status(B.dflash_set_selector, h, sel) == 0
    assert _status(B.dflash_select_block, h, 3, 16, FAKE, FAKE, FAKE, 0.0, 0, 0, FAKE) == 3
    assert _status(B.dflash_select_block, h, 1, 17, FAKE, FAKE, FAKE, 0.0, 0, 0, FAKE) == 3
    assert _status(B.dflash_select_block, h, 1, 16, FAKE, FAKE, FAKE, -1.0, 0, 0, FAKE) == 3
    assert _status(B.dflash_select_block, h, 1, 16, FAKE, FAKE, FAKE, float("inf"), 0, 0, FAKE) == 3
    assert _status(B.dflash_select_block, h, 1, 16, 0, FAKE, FAKE, 0.0, 0, 0, FAKE) == 1
    assert _status(B.dflash_select_block, h, 1, 16, FAKE + 4, FAKE, FAKE, 0.0, 0, 0, FAKE) == 5
    assert _status(B.dflash_select_block, h, 1, 16, FAKE, FAKE, FAKE, 0.0, 0, 0, FAKE, FAKE + 2) == 5
    assert _status(B.dflash_select_block, h, 1, 1, FAKE, FAKE, FAKE, 0.0, 0, 0, FAKE) == 0
    # candidate-set p/q verify
    assert _status(B.dflash_verify_candidates, h, 1, 16, FAKE, FAKE, FAKE, FAKE, 16, 0.0, 0, 0, FAKE, FAKE) == 3
    assert _status(B.dflash_verify_candidates, h, 1, 16, FAKE, FAKE, FAKE, FAKE, 17, 1.0, 0, 0, FAKE, FAKE) == 3
    assert _status(B.dflash_verify_candidates, h, 1, 16, FAKE, FAKE, 0, FAKE, 16, 1.0, 0, 0, FAKE, FAKE) == 1
    assert _status(B.dflash_verify_candidates, h, 3, 16, FAKE, FAKE, FAKE, FAKE, 16, 1.0, 0, 0, FAKE, FAKE) == 3
    assert _status(B.dflash_verify_candidates, h, 1, 16, FAKE, FAKE, FAKE + 2, FAKE, 16, 1.0, 0, 0, FAKE, FAKE) == 5
    assert _status(B.dflash_set_selector, h, None) == 0
    assert _status(B.dflash_select_block, h, 1, 16, FAKE, FAKE, FAKE, 0.0, 0, 0, FAKE) == 7
    # dynamic conv: pointers, shapes, group size, alignment, overlap
    n_y = 16 * c.hidden * 4
    Y, CR = FAKE + (1 << 24), FAKE + (1 << 23)
    assert _status(B.dflash_conv_prepare, h, 1, 16, 16, FAKE, 0, FAKE, FAKE, Y, CR) == 1
    assert _status(B.dflash_conv_prepare, h, 1, 16, 16, 0, FAKE, FAKE, FAKE, Y, CR) == 1
    assert _status(B.dflash_conv_prepare, h, 3, 16, 16, FAKE, FAKE, FAKE, FAKE, Y, CR) == 3
    assert _status(B.dflash_conv_prepare, h, 1, 17, 16, FAKE, FAKE, FAKE, FAKE, Y, CR) == 3
    assert _status(B.dflash_conv_prepare, h, 1, 16, 0, FAKE, FAKE, FAKE, FAKE, Y, CR) == 3
    assert _status(B.dflash_conv_prepare, h, 1, 16, c.hidden, FAKE, FAKE, FAKE, FAKE, Y, CR) == 3
    assert _status(B.dflash_conv_prepare, h, 1, 16, 16, FAKE, FAKE + 8, FAKE, FAKE, Y, CR) == 5
    assert _status(B.dflash_conv_prepare, h, 1, 16, 16, FAKE, FAKE, FAKE + 4, FAKE, Y, CR) == 5
    assert _status(B.dflash_conv_prepare, h, 1, 16, 16, FAKE, FAKE, FAKE, FAKE, FAKE + n_y // 2, CR) == 3
    assert _status(B.dflash_conv_finish, h, 1, 16, 16, FAKE, FAKE, FAKE, 0, Y) == 1
    assert _status(B.dflash_conv_finish, h, 1, 16, 16, FAKE, FAKE, FAKE, CR, FAKE) == 3
    assert _status(B.dflash_conv_finish, h, 1, 0, 16, FAKE, FAKE, FAKE, CR, Y) == 3
    assert _status(B.dflash_conv_prepare, h, 1, 16, 16, FAKE, FAKE, FAKE, FAKE, Y, FAKE) == 3  # corr over x
    # device-resident rounds: pointers, shapes, alignment
    assert _status(B.dflash_draft_block_dev, h, [kv], 0, FAKE, 16, FAKE) == 1
    assert _status(B.dflash_draft_block_dev, h, [kv], FAKE + 2, FAKE, 16, FAKE) == 5
    assert _status(B.dflash_draft_block_dev, h, [kv], FAKE, FAKE, 17, FAKE) == 3
    assert _status(B.dflash_append_dev, h, [kv], FAKE, FAKE, [FAKE] * 5, c.hidden, 17) == 3
    assert _status(B.dflash_append_dev, h, [kv], FAKE, FAKE, [FAKE] * 5, c.hidden, 0) == 3
    assert _status(B.dflash_append_dev, h, [kv], 0, FAKE, [FAKE] * 5, c.hidden, 16) == 1
    assert _status(B.dflash_append_dev, h, [kv], FAKE, FAKE, [FAKE] * 4 + [0], c.hidden, 16) == 1
    assert _status(B.dflash_append_dev, h, [kv], FAKE, FAKE, [FAKE] * 5, c.hidden - 8, 16) == 5
    assert _status(B.dflash_append_dev, h, [kv, kv, kv], FAKE, FAKE, [FAKE] * 5, c.hidden, 16) == 3
    assert _status(B.dflash_kv_trim_dev, h, 0, FAKE, 5) == 3
    assert _status(B.dflash_kv_trim_dev, h, 1, FAKE, -1) == 3
    assert _status(B.dflash_kv_trim_dev, h, 1, 0, 5) == 1
    assert kv.len == 100
    # trim is host metadata only
    assert _status(B.dflash_kv_trim, h, kv, 101) == 3
    assert kv.len == 100
    assert _status(B.dflash_kv_trim, h, kv, 37) == 0
    assert kv.len == 37
    B.dflash_destroy(h)


def test_stage_names_are_the_documented_ones():
    assert tuple(B._lib.dflash_stage_name(i).decode() for i in range(len(B.STAGES))) == B.STAGES
    assert B._lib.dflash_stage_name(len(B.STAGES)).decode() == "unknown"
    assert B._lib.dflash_stage_name(-1).decode() == "unknown"


def test_reference_copy_argument_checks():
    # every case returns during host-side validation: no GPU work
    # (status codes: 1 = DFLASH_E_NULL, 5 = DFLASH_E_ALIGN)
    assert B._lib.dflash_copy_bytes(None, None, 0, None) == B.DFLASH_OK
    assert B._lib.dflash_copy_bytes(None, C.c_void_p(256), 64, None) == 1
    assert B._lib.dflash_copy_bytes(C.c_void_p(256), None, 64, None) == 1
    assert B._lib.dflash_copy_bytes(C.c_void_p(264), C.c_void_p(256), 64, None) == 5
    assert B._lib.dflash_copy_bytes(C.c_void_p(256), C.c_void_p(512), 72, None) == 5
