"""ctypes binding of libdflash.so: the C ABI of include/dflash.h, same names.

Argument marshalling only. Device buffers are passed as integer addresses
(``tensor.data_ptr()``); torch supplies the memory and the stream, every step
of the path runs in the library's HIP kernels. Importing this module loads the
library and raises if it has not been built.
"""
import ctypes as C
import os
from typing import Dict, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdflash.so")

DFLASH_OK = 0
STATUS_NAMES = {0: "DFLASH_OK", 1: "DFLASH_E_NULL", 2: "DFLASH_E_CONFIG",
                3: "DFLASH_E_SHAPE", 4: "DFLASH_E_CAPACITY", 5: "DFLASH_E_ALIGN",
                6: "DFLASH_E_DEVICE", 7: "DFLASH_E_STATE"}


class dflash_config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_feat_layers", C.c_int32),
                ("n_layers", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("block_size", C.c_int32), ("mask_token_id", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class dflash_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down",
                 "attn_norm", "mlp_norm")]


class dflash_weights(C.Structure):
    _fields_ = [("w_c", C.c_void_p), ("ctx_norm", C.c_void_p),
                ("embed", C.c_void_p), ("lm_head", C.c_void_p),
                ("final_norm", C.c_void_p),
                ("layers", C.POINTER(dflash_layer_weights))]


class dflash_selector(C.Structure):
    _fields_ = [("hidden_proj", C.c_void_p), ("pred_codebook", C.c_void_p),
                ("succ_codebook", C.c_void_p), ("rank", C.c_int32), ("top_k", C.c_int32)]


class dflash_conv_layer(C.Structure):
    _fields_ = [("attn_base", C.c_void_p), ("attn_proj", C.c_void_p), ("mlp_base", C.c_void_p),
                ("mlp_proj", C.c_void_p)]


class dflash_kv(C.Structure):
    _fields_ = [("base", C.c_void_p), ("max_ctx", C.c_int32), ("len", C.c_int32)]


class DflashError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


def _hip_runtimes():
    """Paths of every libamdhip64 mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_diffusion_drafter_layer_amd.build`")
    # torch ships its own HIP/HSA runtime. Load it first so that libdflash's
    # libamdhip64.so.7 dependency binds to that same runtime: two HSA runtimes
    # in one process do not share devices, memory or streams.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError(f"more than one HIP runtime is loaded ({rts}); import torch "
                          "before anything that loads the system libamdhip64")
    P, I32, I64, U64, F32, SZ = (C.c_void_p, C.c_int32, C.c_int64, C.c_uint64,
                                 C.c_float, C.c_size_t)
    cfgp = C.POINTER(dflash_config)
    kvp = C.POINTER(dflash_kv)
    sig = {
        "dflash_kv_bytes": (SZ, [cfgp, I32]),
        "dflash_kv_row_capacity": (I32, [cfgp, I32]),
        "dflash_workspace_bytes": (SZ, [cfgp, I32, I32]),
        "dflash_create": (C.c_int, [cfgp, C.POINTER(dflash_weights), P, C.POINTER(P)]),
        "dflash_destroy": (C.c_int, [P]),
        "dflash_set_stream": (C.c_int, [P, P]),
        "dflash_set_workspace": (C.c_int, [P, P, SZ, I32, I32]),
        "dflash_fuse_context": (C.c_int, [P, C.POINTER(P), I64, I32, P]),
        "dflash_inject_kv": (C.c_int, [P, kvp, P, I32, I32]),
        "dflash_kv_trim": (C.c_int, [P, kvp, I32]),
        "dflash_draft_block": (C.c_int, [P, I32, C.POINTER(kvp), P, I32, P, P, P]),
        "dflash_verify": (C.c_int, [P, I32, I32, P, P, P, F32, U64, U64, P, P]),
        "dflash_verify_noalloc": (C.c_int, [P, I32, I32, P, P, P, F32, U64, U64, P, P]),
        "dflash_sample_draft": (C.c_int, [P, I32, I32, P, F32, U64, U64, P]),
        "dflash_verify_candidates": (C.c_int, [P, I32, I32, P, P, P, P, I32, F32, U64, U64, P, P]),
        "dflash_set_selector": (C.c_int, [P, C.POINTER(dflash_selector)]),
        "dflash_set_conv": (C.c_int, [P, C.POINTER(dflash_conv_layer), I32]),
        "dflash_select_block": (C.c_int, [P, I32, I32, P, P, P, F32, U64, U64, P, P, P]),
        "dflash_conv_prepare": (C.c_int, [P, I32, I32, I32, P, P, P, P, P, P]),
        "dflash_conv_finish": (C.c_int, [P, I32, I32, I32, P, P, P, P, P]),
        "dflash_draft_block_dev": (C.c_int, [P, I32, C.POINTER(kvp), P, P, I32, P, P, P]),
        "dflash_append_dev": (C.c_int, [P, I32, C.POINTER(kvp), P, P, C.POINTER(P), I64, I32]),
        "dflash_kv_trim_dev": (C.c_int, [P, I32, P, I32]),
        "dflash_target_layer_ids": (C.c_int, [I32, I32, C.POINTER(I32)]),
        "dflash_profile_enable": (C.c_int, [P, C.c_uint32, I32]),
        "dflash_profile_read": (C.c_int, [P, I32, C.POINTER(I32), C.POINTER(F32), C.POINTER(I32)]),
        "dflash_stage_name": (C.c_char_p, [I32]),
        "dflash_copy_bytes": (C.c_int, [P, P, SZ, P]),
        "dflash_read_bytes": (C.c_int, [P, SZ, P, P]),
        "dflash_status_str": (C.c_char_p, [C.c_int]),
        "dflash_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = tuple(sorted(n for n in dir(_lib) if n.startswith("dflash_")))


def _check(status: int):
    if status != DFLASH_OK:
        raise DflashError(status, _lib.dflash_last_error().decode())
    return status


# --- the ABI, same names -----------------------------------------------------

def dflash_kv_bytes(cfg: dflash_config, max_ctx: int) -> int:
    return _lib.dflash_kv_bytes(C.byref(cfg), max_ctx)


def dflash_kv_row_capacity(cfg: dflash_config, max_ctx: int) -> int:
    return _lib.dflash_kv_row_capacity(C.byref(cfg), max_ctx)


def dflash_workspace_bytes(cfg: dflash_config, max_seqs: int, max_tokens: int) -> int:
    return _lib.dflash_workspace_bytes(C.byref(cfg), max_seqs, max_tokens)


def dflash_create(cfg: dflash_config, weights: dflash_weights, stream: int = 0):
    h = C.c_void_p()
    _check(_lib.dflash_create(C.byref(cfg), C.byref(weights), C.c_void_p(stream), C.byref(h)))
    return h


def dflash_destroy(h):
    return _check(_lib.dflash_destroy(h))


def dflash_set_stream(h, stream: int):
    return _check(_lib.dflash_set_stream(h, C.c_void_p(stream)))


def dflash_set_workspace(h, ws: int, nbytes: int, max_seqs: int, max_tokens: int):
    return _check(_lib.dflash_set_workspace(h, C.c_void_p(ws), nbytes, max_seqs, max_tokens))


def dflash_fuse_context(h, feats: Sequence[int], ld: int, n_tokens: int, ctx_out: int):
    arr = (C.c_void_p * len(feats))(*feats)
    return _check(_lib.dflash_fuse_context(h, arr, ld, n_tokens, C.c_void_p(ctx_out)))


def dflash_inject_kv(h, kv: dflash_kv, ctx_feat: int, n_tokens: int, pos0: int):
    return _check(_lib.dflash_inject_kv(h, C.byref(kv), C.c_void_p(ctx_feat), n_tokens, pos0))


def dflash_kv_trim(h, kv: dflash_kv, keep_len: int):
    return _check(_lib.dflash_kv_trim(h, C.byref(kv), keep_len))


def dflash_draft_block(h, kvs: Sequence[dflash_kv], anchor_ids: int, block_len: int,
                       block_out: int, hidden_out: int = 0, logits_out: int = 0):
    arr = (C.POINTER(dflash_kv) * len(kvs))(*[C.pointer(k) for k in kvs])
    return _check(_lib.dflash_draft_block(h, len(kvs), arr, C.c_void_p(anchor_ids), block_len,
                                          C.c_void_p(block_out), C.c_void_p(hidden_out or None),
                                          C.c_void_p(logits_out or None)))


def dflash_verify(h, n_seqs: int, block_len: int, block_ids: int, target_logits: int,
                  draft_logits: int, temperature: float, seed: int, philox_offset: int,
                  tau_out: int, bonus_out: int):
    return _check(_lib.dflash_verify(h, n_seqs, block_len, C.c_void_p(block_ids),
                                     C.c_void_p(target_logits), C.c_void_p(draft_logits or None),
                                     float(temperature), seed, philox_offset,
                                     C.c_void_p(tau_out), C.c_void_p(bonus_out)))


def dflash_verify_noalloc(h, n_seqs: int, block_len: int, block_ids: int, target_logits: int,
                          draft_logits: int, temperature: float, seed: int, philox_offset: int,
                          tau_out: int, bonus_out: int):
    return _check(_lib.dflash_verify_noalloc(h, n_seqs, block_len, C.c_void_p(block_ids),
                                             C.c_void_p(target_logits),
                                             C.c_void_p(draft_logits or None), float(temperature),
                                             seed, philox_offset, C.c_void_p(tau_out),
                                             C.c_void_p(bonus_out)))


def dflash_draft_block_dev(h, kvs: Sequence[dflash_kv], len_dev: int, anchor_ids: int,
                           block_len: int, block_out: int, hidden_out: int = 0, logits_out: int = 0):
    arr = (C.POINTER(dflash_kv) * len(kvs))(*[C.pointer(k) for k in kvs])
    return _check(_lib.dflash_draft_block_dev(h, len(kvs), arr, C.c_void_p(len_dev),
                                              C.c_void_p(anchor_ids), block_len,
                                              C.c_void_p(block_out), C.c_void_p(hidden_out or None),
                                              C.c_void_p(logits_out or None)))


def dflash_append_dev(h, kvs: Sequence[dflash_kv], len_dev: int, tau_dev: int,
                      feats: Sequence[int], ld: int, rows_per_seq: int):
    arr = (C.POINTER(dflash_kv) * len(kvs))(*[C.pointer(k) for k in kvs])
    fa = (C.c_void_p * len(feats))(*feats)
    return _check(_lib.dflash_append_dev(h, len(kvs), arr, C.c_void_p(len_dev), C.c_void_p(tau_dev),
                                         fa, ld, rows_per_seq))


def dflash_kv_trim_dev(h, n_seqs: int, len_dev: int, keep_len: int):
    return _check(_lib.dflash_kv_trim_dev(h, n_seqs, C.c_void_p(len_dev), keep_len))


def dflash_sample_draft(h, n_seqs: int, block_len: int, draft_logits: int, temperature: float,
                        seed: int, philox_offset: int, block_ids: int):
    return _check(_lib.dflash_sample_draft(h, n_seqs, block_len, C.c_void_p(draft_logits),
                                           float(temperature), seed, philox_offset,
                                           C.c_void_p(block_ids)))


def dflash_set_selector(h, sel):
    """sel: a dflash_selector, or None to remove the selector."""
    return _check(_lib.dflash_set_selector(h, C.byref(sel) if sel is not None else None))


def dflash_set_conv(h, layers, group_size: int):
    """layers: a sequence of dflash_conv_layer (one per draft layer), or None
    to remove the convs."""
    if layers is None:
        return _check(_lib.dflash_set_conv(h, None, 0))
    arr = (dflash_conv_layer * len(layers))(*layers)
    return _check(_lib.dflash_set_conv(h, arr, group_size))


def dflash_select_block(h, n_seqs: int, block_len: int, last_hidden: int, draft_logits: int,
                        anchor_ids: int, temperature: float, seed: int, philox_offset: int,
                        block_ids: int, cand_out: int = 0, q_out: int = 0):
    return _check(_lib.dflash_select_block(h, n_seqs, block_len, C.c_void_p(last_hidden),
                                           C.c_void_p(draft_logits), C.c_void_p(anchor_ids),
                                           float(temperature), seed, philox_offset,
                                           C.c_void_p(block_ids), C.c_void_p(cand_out or None),
                                           C.c_void_p(q_out or None)))


def dflash_verify_candidates(h, n_seqs: int, block_len: int, block_ids: int, target_logits: int,
                             cand: int, q_rows: int, top_k: int, temperature: float, seed: int,
                             philox_offset: int, tau_out: int, bonus_out: int):
    return _check(_lib.dflash_verify_candidates(h, n_seqs, block_len, C.c_void_p(block_ids),
                                                C.c_void_p(target_logits), C.c_void_p(cand),
                                                C.c_void_p(q_rows), top_k, float(temperature),
                                                seed, philox_offset, C.c_void_p(tau_out),
                                                C.c_void_p(bonus_out)))


def dflash_conv_prepare(h, n_seqs: int, block_len: int, group_size: int, base: int, proj: int,
                        x: int, prev: int, y: int, corr_out: int):
    return _check(_lib.dflash_conv_prepare(h, n_seqs, block_len, group_size, C.c_void_p(base),
                                           C.c_void_p(proj), C.c_void_p(x), C.c_void_p(prev),
                                           C.c_void_p(y), C.c_void_p(corr_out)))


def dflash_conv_finish(h, n_seqs: int, block_len: int, group_size: int, base: int, z: int,
                       prev: int, corr: int, y: int):
    return _check(_lib.dflash_conv_finish(h, n_seqs, block_len, group_size, C.c_void_p(base),
                                          C.c_void_p(z), C.c_void_p(prev), C.c_void_p(corr),
                                          C.c_void_p(y)))


def dflash_target_layer_ids(n_target_layers: int, n_feat: int):
    out = (C.c_int32 * n_feat)()
    _check(_lib.dflash_target_layer_ids(n_target_layers, n_feat, out))
    return list(out)


STAGES = ("embed", "qkv", "attention", "o_proj", "gate_up", "down_proj", "lm_head",
          "fuse_context", "inject_kv", "verify", "lm_argmax", "sample_draft", "select",
          "conv")


def dflash_copy_bytes(dst: int, src: int, nbytes: int, stream: int = 0):
    return _check(_lib.dflash_copy_bytes(C.c_void_p(dst), C.c_void_p(src), nbytes, C.c_void_p(stream)))


def dflash_read_bytes(src: int, nbytes: int, sink: int, stream: int = 0):
    return _check(_lib.dflash_read_bytes(C.c_void_p(src), nbytes, C.c_void_p(sink), C.c_void_p(stream)))


def dflash_profile_enable(h, stage_mask: int, max_records: int = 0):
    return _check(_lib.dflash_profile_enable(h, stage_mask, max_records))


def dflash_profile_read(h, cap: int):
    """[(stage_name, ms), ...] of the launches recorded since enabling."""
    st = (C.c_int32 * max(cap, 1))()
    ms = (C.c_float * max(cap, 1))()
    n = C.c_int32()
    _check(_lib.dflash_profile_read(h, cap, st, ms, C.byref(n)))
    return [(dflash_stage_name(st[i]), ms[i]) for i in range(n.value)]


def dflash_stage_name(stage: int) -> str:
    return _lib.dflash_stage_name(stage).decode()


def dflash_status_str(status: int) -> str:
    return _lib.dflash_status_str(status).decode()


def dflash_last_error() -> str:
    return _lib.dflash_last_error().decode()


# --- marshalling helpers ------------------------------------------------------

def make_config(hidden, n_feat_layers, n_layers, n_heads, n_kv_heads, head_dim, ffn,
                vocab, block_size, mask_token_id, rms_eps=1e-6, rope_theta=1e6) -> dflash_config:
    return dflash_config(hidden, n_feat_layers, n_layers, n_heads, n_kv_heads, head_dim,
                         ffn, vocab, block_size, mask_token_id, rms_eps, rope_theta)


class Weights:
    """dflash_weights built from a dict of device tensors (keeps them alive)."""

    def __init__(self, w: Dict):
        self._keep = w
        n = len(w["layers"])
        self._layers = (dflash_layer_weights * n)()
        for i, lw in enumerate(w["layers"]):
            for f, _ in dflash_layer_weights._fields_:
                setattr(self._layers[i], f, lw[f].data_ptr())
        self.struct = dflash_weights(
            w["w_c"].data_ptr(), w["ctx_norm"].data_ptr(), w["embed"].data_ptr(),
            w["lm_head"].data_ptr(), w["final_norm"].data_ptr(),
            C.cast(self._layers, C.POINTER(dflash_layer_weights)))
