"""Plain CPU oracle of the DFlash drafter hot path (numpy, fp64).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module. The GPU library never calls it and
shares no code with it.

Sources (the four web pages on DFlash):
  [Tut]  A3-dflash tutorial (CCODING04 llm-paper-tutorials)
  [Sum]  papercache summary "DFlash: Block Diffusion for Flash Speculative Decoding"
  [Note] tom-jerr paper-reading notes "DFLASH"
  [Code] txtmix code-reading article on the z-lab dflash repository

Every function below is the plain definition of one step, written in fp64
with numpy; matrix products use numpy's matmul as a library step. Inputs that
are stored in bf16 on the GPU arrive here as float arrays holding the same
bf16 values.

Readings taken where the pages are silent (also listed in the design notes):
  * decoder layer = pre-norm RMSNorm -> attention -> residual, RMSNorm ->
    SwiGLU -> residual; final RMSNorm before the LM head; no biases; no QK norm;
  * RoPE is rotate-half over pairs (d, d + hd/2), inv_freq_d = theta^(-2d/hd);
  * GQA: query head a reads kv head a // (Hq/Hkv);
  * argmax ties go to the lowest index (numpy.argmax / torch.argmax rule);
  * Philox4x64-10 counter layout and the inverse-CDF sampler of verify_pq;
  * a cache built with bf16_kv=True stores its context K/V rows rounded to
    bf16 ([Code] section 5 sizes the model's weights and activations at two
    bytes each, BF16); with bf16_kv=False (the default, the plain definition)
    every row is kept in fp64. The block's own K/V rows are never stored in
    the cache ([Code] section 5 concatenates them with the context's inside
    the attention call; only the context rows persist across rounds), so they
    are never rounded.
  * candidate selector: the top-k order (value descending, then index
    ascending), no bias in the hidden projection, the walk's hidden state is
    the LM head's input (final RMSNorm applied), and sampling draws from
    softmax(scores / T) over the k candidates with Philox purpose 3.
  * grouped dynamic two-tap conv: the projection's 2*k*groups outputs are
    laid out (call, tap, group) row-major, call 0 = "prepare", call 1 =
    "finish"; both halves come from the hidden state the prepare call reads
    (its own input), and the finish half is handed to the finish call; the
    conv output replaces its input (no residual inside the module); the
    block's first position reads a caller-given row standing for the last
    confirmed token. Where the two calls sit in the layer is left to the
    caller.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def target_layer_ids(n_target_layers: int, n_feat: int) -> List[int]:
    """[Code] section 5 (build_target_layer_ids): n_feat ids spread evenly over
    the 0-based range 1 .. n_target_layers-3; the middle layer if n_feat == 1.
    Grid points are rounded to the nearest integer (halves up)."""
    if n_feat == 1:
        return [n_target_layers // 2]
    lo, hi = 1.0, float(n_target_layers - 3)
    step = (hi - lo) / (n_feat - 1)
    return [int(np.floor(lo + i * step + 0.5)) for i in range(n_feat)]


def round_bf16(x):
    """Round to the nearest bfloat16 value, ties to even (the top 16 bits of
    the IEEE binary32 pattern after adding 0x7FFF plus the lowest kept bit).
    Inputs are first rounded to binary32; finite values only."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(F64)


def rms_norm(x, gain, eps):
    """[Tut] section 2.1.1 (SimpleRMSNorm): x / sqrt(mean(x^2) + eps) * gain,
    eps inside the square root, gain applied after the division."""
    x = np.asarray(x, dtype=F64)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / rms * np.asarray(gain, dtype=F64)


def linear(x, w, chunk_rows: int = 16384):
    """y = x @ w.T for a weight in [out, in] layout (nn.Linear convention).

    The output columns are computed in slices of ``chunk_rows`` weight rows only
    to bound the fp64 temporary; each output is the same full dot product."""
    x = np.asarray(x, dtype=F64)
    n_out = w.shape[0]
    out = np.empty(x.shape[:-1] + (n_out,), dtype=F64)
    for r0 in range(0, n_out, chunk_rows):
        wc = np.asarray(w[r0:r0 + chunk_rows], dtype=F64)
        out[..., r0:r0 + chunk_rows] = x @ wc.T
    return out


def silu(x):
    return x / (1.0 + np.exp(-x))


def softmax(x, axis=-1):
    x = np.asarray(x, dtype=F64)
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


# ----------------------------------------------------------------------------
# Target-context fusion
# ----------------------------------------------------------------------------

def fuse_context(feats: Sequence, w_c, gain, eps: float = 1e-6):
    """H_t = RMSNorm(W_c [H^(l1); ...; H^(l5)]).

    [Tut] section 2.1.1 (concat of the sampled layers along the hidden axis,
    then the fc projection and RMSNorm) and section 2.1.2 (the H_t equation);
    [Code] section 5 (extract_context_feature, fc, hidden_norm).
    feats: n arrays [T, D] in increasing layer order; w_c: [D, n*D].
    """
    c = np.concatenate([np.asarray(f, dtype=F64) for f in feats], axis=-1)
    y = linear(c, w_c)
    return rms_norm(y, gain, eps)


# ----------------------------------------------------------------------------
# rotary position embedding
# ----------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, theta: float):
    d = np.arange(head_dim // 2, dtype=F64)
    return theta ** (-2.0 * d / head_dim)


def apply_rope(x, positions, theta: float):
    """Rotate-half RoPE on the last axis: for d < hd/2 the pair (x_d, x_{d+hd/2})
    is rotated by angle pos * theta^(-2d/hd). x: [T, H, hd]; positions: [T]."""
    x = np.asarray(x, dtype=F64)
    hd = x.shape[-1]
    half = hd // 2
    ang = np.asarray(positions, dtype=F64)[:, None] * rope_inv_freq(hd, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------
# KV injection into the draft cache, trim and append
# ----------------------------------------------------------------------------

def inject_kv(ctx_feat, wk, wv, pos0: int, n_kv_heads: int, head_dim: int,
              theta: float):
    """Per-layer K/V of the fused context: K = RoPE(W_K H_t), V = W_V H_t.

    [Tut] section 2.1.2 (the target feature enters only as K and V entries of
    every draft layer); [Code] section 5 (k_ctx = k_proj(target_hidden)).
    Context row t sits at absolute position pos0 + t.
    Returns K, V as [T, Hkv, hd].
    """
    T = ctx_feat.shape[0]
    k = linear(ctx_feat, wk).reshape(T, n_kv_heads, head_dim)
    v = linear(ctx_feat, wv).reshape(T, n_kv_heads, head_dim)
    k = apply_rope(k, np.arange(pos0, pos0 + T), theta)
    return k, v


@dataclass
class DraftCache:
    """One sequence's draft KV cache: per layer, the context rows' K and V.

    [Sum] section 4.1 and [Code] section 5: projected target features are kept
    in the draft model's KV cache and reused across drafting rounds; [Code]
    section 9: after verification the cache is cropped back to the accepted
    prefix. Rows at positions >= len are not part of the cache.

    bf16_kv: rows are rounded to bf16 when stored (see store()).
    """
    n_layers: int
    k: List[np.ndarray] = field(default_factory=list)
    v: List[np.ndarray] = field(default_factory=list)
    bf16_kv: bool = False

    def __post_init__(self):
        if not self.k:
            self.k = [None] * self.n_layers
            self.v = [None] * self.n_layers

    @property
    def len(self) -> int:
        return 0 if self.k[0] is None else int(self.k[0].shape[0])

    def trim(self, keep: int):
        if keep < 0 or keep > self.len:
            raise ValueError("trim beyond the cache length")
        for i in range(self.n_layers):
            if self.k[i] is not None:
                self.k[i] = self.k[i][:keep]
                self.v[i] = self.v[i][:keep]

    def store(self, x):
        """The value a row holds once written to this cache."""
        return round_bf16(x) if self.bf16_kv else np.asarray(x, F64)

    def append(self, layer: int, k, v, pos0: int):
        """Write rows at positions pos0.. after dropping everything >= pos0."""
        k, v = self.store(k), self.store(v)
        if self.k[layer] is None:
            if pos0 != 0:
                raise ValueError("first append must start at position 0")
            self.k[layer], self.v[layer] = np.asarray(k, F64), np.asarray(v, F64)
            return
        if pos0 > self.k[layer].shape[0]:
            raise ValueError("append past the cache length")
        self.k[layer] = np.concatenate([self.k[layer][:pos0], np.asarray(k, F64)])
        self.v[layer] = np.concatenate([self.v[layer][:pos0], np.asarray(v, F64)])


def cache_inject(cache: DraftCache, ctx_feat, layers_w, cfg, pos0: int):
    """Trim the cache to pos0 and append the K/V of ctx_feat in every layer."""
    for i, lw in enumerate(layers_w):
        k, v = inject_kv(ctx_feat, lw["wk"], lw["wv"], pos0, cfg.n_kv_heads,
                         cfg.head_dim, cfg.rope_theta)
        cache.append(i, k, v, pos0)


# ----------------------------------------------------------------------------
# Block attention
# ----------------------------------------------------------------------------

def block_attention(q, k, v):
    """o = softmax(q k^T / sqrt(hd)) v with no mask, grouped-query heads.

    q: [B, Hq, hd]; k, v: [S+B, Hkv, hd] = context rows then the block's own
    rows ([Code] section 5: torch.cat([k_ctx, k_noise], dim=1)). Every block
    position sees every key: the draft's full-attention layers are not causal
    ([Code] section 6). Query head a uses kv head a // (Hq/Hkv).
    """
    B, Hq, hd = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.empty((B, Hq, hd), dtype=F64)
    for a in range(Hq):
        g = a // G
        s = (np.asarray(q[:, a, :], F64) @ np.asarray(k[:, g, :], F64).T) / np.sqrt(hd)
        o[:, a, :] = softmax(s, axis=-1) @ np.asarray(v[:, g, :], F64)
    return o


# ----------------------------------------------------------------------------
# One draft forward over a block
# ----------------------------------------------------------------------------

def draft_block(cfg, weights: Dict, caches: Sequence[DraftCache],
                anchors: Sequence[int], block_len: Optional[int] = None,
                conv: Optional[Dict] = None):
    """One parallel forward of the drafter over [anchor, mask x (block_len-1)].

    [Code] section 6 (block = last confirmed token + block_size-1 mask tokens,
    one forward fills every masked position, no iterative denoising) and
    section 9 (positions continue from the context; the LM head is applied to
    the block rows after the anchor, argmax gives the draft tokens);
    [Tut] section 2.1.2 (Q from the draft only, K/V = [context ; block]);
    [Tut] section 2.2.3 / [Code] section 3 (embedding and LM head are the
    target's, shared and frozen).

    caches[s] holds sequence s's context K/V; its length S_s is the anchor's
    position. The block's own K/V rows exist only inside this forward and
    keep full precision.

    conv (optional): the DFlash 2 grouped dynamic two-tap convs of every
    layer ([Code] section 13: short-range in-block mixing that takes over
    from block attention; section 14: one instance by attention and one by
    the MLP, base_kernel[0] for the "prepare" call and base_kernel[1] for the
    "finish" call). {"group_size": g, "layers": [{"attn_base", "attn_proj",
    "mlp_base", "mlp_proj"} per layer]}. Reading of where the calls sit (the
    pages do not say): prepare on the sublayer's normed input, whose
    projection also yields the finish call's corrections, finish on the
    sublayer's output before the residual add; the module carries no state
    across steps, so the block's first row reads a zero row as its
    predecessor. Returns a dict with
      draft  [n_seq, block_len-1] int   argmax tokens of rows 1..block_len-1
      hidden [L, n_seq, block_len, D]   residual stream after each layer
      logits [n_seq, block_len-1, V]
      gap    [n_seq, block_len-1]       top-1 minus top-2 logit
    """
    B = cfg.block_size if block_len is None else block_len
    L, D = cfg.n_layers, cfg.hidden
    Hq, Hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    eps, theta = cfg.rms_eps, cfg.rope_theta
    n_seq = len(anchors)
    hidden = np.empty((L, n_seq, B, D), dtype=F64)
    out_draft = np.zeros((n_seq, max(B - 1, 0)), dtype=np.int64)
    out_logits = np.zeros((n_seq, max(B - 1, 0), cfg.vocab), dtype=F64)
    out_gap = np.zeros((n_seq, max(B - 1, 0)), dtype=F64)
    embed = weights["embed"]
    for s in range(n_seq):
        S = caches[s].len
        ids = [int(anchors[s])] + [cfg.mask_token_id] * (B - 1)
        x = np.asarray(embed[ids], dtype=F64)            # [B, D]
        pos = np.arange(S, S + B)
        zero = np.zeros((1, D), dtype=F64)
        for i, lw in enumerate(weights["layers"]):
            cw = conv["layers"][i] if conv is not None else None
            h = rms_norm(x, lw["attn_norm"], eps)
            if cw is not None:
                h, corr_a = dynamic_conv_prepare(h, zero, B, cw["attn_base"], cw["attn_proj"],
                                                 conv["group_size"])
            q = linear(h, lw["wq"]).reshape(B, Hq, hd)
            kb = linear(h, lw["wk"]).reshape(B, Hkv, hd)
            vb = linear(h, lw["wv"]).reshape(B, Hkv, hd)
            q = apply_rope(q, pos, theta)
            kb = apply_rope(kb, pos, theta)
            if S > 0:
                k_all = np.concatenate([caches[s].k[i], kb])
                v_all = np.concatenate([caches[s].v[i], vb])
            else:
                k_all, v_all = kb, vb
            o = block_attention(q, k_all, v_all).reshape(B, Hq * hd)
            a = linear(o, lw["wo"])
            if cw is not None:
                a = dynamic_conv_finish(a, zero, B, cw["attn_base"], corr_a, conv["group_size"])
            x = x + a
            h2 = rms_norm(x, lw["mlp_norm"], eps)
            if cw is not None:
                h2, corr_m = dynamic_conv_prepare(h2, zero, B, cw["mlp_base"], cw["mlp_proj"],
                                                  conv["group_size"])
            m = linear(silu(linear(h2, lw["w_gate"])) * linear(h2, lw["w_up"]), lw["w_down"])
            if cw is not None:
                m = dynamic_conv_finish(m, zero, B, cw["mlp_base"], corr_m, conv["group_size"])
            x = x + m
            hidden[i, s] = x
        if B > 1:
            z = rms_norm(x[1:], weights["final_norm"], eps)
            logits = linear(z, weights["lm_head"])
            out_logits[s] = logits
            out_draft[s] = np.argmax(logits, axis=-1)
            top2 = np.sort(logits, axis=-1)[:, -2:]
            out_gap[s] = top2[:, 1] - top2[:, 0]
    return {"draft": out_draft, "hidden": hidden, "logits": out_logits,
            "gap": out_gap}


# ----------------------------------------------------------------------------
# Greedy verification
# ----------------------------------------------------------------------------

def verify_greedy(block_ids, target_logits):
    """Longest matching prefix plus one bonus token.

    [Code] section 8: posterior = argmax(target logits); the acceptance length
    is the cumulative product of (block[1:] == posterior[:-1]) summed; the bonus
    is posterior[acceptance]. tau = acceptance + 1, in 1..len(block)
    ([Sum] section 3.1; [Code] section 4: tau counts the bonus token).
    block_ids: [B] ints (anchor then drafts); target_logits: [B, V].
    Returns (tau, bonus).
    """
    posterior = np.argmax(np.asarray(target_logits), axis=-1)
    match = np.asarray(block_ids)[1:] == posterior[:-1]
    accepted = int(np.cumprod(match.astype(np.int64)).sum())
    return accepted + 1, int(posterior[accepted])


# ----------------------------------------------------------------------------
# Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC 2011), written from the paper's round function
# ----------------------------------------------------------------------------

_M64 = (1 << 64) - 1
_PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
_PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox4x64_10(counter, key):
    """One Philox4x64 block with 10 rounds. counter: 4 words, key: 2 words."""
    x0, x1, x2, x3 = (int(c) & _M64 for c in counter)
    k0, k1 = (int(k) & _M64 for k in key)
    for _ in range(10):
        p0 = _PHILOX_M[0] * x0
        p1 = _PHILOX_M[1] * x2
        x0, x1, x2, x3 = (((p1 >> 64) ^ x1 ^ k0) & _M64, p1 & _M64,
                          ((p0 >> 64) ^ x3 ^ k1) & _M64, p0 & _M64)
        k0 = (k0 + _PHILOX_W[0]) & _M64
        k1 = (k1 + _PHILOX_W[1]) & _M64
    return x0, x1, x2, x3


PURPOSE_ACCEPT, PURPOSE_RESAMPLE, PURPOSE_DRAFT = 0, 1, 2


def philox_uniform(seed: int, row: int, seq: int, purpose: int) -> float:
    """u in [0, 1) from word 0 of block counter (row, seq, purpose, 0), key
    (seed, 0): u = (w >> 11) * 2^-53."""
    w = philox4x64_10((row, seq, purpose, 0), (seed, 0))[0]
    return (w >> 11) * (2.0 ** -53)


def sample_inverse_cdf(weights, u: float):
    """Smallest v with sum_{w <= v} weights[w] > u * sum(weights), running sums
    in vocab order in fp64. Returns (token, margin) where margin is the fp64
    distance of u*sum to the nearest of the two bracketing running sums."""
    r = np.asarray(weights, dtype=F64)
    c = np.cumsum(r)
    target = u * c[-1]
    v = int(np.searchsorted(c, target, side="right"))
    v = min(v, len(r) - 1)
    lo = c[v - 1] if v > 0 else 0.0
    margin = min(abs(c[v] - target), abs(target - lo))
    return v, margin


# ----------------------------------------------------------------------------
# p/q rejection-sampling verification
# ----------------------------------------------------------------------------

def verify_pq_with_uniforms(block_ids, target_logits, draft_logits,
                            temperature: float, u_accept, u_resample):
    """Speculative-sampling verification of one drafted block, uniforms given.

    [Code] section 8 (_rejection_sample): the drafted token at row j is kept
    with probability p/q (p the target's, q the draft's probability of that
    token); acceptance stops at the first rejection (cumprod prefix); at a
    rejection the replacement is drawn from max(p - q, 0) renormalised; when
    the whole block is kept the bonus token comes from the target's
    distribution at the last row. Probabilities are softmax(logits / T) in fp64.

    Row j (0-based, j < gamma) is accepted iff u_accept[j] < p_j(x)/q_j(x) with
    x = block_ids[j+1]; the replacement at row j or the bonus at row gamma is
    sample_inverse_cdf(weights, u_resample[row]).
    Returns (tau, bonus, diag); diag holds |p/q - u| per tested row and the
    inverse-CDF margin of the final draw (relative to the weights' sum).
    """
    T = np.asarray(target_logits, dtype=F64) / temperature
    Q = np.asarray(draft_logits, dtype=F64) / temperature
    ids = [int(t) for t in block_ids]
    gamma = len(ids) - 1
    diag = {"ratio_margin": [], "cdf_margin": None}
    for j in range(gamma):
        p = softmax(T[j])
        q = softmax(Q[j])
        tok = ids[j + 1]
        ratio = p[tok] / q[tok]
        u = float(u_accept[j])
        diag["ratio_margin"].append(abs(ratio - u))
        if not (u < ratio):
            resid = np.maximum(p - q, 0.0)
            tok2, margin = sample_inverse_cdf(resid, float(u_resample[j]))
            diag["cdf_margin"] = margin / resid.sum()
            return j + 1, tok2, diag
    p = softmax(T[gamma])
    tok2, margin = sample_inverse_cdf(p, float(u_resample[gamma]))
    diag["cdf_margin"] = margin / p.sum()
    return gamma + 1, tok2, diag


def verify_pq(block_ids, target_logits, draft_logits, temperature: float,
              seed: int, row_offset: int = 0, seq: int = 0):
    """verify_pq_with_uniforms with Philox uniforms: the accept test of row j
    uses philox_uniform(seed, row_offset + j, seq, 0), the replacement or bonus
    draw at row j uses philox_uniform(seed, row_offset + j, seq, 1)."""
    B = len(block_ids)
    ua = [philox_uniform(seed, row_offset + j, seq, PURPOSE_ACCEPT)
          for j in range(B - 1)]
    ur = [philox_uniform(seed, row_offset + j, seq, PURPOSE_RESAMPLE)
          for j in range(B)]
    return verify_pq_with_uniforms(block_ids, target_logits, draft_logits,
                                   temperature, ua, ur)


def sample_draft_tokens(draft_logits, temperature: float, seed: int,
                        row_offset: int = 0, seq: int = 0):
    """Draft tokens x_j ~ q_j = softmax(draft_logits[j] / T) by inverse CDF with
    philox_uniform(seed, row_offset + j, seq, 2) ([Code] section 6: the masked
    positions are filled by sampling from the draft distribution when not
    greedy). Returns (tokens, margins)."""
    toks, margins = [], []
    for j in range(draft_logits.shape[0]):
        q = softmax(np.asarray(draft_logits[j], F64) / temperature)
        u = philox_uniform(seed, row_offset + j, seq, PURPOSE_DRAFT)
        t, m = sample_inverse_cdf(q, u)
        toks.append(t)
        margins.append(m)
    return np.array(toks, dtype=np.int64), np.array(margins)


# ----------------------------------------------------------------------------
# DFlash 2 candidate selector
# ----------------------------------------------------------------------------

PURPOSE_SELECT = 3


def top_k_candidates(logits_row, k: int):
    """[Code] section 14 (CandidateSelector.select starts from the top-k of
    each drafted row's logits): the k largest entries of one row, ordered by
    value descending and, among equal values, by index ascending.
    Returns (token ids [k], values [k])."""
    z = np.asarray(logits_row, dtype=F64)
    order = sorted(range(len(z)), key=lambda i: (-z[i], i))[:k]
    idx = np.array(order, dtype=np.int64)
    return idx, z[idx]


def select_candidates(logits, final_hidden, anchor: int, w_proj, pred_codebook,
                      succ_codebook, k: int, temperature: float = 0.0,
                      uniforms=None):
    """The DFlash 2 candidate selector over one drafted block.

    [Code] section 13: every adjacent pair of candidates is scored as
    S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>: U_t the drafter's own logit of
    b at position t, A and B two embedding tables (predecessor and successor
    codes), H(h_t) a projection of the position's hidden state that gates the
    product; the scores are computed in parallel and one greedy walk over them
    is the only serial step. [Code] section 14: the walk starts from the
    anchor (the last confirmed token), takes at each position the top-k
    candidates of that row's logits, moves to the candidate of highest score
    given the current predecessor, and samples from the scores instead when
    the temperature is above zero.

    logits       [P, V]  drafted rows' logits (block rows 1 .. P)
    final_hidden [P, D]  the same rows' hidden states as the LM head reads
                         them (final RMSNorm applied)
    w_proj [r, D], pred_codebook [V, r], succ_codebook [V, r]
    temperature 0: argmax (lowest candidate position on ties); > 0: the
    candidate is drawn from softmax(S / T) over the k candidates with
    uniforms[t] (sample_inverse_cdf in candidate order).
    Returns a dict: path [P] token ids, cand [P, k], scores [P, k] (the scores
    of the step actually taken), q [P, k] (softmax(S / T); one-hot of the
    choice at T = 0), gap [P] (top-1 minus top-2 score at T = 0), margin [P]
    (inverse-CDF margin relative to the total at T > 0).
    """
    Z = np.asarray(logits, dtype=F64)
    P = Z.shape[0]
    A = np.asarray(pred_codebook, dtype=F64)
    Bc = np.asarray(succ_codebook, dtype=F64)
    g = linear(np.asarray(final_hidden, dtype=F64), w_proj)   # H(h_t): [P, r]
    out = {"path": np.zeros(P, np.int64), "cand": np.zeros((P, k), np.int64),
           "scores": np.zeros((P, k)), "q": np.zeros((P, k)), "gap": np.full(P, np.inf),
           "margin": np.full(P, np.inf)}
    pred = int(anchor)
    for t in range(P):
        cand, unary = top_k_candidates(Z[t], k)
        s = unary + (A[pred] * g[t]) @ Bc[cand].T
        if temperature == 0.0:
            i = int(np.argmax(s))
            q = np.zeros(k)
            q[i] = 1.0
            if k > 1:
                top2 = np.sort(s)[-2:]
                out["gap"][t] = top2[1] - top2[0]
        else:
            q = softmax(s / temperature)
            i, m = sample_inverse_cdf(q, float(uniforms[t]))
            out["margin"][t] = m / q.sum()
        pred = int(cand[i])
        out["path"][t], out["cand"][t], out["scores"][t], out["q"][t] = pred, cand, s, q
    return out


def select_candidates_philox(logits, final_hidden, anchor: int, w_proj, pred_codebook,
                             succ_codebook, k: int, temperature: float, seed: int,
                             row_offset: int = 0, seq: int = 0):
    """select_candidates with the walk's uniforms from
    philox_uniform(seed, row_offset + t, seq, 3)."""
    P = np.asarray(logits).shape[0]
    u = [philox_uniform(seed, row_offset + t, seq, PURPOSE_SELECT) for t in range(P)]
    return select_candidates(logits, final_hidden, anchor, w_proj, pred_codebook,
                             succ_codebook, k, temperature, u)


def verify_pq_candidates_with_uniforms(block_ids, target_logits, cand, q_rows,
                                       temperature: float, u_accept, u_resample):
    """p/q verification when the draft distribution lives on candidate sets.

    [Code] section 14: with the candidate selector the draft distribution at
    row j is not a softmax over the vocabulary but the walk's distribution over
    that row's candidates, so q_j(x) is the sum of the row's q entries whose
    candidate is x (zero for every other token) before the p/q rule of
    [Code] section 8 applies unchanged: accept row j iff
    u_accept[j] < p_j(x)/q_j(x) (always when q_j(x) is zero), replacement from
    max(p_j - q_j, 0) renormalised, bonus from p_gamma when every row is kept.

    cand [gamma, k] token ids, q_rows [gamma, k] probabilities.
    Returns (tau, bonus, diag) as verify_pq_with_uniforms."""
    T = np.asarray(target_logits, dtype=F64) / temperature
    ids = [int(t) for t in block_ids]
    gamma = len(ids) - 1
    V = T.shape[1]
    diag = {"ratio_margin": [], "cdf_margin": None}
    for j in range(gamma):
        p = softmax(T[j])
        q = np.zeros(V)
        for c, w in zip(np.asarray(cand[j]), np.asarray(q_rows[j], dtype=F64)):
            q[int(c)] += w
        tok = ids[j + 1]
        u = float(u_accept[j])
        if q[tok] > 0.0:
            ratio = p[tok] / q[tok]
            diag["ratio_margin"].append(abs(ratio - u))
            if not (u < ratio):
                resid = np.maximum(p - q, 0.0)
                tok2, margin = sample_inverse_cdf(resid, float(u_resample[j]))
                diag["cdf_margin"] = margin / resid.sum()
                return j + 1, tok2, diag
        else:
            diag["ratio_margin"].append(np.inf)
    p = softmax(T[gamma])
    tok2, margin = sample_inverse_cdf(p, float(u_resample[gamma]))
    diag["cdf_margin"] = margin / p.sum()
    return gamma + 1, tok2, diag


def verify_pq_candidates(block_ids, target_logits, cand, q_rows, temperature: float,
                         seed: int, row_offset: int = 0, seq: int = 0):
    """verify_pq_candidates_with_uniforms with the Philox uniforms of verify_pq."""
    B = len(block_ids)
    ua = [philox_uniform(seed, row_offset + j, seq, PURPOSE_ACCEPT) for j in range(B - 1)]
    ur = [philox_uniform(seed, row_offset + j, seq, PURPOSE_RESAMPLE) for j in range(B)]
    return verify_pq_candidates_with_uniforms(block_ids, target_logits, cand, q_rows,
                                              temperature, ua, ur)


# ----------------------------------------------------------------------------
# DFlash 2 grouped dynamic two-tap causal conv
# ----------------------------------------------------------------------------

CONV_TAPS = 2


def dynamic_conv_param_count(hidden: int, group_size: int, n_layers: int,
                             instances_per_layer: int = 2) -> int:
    """[Code] section 14 (GroupedDynamicCausalConv): each instance holds a base
    kernel of shape (2, taps, hidden) and a bias-free projection from the
    hidden state to 2 * taps * groups values, groups = hidden / group_size;
    every layer has two instances (one by attention, one by the MLP)."""
    groups = hidden // group_size
    per = 2 * CONV_TAPS * hidden + hidden * 2 * CONV_TAPS * groups
    return n_layers * instances_per_layer * per


def dynamic_conv_coefficients(h_row, base_call, proj, group_size: int, call: int):
    """Per-channel tap coefficients of one position for one call ([Code]
    section 13: learned base kernel plus a correction computed from the
    current hidden state, one correction per group of group_size channels).
    h_row [D]; base_call [taps, D] = base[call]; proj [2 * taps * G, D].
    Returns coef [taps, D]."""
    D = len(h_row)
    G = D // group_size
    corr = np.asarray(proj, dtype=F64) @ np.asarray(h_row, dtype=F64)  # [2 * taps * G]
    corr = corr.reshape(2, CONV_TAPS, G)[call]                          # [taps, G]
    group_of = np.arange(D) // group_size
    return np.asarray(base_call, dtype=F64) + corr[:, group_of]


def _conv_block(x, prev, block_len: int, coef_rows):
    """y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1} ([Code] section 13) over blocks
    of block_len consecutive rows; the first row of block s reads prev[s]."""
    x = np.asarray(x, dtype=F64)
    prev = np.asarray(prev, dtype=F64)
    y = np.empty_like(x)
    for m in range(x.shape[0]):
        s, t = divmod(m, block_len)
        before = prev[s] if t == 0 else x[m - 1]
        k = coef_rows[m]
        y[m] = k[0] * x[m] + k[1] * before
    return y


def dynamic_conv_prepare(x, prev, block_len: int, base, proj, group_size: int):
    """The "prepare" call of one conv instance over n_seqs blocks.

    x [n_seqs * block_len, D]  the module's input rows, block by block
    prev [n_seqs, D]           the row each block's first position reads
    base [2, taps, D], proj [2 * taps * G, D]
    Returns (y [rows, D], corr_finish [rows, taps * G]): the conv of x with
    the call-0 coefficients, and the call-1 half of every row's correction
    for the finish call."""
    x = np.asarray(x, dtype=F64)
    D = x.shape[1]
    G = D // group_size
    base = np.asarray(base, dtype=F64)
    coef = [dynamic_conv_coefficients(x[m], base[0], proj, group_size, 0)
            for m in range(x.shape[0])]
    corr = (x @ np.asarray(proj, dtype=F64).T).reshape(-1, 2, CONV_TAPS, G)[:, 1]
    return _conv_block(x, prev, block_len, coef), corr.reshape(-1, CONV_TAPS * G)


def dynamic_conv_finish(z, prev, block_len: int, base, corr_finish, group_size: int):
    """The "finish" call: the conv of z with base[1] plus the call-1
    corrections the prepare call computed for the same rows.
    z [rows, D], prev [n_seqs, D], corr_finish [rows, taps * G]."""
    z = np.asarray(z, dtype=F64)
    D = z.shape[1]
    G = D // group_size
    base = np.asarray(base, dtype=F64)
    c = np.asarray(corr_finish, dtype=F64).reshape(-1, CONV_TAPS, G)
    group_of = np.arange(D) // group_size
    coef = [base[1] + c[m][:, group_of] for m in range(z.shape[0])]
    return _conv_block(z, prev, block_len, coef)
