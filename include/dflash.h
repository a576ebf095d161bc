/*
 * dflash.h - C ABI of the DFlash drafter hot path on MI355X (gfx950).
 *
 * DFlash drafts a whole block in one forward pass: the anchor token (the last
 * confirmed token) followed by block_size-1 mask tokens, conditioned on a
 * fused feature of the target model's hidden states that is injected as extra
 * K/V entries into every draft layer; the drafted block is then verified
 * against the target's logits.
 *
 * Sources: the four web pages on DFlash, cited as
 *   [Tut]  A3-dflash tutorial (CCODING04 llm-paper-tutorials)
 *   [Sum]  papercache summary "DFlash: Block Diffusion for Flash Speculative Decoding"
 *   [Note] tom-jerr paper-reading notes "DFLASH"
 *   [Code] txtmix code-reading article on the z-lab dflash repository
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates no device memory: scratch space comes from the workspace the
 *     caller hands over with dflash_set_workspace.
 *   - Weights are borrowed for the handle's lifetime and never written.
 *     Matrices are bf16, row-major, nn.Linear layout [out_features, in_features].
 *   - Calls only enqueue work on the handle's HIP stream; results are valid
 *     after that stream is synchronised. Host-side metadata (dflash_kv.len) is
 *     updated when the call returns.
 *   - All argument checks run on the host before anything is enqueued. On any
 *     error nothing is written and every dflash_kv.len is unchanged.
 *   - DFLASH_E_DEVICE reports a failed HIP launch; the handle should then be
 *     destroyed.
 *   - A handle is not re-entrant: use one handle per host thread and stream.
 *   - dflash_last_error() returns a thread-local text for the last failure.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dflash_status {
  DFLASH_OK = 0,
  DFLASH_E_NULL = 1,      /* a required pointer is NULL */
  DFLASH_E_CONFIG = 2,    /* configuration invalid or unsupported */
  DFLASH_E_SHAPE = 3,     /* a size or index argument is out of range */
  DFLASH_E_CAPACITY = 4,  /* a cache or the workspace is too small */
  DFLASH_E_ALIGN = 5,     /* a pointer or stride is not suitably aligned */
  DFLASH_E_DEVICE = 6,    /* a HIP call failed */
  DFLASH_E_STATE = 7      /* call made in the wrong state (e.g. no workspace) */
} dflash_status;

/*
 * Model dimensions and the draft configuration. The required keys mirror the
 * checkpoint's dflash_config ([Code] section 11): mask_token_id has no
 * default (a negative value is DFLASH_E_CONFIG); block_size defaults to 16.
 * Supported: hidden % 64 == 0, head_dim in {16, 32, 64, 128},
 * n_heads % n_kv_heads == 0 with n_heads / n_kv_heads <= 16, ffn % 32 == 0, (n_heads + 2*n_kv_heads)*head_dim % 32 == 0,
 * 1 <= block_size <= 16, n_feat_layers in 1..8.
 */
typedef struct dflash_config {
  int32_t hidden;         /* D: hidden size of target and draft */
  int32_t n_feat_layers;  /* number of fused target layers (5 on the pages) */
  int32_t n_layers;       /* draft decoder layers */
  int32_t n_heads;        /* query heads */
  int32_t n_kv_heads;     /* key/value heads (grouped-query attention) */
  int32_t head_dim;
  int32_t ffn;            /* SwiGLU intermediate size */
  int32_t vocab;
  int32_t block_size;     /* 0 -> 16 */
  int32_t mask_token_id;  /* required, 0 <= id < vocab */
  float rms_eps;          /* <= 0 -> 1e-6 */
  float rope_theta;       /* <= 0 -> 1e6 */
} dflash_config;

/* One draft decoder layer (pre-norm attention + SwiGLU MLP), bf16. */
typedef struct dflash_layer_weights {
  const void* wq;         /* [n_heads*head_dim, D] */
  const void* wk;         /* [n_kv_heads*head_dim, D] */
  const void* wv;         /* [n_kv_heads*head_dim, D] */
  const void* wo;         /* [D, n_heads*head_dim] */
  const void* w_gate;     /* [ffn, D] */
  const void* w_up;       /* [ffn, D] */
  const void* w_down;     /* [D, ffn] */
  const void* attn_norm;  /* [D] RMSNorm gain before attention */
  const void* mlp_norm;   /* [D] RMSNorm gain before the MLP */
} dflash_layer_weights;

/*
 * All parameters. The embedding and LM head are the target's own, shared and
 * frozen ([Tut] section 2.2.3; [Code] section 3). w_c is the fusion matrix
 * W_c of [Tut] section 2.1.2, D x (n_feat_layers*D).
 */
typedef struct dflash_weights {
  const void* w_c;         /* [D, n_feat_layers*D] */
  const void* ctx_norm;    /* [D] RMSNorm gain of the fused feature */
  const void* embed;       /* [vocab, D] */
  const void* lm_head;     /* [vocab, D] */
  const void* final_norm;  /* [D] RMSNorm gain before the LM head */
  const dflash_layer_weights* layers;  /* host array [n_layers], copied */
} dflash_weights;

/*
 * One sequence's draft KV cache: the context K/V of every draft layer
 * ([Sum] section 4.1: the projected target features are kept in the draft
 * model's KV cache and reused across drafting rounds).
 *
 * `base` is a caller-allocated device buffer of dflash_kv_bytes(cfg, max_ctx)
 * bytes, 256-byte aligned. With cap = dflash_kv_row_capacity(cfg, max_ctx),
 * H = n_kv_heads, hd = head_dim, the bf16 elements are laid out as
 *   K (after RoPE): layer i, head g, position p, dim d at
 *       ((2*i + 0)*H + g)*cap*hd + p*hd + d
 *   V:              layer i, head g, position p, dim d at
 *       ((2*i + 1)*H + g)*cap*hd + d*cap + p
 * i.e. K is position-major and V dim-major within each head. Positions
 * >= len are never part of the context; dflash_draft_block writes nothing
 * into the cache (the block's own K/V stay in the workspace, in fp32). Rows
 * past max_ctx (cap >= max_ctx + block_size) are never written or read.
 * `len` is host metadata: the number of context positions held.
 */
typedef struct dflash_kv {
  void* base;
  int32_t max_ctx;   /* context positions the buffer can hold */
  int32_t len;       /* current context length */
} dflash_kv;

typedef struct dflash_handle dflash_handle;

/* Bytes of a KV buffer for max_ctx context positions (plus block scratch). */
size_t dflash_kv_bytes(const dflash_config* cfg, int32_t max_ctx);
/* Row capacity `cap` used in the layout above (>= max_ctx + block_size). */
int32_t dflash_kv_row_capacity(const dflash_config* cfg, int32_t max_ctx);

/*
 * Workspace bytes for draft calls of up to max_seqs sequences and fuse/inject
 * calls of up to max_tokens rows. 0 on an invalid config.
 */
size_t dflash_workspace_bytes(const dflash_config* cfg, int32_t max_seqs,
                              int32_t max_tokens);

/*
 * Create a handle. `stream` is a hipStream_t (NULL = the default stream).
 * Copies the config and the weight pointers; validates them (DFLASH_E_CONFIG,
 * DFLASH_E_NULL, DFLASH_E_ALIGN for matrices not 16-byte aligned).
 */
dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w,
                            void* stream, dflash_handle** out);
dflash_status dflash_destroy(dflash_handle* h);
dflash_status dflash_set_stream(dflash_handle* h, void* stream);

/*
 * Hand over the workspace: a device buffer of at least
 * dflash_workspace_bytes(cfg, max_seqs, max_tokens) bytes, 256-byte aligned,
 * owned by the caller and not touched by anyone else while the handle uses it.
 */
dflash_status dflash_set_workspace(dflash_handle* h, void* ws, size_t bytes,
                                   int32_t max_seqs, int32_t max_tokens);

/*
 * Context fusion ([Tut] sections 2.1.1-2.1.2; [Code] section 5):
 *   ctx_out[t] = RMSNorm(W_c [h_1[t]; ...; h_n[t]]) * ctx_norm, eps inside the
 *   square root.
 * feats: host array of n_feat_layers device pointers, each bf16 [n_tokens, ld]
 * (row stride ld elements, ld >= D, ld % 8 == 0), in increasing layer order;
 * the concatenation is never materialised. ctx_out: bf16 [n_tokens, D]; the
 * projection stays fp32 until the norm, so each output is rounded to bf16
 * once. 1 <= n_tokens <= max_tokens of the workspace.
 */
dflash_status dflash_fuse_context(dflash_handle* h, const void* const* feats,
                                  int64_t ld, int32_t n_tokens, void* ctx_out);

/*
 * KV injection ([Tut] section 2.1.2: K_i = [W_i^K H_t ; ...],
 * V_i = [W_i^V H_t ; ...]; [Code] section 5): for every draft layer i and
 * t < n_tokens, K = RoPE(wk_i ctx_feat[t], pos0 + t) and V = wv_i ctx_feat[t]
 * are written at position pos0 + t. The cache is first cut back to pos0
 * (0 <= pos0 <= kv->len), so a trim of rejected positions followed by an
 * append of the accepted prefix is one call ([Code] section 9).
 * On success kv->len = pos0 + n_tokens (<= kv->max_ctx, else DFLASH_E_CAPACITY).
 * ctx_feat: bf16 [n_tokens, D]; 1 <= n_tokens <= max_tokens.
 */
dflash_status dflash_inject_kv(dflash_handle* h, dflash_kv* kv,
                               const void* ctx_feat, int32_t n_tokens,
                               int32_t pos0);

/* Trim: kv->len = keep_len (0 <= keep_len <= kv->len). Host only. */
dflash_status dflash_kv_trim(dflash_handle* h, dflash_kv* kv, int32_t keep_len);

/*
 * One draft forward over n_seqs blocks ([Code] sections 6 and 9;
 * [Tut] section 2.1.2):
 *   block row r of sequence s holds anchor_ids[s] (r = 0) or mask_token_id,
 *   at position kvs[s]->len + r; every row attends, without any mask, to the
 *   sequence's context K/V and to the block's own K/V; the LM head and argmax
 *   are applied to rows 1..block_len-1.
 * anchor_ids: device int32 [n_seqs].
 * block_out:  device int32 [n_seqs, block_len] - column 0 is the anchor,
 *             columns 1.. the drafted tokens (lowest index on exact ties);
 *             this is the block dflash_verify takes.
 * hidden_out: optional device fp32 [n_layers, n_seqs*block_len, D] - residual
 *             stream after every layer (row s*block_len + r).
 * logits_out: optional device fp32 [n_seqs, block_len-1, vocab].
 * 1 <= n_seqs <= max_seqs; 1 <= block_len <= block_size; each kvs[s]->len is
 * left unchanged and the cache is only read (the block's own K/V are kept in
 * the workspace in fp32 and enter attention in its merge step).
 */
dflash_status dflash_draft_block(dflash_handle* h, int32_t n_seqs,
                                 dflash_kv* const* kvs,
                                 const int32_t* anchor_ids, int32_t block_len,
                                 int32_t* block_out, float* hidden_out,
                                 float* logits_out);

/*
 * Device-resident speculative rounds ([Code] section 9: draft, verify, crop
 * the cache to the accepted prefix, append the accepted rows' features).
 * Here the context length of each sequence lives in device memory
 * (len_dev: device int32 [n_seqs], one per kvs[s]) instead of kvs[s]->len,
 * so that tau never has to come back to the host and a whole round can be
 * captured into a graph. kvs[s]->base and ->max_ctx are still read on the
 * host; kvs[s]->len is not used by these calls. A device length outside
 * 0..max_ctx is clamped into it.
 *
 * dflash_draft_block_dev: dflash_draft_block with the lengths read from
 *   len_dev (attention is planned for the buffers' capacity; key ranges past
 *   a sequence's length are skipped). len_dev is not changed.
 * dflash_append_dev: the append after verification. feats: n_feat_layers
 *   device bf16 arrays [n_seqs * rows_per_seq, hidden] (row stride ld) with
 *   the target's hidden states of each sequence's verified block rows,
 *   sequence s at rows s*rows_per_seq ...; the rows are fused
 *   (dflash_fuse_context), the first tau_dev[s] rows of sequence s are
 *   injected (dflash_inject_kv) at positions len_dev[s] ..., rows that would
 *   land at or past max_ctx are dropped, and len_dev[s] becomes
 *   min(len_dev[s] + tau_dev[s], max_ctx). tau_dev: device int32 [n_seqs]
 *   (dflash_verify's tau_out). 1 <= rows_per_seq <= block_size;
 *   n_seqs * rows_per_seq <= max_tokens of the workspace.
 * dflash_kv_trim_dev: len_dev[s] = min(len_dev[s], keep_len), s < n_seqs.
 * Errors as for the other calls: checked on the host before any launch.
 */
dflash_status dflash_draft_block_dev(dflash_handle* h, int32_t n_seqs,
                                     dflash_kv* const* kvs, const int32_t* len_dev,
                                     const int32_t* anchor_ids, int32_t block_len,
                                     int32_t* block_out, float* hidden_out,
                                     float* logits_out);
dflash_status dflash_append_dev(dflash_handle* h, int32_t n_seqs, dflash_kv* const* kvs,
                                int32_t* len_dev, const int32_t* tau_dev,
                                const void* const* feats, int64_t ld,
                                int32_t rows_per_seq);
dflash_status dflash_kv_trim_dev(dflash_handle* h, int32_t n_seqs, int32_t* len_dev,
                                 int32_t keep_len);

/*
 * Sampling-mode drafting ([Code] section 6: away from greedy decoding the
 * masked positions take tokens sampled from the draft's distribution; the
 * p/q rule of dflash_verify needs x ~ q): for each sequence s and drafted row
 * j < block_len-1, block_ids[s][j+1] becomes the token drawn from
 * q = softmax(draft_logits[s][j] / temperature) (fp64) as the smallest v whose
 * running sum in vocab order exceeds u * total, with u the Philox4x64-10
 * uniform of counter (philox_offset + j, s, 2, 0), key (seed, 0),
 * u = (word0 >> 11) * 2^-53.
 * draft_logits: device fp32 [n_seqs, block_len-1, vocab] (dflash_draft_block's
 *               logits_out);
 * block_ids:    device int32 [n_seqs, block_len]; column 0 (the anchor) is
 *               left as it is.
 * temperature > 0 (finite); 1 <= n_seqs <= max_seqs; 1 <= block_len <=
 * block_size (block_len == 1: nothing to do). Errors as for the other calls:
 * checked on the host before any launch, nothing written on error.
 */
dflash_status dflash_sample_draft(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                  const float* draft_logits, float temperature,
                                  uint64_t seed, uint64_t philox_offset,
                                  int32_t* block_ids);

/*
 * Verification of n_seqs drafted blocks against the target's logits.
 * temperature == 0: greedy ([Code] section 8): posterior = argmax of each
 *   target row (lowest index on ties); accepted a = length of the prefix with
 *   block[j+1] == posterior[j]; bonus = posterior[a]; tau = a + 1.
 * temperature > 0: p/q rejection sampling ([Code] section 8): with
 *   p_j = softmax(target_logits[j]/T), q_j = softmax(draft_logits[j]/T) in fp64,
 *   row j is accepted iff u_j < p_j(x)/q_j(x), x = block[j+1]; at the first
 *   rejection the bonus is drawn from max(p_j - q_j, 0) normalised; when all
 *   rows are accepted it is drawn from p_{block_len-1}. Uniforms come from
 *   Philox4x64-10 with key (seed, 0) and counter
 *   (philox_offset + row, sequence, purpose, 0), purpose 0 = accept test,
 *   1 = replacement/bonus draw; u = (word0 >> 11) * 2^-53. A draw picks the
 *   smallest v whose running fp64 sum in vocab order exceeds u * total.
 * block_ids:     device int32 [n_seqs, block_len]
 * target_logits: device fp32 [n_seqs, block_len, vocab]
 * draft_logits:  device fp32 [n_seqs, block_len-1, vocab]; NULL iff T == 0
 * tau_out, bonus_out: device int32 [n_seqs]; 1 <= tau <= block_len.
 * 1 <= n_seqs <= max_seqs; 1 <= block_len <= block_size.
 */
dflash_status dflash_verify(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                            const int32_t* block_ids, const float* target_logits,
                            const float* draft_logits, float temperature,
                            uint64_t seed, uint64_t philox_offset,
                            int32_t* tau_out, int32_t* bonus_out);

/*
 * dflash_verify without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments, checks and results as
 * dflash_verify, but the handle needs no workspace (dflash_set_workspace is
 * not required) and the kernels' partials live in a fixed scratch array of
 * the library, one per GPU, 2.6 MiB, held until the process ends. Nothing is
 * allocated and nothing in the scratch needs clearing (every partial is
 * written before it is read).
 * Limits: 1 <= n_seqs <= 64; the verification rows - n_seqs * block_len
 * (greedy) or n_seqs * (2 * block_len - 1) (p/q) - at most 2048, else
 * DFLASH_E_CAPACITY with nothing launched.
 * All calls on one GPU share that GPU's scratch: calls that overlap on one
 * GPU (concurrent streams, or several host threads) race and must not be
 * made. The scratch's device address is looked up on the first call on each
 * device (with that device current); a failure there is DFLASH_E_DEVICE.
 */
dflash_status dflash_verify_noalloc(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                    const int32_t* block_ids, const float* target_logits,
                                    const float* draft_logits, float temperature,
                                    uint64_t seed, uint64_t philox_offset,
                                    int32_t* tau_out, int32_t* bonus_out);

/*
 * DFlash 2 grouped dynamic two-tap causal conv inside every draft layer
 * ([Code] section 13: y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1} per channel,
 * each coefficient a learned base plus a correction computed from the hidden
 * state, one correction per group_size channels, acting only inside the
 * block with no state across steps; section 14: two instances per layer, one
 * by attention and one by the MLP, base kernel (2, taps, hidden) whose first
 * index separates the "prepare" and "finish" calls, a bias-free projection
 * to 2 * taps * groups corrections).
 * dflash_set_conv borrows one dflash_conv_layer per draft layer (layers[i]
 * for layer i; NULL layers removes the convs); from then on
 * dflash_draft_block and dflash_draft_block_dev run each layer as
 *   h = RMSNorm(x); (h', c) = prepare(h); attention on h';
 *   x += finish(o_proj output; c); h2 = RMSNorm(x); (h2', c2) = prepare(h2);
 *   x += finish(MLP(h2'); c2)
 * where prepare(v) convolves v with base[0] plus the call-0 corrections of
 * the projection of v and returns the call-1 corrections c; finish(z; c)
 * convolves z with base[1] plus c; the block's first row reads a zero row as
 * its predecessor. (That the calls sit on the sublayer's normed input and
 * output is this library's reading; the pages do not place them.)
 * Tables: *_base bf16 [2, 2, hidden] (call, tap, channel); *_proj bf16
 * [4 * hidden / group_size, hidden], rows ordered (call, tap, group), as
 * dflash_conv_prepare. hidden % (16 * group_size) == 0; tables 16-byte
 * aligned. The handle keeps the pointers; nothing is copied or allocated.
 */
typedef struct {
  const void* attn_base;
  const void* attn_proj;
  const void* mlp_base;
  const void* mlp_proj;
} dflash_conv_layer;
dflash_status dflash_set_conv(dflash_handle* h, const dflash_conv_layer* layers, int32_t group_size);

/*
 * DFlash 2 candidate selector ([Code] section 13: the right token is usually
 * among a drafted row's top candidates; each adjacent pair is scored as
 * S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>, and one walk over the scores
 * picks the block; [Code] section 14: CandidateSelector.select).
 *
 * dflash_set_selector: borrows the selector's tables for the handle's
 *   lifetime (NULL sel removes them).
 *   hidden_proj:   bf16 [rank, hidden]  H, no bias
 *   pred_codebook: bf16 [vocab, rank]   A (predecessor codes)
 *   succ_codebook: bf16 [vocab, rank]   B (successor codes)
 *   1 <= top_k <= 16; 64 <= rank <= 256, rank % 64 == 0.
 *
 * dflash_select_block: for sequence s and drafted row j < block_len-1 (block
 *   row j+1): the candidates are the top_k tokens of draft_logits[s][j]
 *   (value descending, index ascending among equal values); g_j = H h_j with
 *   h_j the LM head's input row (the final RMSNorm of last_hidden's block row
 *   j+1, weighted by the final norm gain); the walk starts at a =
 *   anchor_ids[s], scores every candidate b as
 *   logit(b) + sum_x A[a][x] g_j[x] B[b][x] (fp32), and moves to
 *   temperature == 0: the best candidate (first in candidate order on ties);
 *   temperature > 0:  the candidate drawn from q = softmax(scores / T) in
 *     fp64: the first whose running sum in candidate order exceeds u * total,
 *     u the Philox4x64-10 uniform of counter (philox_offset + j, s, 3, 0),
 *     key (seed, 0), u = (word0 >> 11) * 2^-53.
 *   block_ids[s][j+1] becomes the chosen token (column 0 is left as it is).
 * last_hidden: device fp32 [n_seqs * block_len, hidden] - the residual stream
 *              after the last layer (dflash_draft_block's hidden_out, layer
 *              n_layers-1), row s*block_len + r;
 * draft_logits: device fp32 [n_seqs, block_len-1, vocab] (logits_out);
 * anchor_ids:  device int32 [n_seqs] (a value outside the vocabulary is
 *              clamped into it for the code lookup);
 * block_ids:   device int32 [n_seqs, block_len];
 * cand_out:    optional device int32 [n_seqs, block_len-1, top_k] - the
 *              candidates of every row, in candidate order;
 * q_out:       optional device fp32 [n_seqs, block_len-1, top_k] - the walk's
 *              distribution at each row (one-hot of the choice at T == 0).
 * A selector must be set; 1 <= n_seqs <= max_seqs; 1 <= block_len <=
 * block_size, block_len - 1 <= 64; top_k <= vocab. Errors as for the other
 * calls: checked on the host before any launch, nothing written on error.
 */
typedef struct dflash_selector {
  const void* hidden_proj;
  const void* pred_codebook;
  const void* succ_codebook;
  int32_t rank;
  int32_t top_k;
} dflash_selector;

dflash_status dflash_set_selector(dflash_handle* h, const dflash_selector* sel);
dflash_status dflash_select_block(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                  const float* last_hidden, const float* draft_logits,
                                  const int32_t* anchor_ids, float temperature,
                                  uint64_t seed, uint64_t philox_offset,
                                  int32_t* block_ids, int32_t* cand_out, float* q_out);

/*
 * p/q verification with the draft distribution on candidate sets ([Code]
 * section 14: with the candidate selector the draft's distribution at a row
 * is the walk's distribution over that row's candidates, so q(x) is summed
 * over the candidates equal to x, zero for any other token; without this the
 * rule is no longer lossless). Otherwise dflash_verify at temperature > 0:
 * row j is accepted iff u_j < p_j(x)/q_j(x) (always when q_j(x) == 0), the
 * replacement is drawn from max(p_j - q_j, 0) normalised, the bonus from
 * p_{block_len-1}; same Philox counters, inverse-CDF rule and outputs.
 * cand:   device int32 [n_seqs, block_len-1, top_k] (dflash_select_block's
 *         cand_out);
 * q_rows: device fp32 [n_seqs, block_len-1, top_k] (its q_out);
 * 1 <= top_k <= 16; temperature > 0 (finite); other arguments and errors as
 * for dflash_verify.
 */
dflash_status dflash_verify_candidates(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                       const int32_t* block_ids, const float* target_logits,
                                       const int32_t* cand, const float* q_rows, int32_t top_k,
                                       float temperature, uint64_t seed, uint64_t philox_offset,
                                       int32_t* tau_out, int32_t* bonus_out);

/*
 * DFlash 2 grouped dynamic two-tap causal conv ([Code] section 13: each
 * channel's output is k_{t,0} * x_t + k_{t,1} * x_{t-1}, every coefficient
 * a learned base value plus a correction computed from the current hidden
 * state, one correction shared by each group of channels, and a block's
 * first position reading the last confirmed token's representation;
 * [Code] section 14: GroupedDynamicCausalConv with a base kernel of shape
 * (2, taps, hidden) whose first index separates the "prepare" and "finish"
 * calls, and a bias-free projection to 2 * taps * groups values).
 * Readings: two taps; the projection's outputs are ordered (call, tap,
 * group) row-major; both calls' corrections come from the prepare call's
 * input; the output replaces the input (no residual inside the module).
 * Where the calls sit in a decoder layer is the caller's choice.
 *
 * Rows: n_seqs blocks of block_len consecutive rows (row s*block_len + t).
 * G = hidden / group_size.
 * base: device bf16 [2, 2, hidden] (call, tap, channel)
 * proj: device bf16 [4 * G, hidden], row (call * 2 + tap) * G + g
 *
 * dflash_conv_prepare:
 *   y[m][c] = (base[0][0][c] + P0[m][g]) * x[m][c]
 *           + (base[0][1][c] + P1[m][g]) * (t > 0 ? x[m-1][c] : prev[s][c])
 *   with P = proj . x[m] (fp32 accumulation of the bf16 weights against the
 *   fp32 row split into bf16 high and low halves), g = c / group_size;
 *   corr_out[m] = the call-1 corrections (tap, group): [2 * G] per row.
 * dflash_conv_finish:
 *   y[m][c] = (base[1][0][c] + corr[m][g]) * z[m][c]
 *           + (base[1][1][c] + corr[m][G + g]) * (t > 0 ? z[m-1][c] : prev[s][c])
 * x, z, y:     device fp32 [n_seqs * block_len, hidden] (x and z 16-byte
 *              aligned, y 4-byte);
 * prev:        device fp32 [n_seqs, hidden];
 * corr_out / corr: device fp32 [n_seqs * block_len, 2 * G]; corr_out must
 *              not overlap x. base and proj 16-byte aligned.
 * 1 <= n_seqs <= max_seqs; 1 <= block_len <= block_size; group_size >= 1,
 * hidden % (16 * group_size) == 0. y must not overlap the inputs. Errors are
 * found on the host before any launch; nothing is written on error. The
 * prepare call uses the handle's workspace (calls on one handle are ordered
 * on its stream).
 */
dflash_status dflash_conv_prepare(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                  int32_t group_size, const void* base, const void* proj,
                                  const float* x, const float* prev, float* y, float* corr_out);
dflash_status dflash_conv_finish(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                 int32_t group_size, const void* base, const float* z,
                                 const float* prev, const float* corr, float* y);

/*
 * Host helper ([Code] section 5, build_target_layer_ids): n_feat target layer
 * indices spread evenly over 1 .. n_target_layers-3 (0-based), rounded to
 * nearest; the middle layer when n_feat == 1. out: host int32 [n_feat].
 */
dflash_status dflash_target_layer_ids(int32_t n_target_layers, int32_t n_feat,
                                      int32_t* out);

/*
 * Optional timing of the launches a handle makes (tracing). Stages:
 *   0 embed, 1 qkv, 2 attention (split + merge), 3 o_proj, 4 gate_up,
 *   5 down_proj, 6 lm_head (the LM-head GEMM kernel alone), 7 fuse_context,
 *   8 inject_kv, 9 verify, 10 lm_argmax (split sums, optional logits and the
 *   argmax reduction that writes the drafted tokens).
 * With bit k of stage_mask set, every launch of stage k is bracketed by two
 * hipEvents recorded on the handle's stream, up to max_records launches
 * (later ones are not recorded). The events are host-side objects created
 * here; no device memory is allocated. stage_mask 0 disables timing and
 * releases the events. Enabling clears previous records.
 */
dflash_status dflash_profile_enable(dflash_handle* h, uint32_t stage_mask,
                                    int32_t max_records);
/*
 * Read the records made since enabling (waits for their events): up to
 * `cap` entries of stage id and elapsed milliseconds, in launch order;
 * *n_out receives the number of records. Clears the records.
 */
dflash_status dflash_profile_read(dflash_handle* h, int32_t cap, int32_t* stage_out,
                                  float* ms_out, int32_t* n_out);
const char* dflash_stage_name(int32_t stage);

/*
 * Measurement reference, not part of the drafting method: copy `bytes` from
 * device memory src to device memory dst on `stream` (a hipStream_t, NULL =
 * the default stream) with the access shape of the weight streams (16-byte
 * vector loads and stores, a contiguous kilobyte per wave instruction).
 * Byte counters read for this copy calibrate the traffic measured for the
 * other kernels. Both pointers 16-byte aligned and bytes a multiple of 16,
 * else DFLASH_E_ALIGN; null pointers with bytes > 0 give DFLASH_E_NULL. The
 * buffers must not overlap. Nothing is allocated.
 */
dflash_status dflash_copy_bytes(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Measurement reference, not part of the drafting method: read `bytes` of
 * device memory src on `stream` with the access pattern of the weight
 * streams (512-byte pieces of 16 rows of 8 KB, direct global-to-LDS loads
 * with the non-temporal hint, one workgroup per CU), computing nothing; its
 * rate is the read ceiling those kernels can reach. sink: device memory of at
 * least 256 32-bit words, written only in a case that cannot occur (so the
 * loads are not removed). src 16-byte aligned, sink 4-byte aligned, bytes a
 * multiple of 128 KiB, else DFLASH_E_ALIGN; null pointers with bytes > 0
 * give DFLASH_E_NULL. Nothing is allocated.
 */
dflash_status dflash_read_bytes(const void* src, size_t bytes, void* sink, void* stream);

const char* dflash_status_str(dflash_status s);
const char* dflash_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
