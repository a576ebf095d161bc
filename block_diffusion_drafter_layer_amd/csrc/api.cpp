// Host side of the C ABI declared in include/dflash.h: argument checks,
// workspace carving and the launch order of each call. Everything the calls
// compute runs in the HIP kernels of this directory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "dflash.h"
#include "launch.h"

using namespace dfl;

namespace {

thread_local std::string g_err;

dflash_status fail(dflash_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

dflash_status dev_fail(hipError_t e, const char* what) {
  return fail(DFLASH_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

dflash_config normalized(const dflash_config& c) {
  dflash_config n = c;
  if (n.block_size == 0) n.block_size = 16;
  if (!(n.rms_eps > 0.f)) n.rms_eps = 1e-6f;
  if (!(n.rope_theta > 0.f)) n.rope_theta = 1e6f;
  return n;
}

dflash_status check_config(const dflash_config& c) {
  if (c.hidden <= 0 || c.hidden % 64)
    return fail(DFLASH_E_CONFIG, "hidden=%d must be a positive multiple of 64", c.hidden);
  if (c.n_feat_layers < 1 || c.n_feat_layers > kMaxFeat)
    return fail(DFLASH_E_CONFIG, "n_feat_layers=%d outside 1..%d", c.n_feat_layers, kMaxFeat);
  if (c.n_layers < 1 || c.n_layers > kMaxLayers)
    return fail(DFLASH_E_CONFIG, "n_layers=%d outside 1..%d", c.n_layers, kMaxLayers);
  if (!(c.head_dim == 16 || c.head_dim == 32 || c.head_dim == 64 || c.head_dim == 128))
    return fail(DFLASH_E_CONFIG, "head_dim=%d not in {16,32,64,128}", c.head_dim);
  if (c.n_kv_heads < 1 || c.n_kv_heads > 16 || c.n_heads < c.n_kv_heads ||
      c.n_heads % c.n_kv_heads || c.n_heads / c.n_kv_heads > 16)
    return fail(DFLASH_E_CONFIG, "heads %d/%d: need n_heads %% n_kv_heads == 0, group <= 16, n_kv_heads <= 16",
                c.n_heads, c.n_kv_heads);
  if ((c.n_heads * c.head_dim) % 32 || ((c.n_heads + 2 * c.n_kv_heads) * c.head_dim) % 32)
    return fail(DFLASH_E_CONFIG, "q and qkv widths must be multiples of 32");
  if (c.ffn <= 0 || c.ffn % 32) return fail(DFLASH_E_CONFIG, "ffn=%d must be a positive multiple of 32", c.ffn);
  if (c.vocab < 2) return fail(DFLASH_E_CONFIG, "vocab=%d", c.vocab);
  if (c.block_size < 1 || c.block_size > 16)
    return fail(DFLASH_E_CONFIG, "block_size=%d outside 1..16", c.block_size);
  if (c.mask_token_id < 0 || c.mask_token_id >= c.vocab)
    return fail(DFLASH_E_CONFIG, "mask_token_id=%d is required and must lie in [0, vocab)", c.mask_token_id);
  if (!std::isfinite(c.rms_eps) || !std::isfinite(c.rope_theta) || c.rope_theta <= 1.f)
    return fail(DFLASH_E_CONFIG, "rms_eps / rope_theta invalid");
  return DFLASH_OK;
}

int32_t row_capacity(const dflash_config& c, int32_t max_ctx) {
  return (int32_t)align_up((size_t)max_ctx + (size_t)c.block_size, 64);
}

constexpr size_t kSplitPartFloats = (size_t)kSplitMaxWG * 32 * 64;  // <= 32 rows x 64 columns each

// split buffer: the register-streaming kernel's partial tiles, or the
// LDS-staged kernel's [pair][slice][16][32] partials of the largest GEMM
size_t split_floats(const dflash_config& c) {
  const int qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  const int nf = c.n_feat_layers > 0 ? c.n_feat_layers : 1;
  size_t f = kSplitPartFloats;
  f = std::max(f, stream_part_floats(qd + 2 * kvd, c.hidden));
  f = std::max(f, stream_part_floats(c.hidden, qd));
  f = std::max(f, stream_part_floats(2 * c.ffn, c.hidden));
  f = std::max(f, stream_part_floats(c.hidden, c.ffn));
  f = std::max(f, stream_part_floats(c.vocab, c.hidden));
  f = std::max(f, stream_part_floats(c.hidden, nf * c.hidden));
  f = std::max(f, stream_part_floats(c.n_layers * 2 * kvd, c.hidden));
  return f;
}

struct Layout {
  size_t split_part, x, xh, xl, ssq, q, q_lo, blk_k, blk_v, ob_h, ob_l, act_h, act_l, lm_part, att_acc, att_ml, vpart, fuse_ssq;
  size_t gemm_part, gemm_ctr;   // context-GEMM split-K partials and counters (0 bytes if unused)
  size_t app_ctx, app_ctx_lo;   // fused rows of a device-resident append (bf16 hi, lo)
  size_t fuse_y;                // fp32 projection of the fused rows before the norm
  size_t vcdf;                  // verify / sampling draws: merged row statistics and slice sums
  size_t sel_keys, sel_gpart, sel_spart, sel_S, sel_cand;  // candidate selector
  size_t conv_xh, conv_xl;      // the dynamic conv's hi/lo input rows
  size_t conv_h, conv_y, conv_ah, conv_al, conv_o, conv_corr_a, conv_corr_m;  // convs in the layers
  size_t total;
};

Layout make_layout(const dflash_config& c, int32_t max_seqs, int32_t max_tokens) {
  const size_t Mmax = (size_t)max_seqs * c.block_size;
  const size_t D = c.hidden, qd = (size_t)c.n_heads * c.head_dim, F = c.ffn;
  const size_t G = c.n_heads / c.n_kv_heads;
  const size_t lm_tiles = ((size_t)c.vocab + skinny_tile_cols() - 1) / skinny_tile_cols();
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.split_part = take(split_floats(c) * 4);
  L.x = take(Mmax * D * 4);
  L.xh = take(Mmax * D * 2);
  L.xl = take(Mmax * D * 2);
  L.ssq = take(Mmax * (D / 32) * 4);
  L.q = take(Mmax * qd * 2);
  L.q_lo = take(Mmax * qd * 2);
  L.blk_k = take(Mmax * c.n_kv_heads * c.head_dim * 4);
  L.blk_v = take(Mmax * c.n_kv_heads * c.head_dim * 4);
  L.ob_h = take(Mmax * qd * 2);
  L.ob_l = take(Mmax * qd * 2);
  L.act_h = take(Mmax * F * 2);
  L.act_l = take(Mmax * F * 2);
  L.lm_part = take(lm_tiles * Mmax * 8);
  const size_t slots = attn_slots(max_seqs, c.n_kv_heads);
  L.att_acc = take(slots * G * 16 * c.head_dim * 4);
  L.att_ml = take(slots * G * 16 * 2 * 4);
  L.vpart = take(2 * Mmax * kVerifyMaxSplits * 16);
  // per-row partial sums of y^2: 256-column tiles (tiled GEMM) or 32-column
  // groups (streaming path for few rows)
  L.fuse_ssq = take(std::max((size_t)max_tokens * ((D + kFuseTileN - 1) / kFuseTileN),
                             (size_t)std::min(max_tokens, kContextRowsStreaming) * (D / 32)) * 4);
  // the tiled context GEMMs run only for more rows than the streaming path takes
  const bool tiled = max_tokens > kContextRowsStreaming;
  L.gemm_part = take(tiled ? ctx_gemm_part_floats() * 4 : 0);
  L.gemm_ctr = take(tiled ? (size_t)kGemmMaxCounters * 4 : 0);
  L.app_ctx = take(std::min((size_t)max_tokens, Mmax) * D * 2);
  L.app_ctx_lo = take(std::min((size_t)max_tokens, Mmax) * D * 2);
  L.fuse_y = take((size_t)max_tokens * D * 4);
  L.vcdf = take(2 * Mmax * 16 + Mmax * kVerifyMaxSplits * 8);
  const size_t sel_rows = (size_t)max_seqs * (c.block_size > 1 ? c.block_size - 1 : 1);
  L.sel_keys = take(sel_rows * sel_slices(c.vocab) * kSelMaxK * 8);
  L.sel_gpart = take((size_t)sel_kz(c.hidden) * sel_rows * kSelMaxRank * 4);
  L.sel_spart = take((size_t)sel_kz(c.hidden) * sel_rows * 4);
  L.sel_S = take(sel_rows * kSelMaxK * kSelMaxK * 4);
  L.sel_cand = take(sel_rows * kSelMaxK * 4);
  L.conv_xh = take(Mmax * D * 2);
  L.conv_xl = take(Mmax * D * 2);
  L.conv_h = take(Mmax * D * 4);
  L.conv_y = take(Mmax * D * 4);
  L.conv_ah = take(Mmax * D * 2);
  L.conv_al = take(Mmax * D * 2);
  L.conv_o = take(Mmax * D * 4);
  L.conv_corr_a = take(Mmax * 2 * D * 4);  // 2 * D / group_size per row, any group size
  L.conv_corr_m = take(Mmax * 2 * D * 4);
  L.total = o;
  return L;
}

}  // namespace

enum Stage { ST_EMBED, ST_QKV, ST_ATTN, ST_OPROJ, ST_GATEUP, ST_DOWN, ST_LM, ST_FUSE, ST_INJECT,
             ST_VERIFY, ST_LM_ARGMAX, ST_SAMPLE, ST_SELECT, ST_CONV, ST_COUNT };
const char* kStageNames[ST_COUNT] = {"embed", "qkv", "attention", "o_proj", "gate_up",
                                     "down_proj", "lm_head", "fuse_context", "inject_kv", "verify",
                                     "lm_argmax", "sample_draft", "select", "conv"};

struct Profiler {
  uint32_t mask = 0;
  std::vector<hipEvent_t> ev;   // 2 per record
  std::vector<int32_t> stage;
  int32_t n = 0;
};

struct dflash_handle {
  Profiler prof;
  dflash_config cfg;
  dflash_weights w;
  std::vector<dflash_layer_weights> layers;
  hipStream_t stream = nullptr;
  unsigned char* ws = nullptr;
  size_t ws_bytes = 0;
  int32_t max_seqs = 0, max_tokens = 0;
  Layout lay{};
  dflash_selector sel{};         // candidate selector tables (rank 0: none)
  std::vector<dflash_conv_layer> conv;  // DFlash 2 convs of every layer (empty: none)
  int32_t conv_gs = 0;
};

// Launch `fn` as stage `st`, bracketed by timing events when that stage is
// being profiled.
template <class Fn>
static hipError_t timed(dflash_handle* h, int st, Fn&& fn) {
  Profiler& P = h->prof;
  const bool on = (P.mask >> st) & 1u && 2 * (size_t)(P.n + 1) <= P.ev.size();
  if (on) (void)hipEventRecord(P.ev[2 * P.n], h->stream);
  hipError_t e = fn();
  if (on) {
    (void)hipEventRecord(P.ev[2 * P.n + 1], h->stream);
    P.stage[P.n] = st;
    ++P.n;
  }
  return e;
}

static void profiler_release(Profiler& P) {
  for (hipEvent_t e : P.ev) (void)hipEventDestroy(e);
  P.ev.clear();
  P.stage.clear();
  P.n = 0;
  P.mask = 0;
}

static SplitWs split_ws(const dflash_handle* h) {
  SplitWs w;
  w.part = (float*)(h->ws + h->lay.split_part);
  w.part_floats = split_floats(h->cfg);
  return w;
}

static GemmWs gemm_ws(const dflash_handle* h) {
  GemmWs g{};
  if (h->max_tokens > kContextRowsStreaming) {
    g.part = (float*)(h->ws + h->lay.gemm_part);
    g.part_floats = ctx_gemm_part_floats();
    g.ctr = (int32_t*)(h->ws + h->lay.gemm_ctr);
    g.n_ctr = kGemmMaxCounters;
  }
  return g;
}

extern "C" {

dflash_status dflash_copy_bytes(void* dst, const void* src, size_t bytes, void* stream) {
  if (!bytes) return DFLASH_OK;
  if (!dst || !src) return fail(DFLASH_E_NULL, "copy: null pointer");
  if (((uintptr_t)dst | (uintptr_t)src | bytes) & 15)
    return fail(DFLASH_E_ALIGN, "copy: pointers and size must be multiples of 16 bytes");
  hipError_t e = launch_copy_bytes(dst, src, bytes, (hipStream_t)stream);
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "copy");
}

dflash_status dflash_read_bytes(const void* src, size_t bytes, void* sink, void* stream) {
  if (!bytes) return DFLASH_OK;
  if (!src || !sink) return fail(DFLASH_E_NULL, "read: null pointer");
  if (((uintptr_t)src & 15) || ((uintptr_t)sink & 3) || bytes % (128 * 1024))
    return fail(DFLASH_E_ALIGN, "read: src 16-byte aligned, sink 4-byte aligned, size a multiple of 128 KiB");
  hipError_t e = launch_read_bytes(src, bytes, (uint32_t*)sink, (hipStream_t)stream);
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "read");
}

const char* dflash_stage_name(int32_t stage) {
  return stage >= 0 && stage < ST_COUNT ? kStageNames[stage] : "unknown";
}

dflash_status dflash_profile_enable(dflash_handle* h, uint32_t stage_mask, int32_t max_records) {
  if (!h) return fail(DFLASH_E_NULL, "handle is NULL");
  if (stage_mask && (max_records < 1 || max_records > (1 << 20)))
    return fail(DFLASH_E_SHAPE, "max_records=%d outside 1..2^20", max_records);
  profiler_release(h->prof);
  if (!stage_mask) return DFLASH_OK;
  h->prof.ev.resize(2 * (size_t)max_records);
  for (size_t i = 0; i < h->prof.ev.size(); ++i) {
    hipError_t e = hipEventCreate(&h->prof.ev[i]);
    if (e != hipSuccess) {
      h->prof.ev.resize(i);
      profiler_release(h->prof);
      return dev_fail(e, "hipEventCreate");
    }
  }
  h->prof.stage.assign(max_records, -1);
  h->prof.mask = stage_mask;
  return DFLASH_OK;
}

dflash_status dflash_profile_read(dflash_handle* h, int32_t cap, int32_t* stage_out, float* ms_out,
                                  int32_t* n_out) {
  if (!h || !n_out) return fail(DFLASH_E_NULL, "handle and n_out are required");
  if (cap > 0 && (!stage_out || !ms_out)) return fail(DFLASH_E_NULL, "output arrays are required");
  Profiler& P = h->prof;
  const int32_t n = std::min(P.n, std::max(cap, 0));
  for (int32_t i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(P.ev[2 * i + 1]);
    if (e != hipSuccess) return dev_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, P.ev[2 * i], P.ev[2 * i + 1]);
    if (e != hipSuccess) return dev_fail(e, "hipEventElapsedTime");
    stage_out[i] = P.stage[i];
    ms_out[i] = ms;
  }
  *n_out = n;
  P.n = 0;
  return DFLASH_OK;
}

const char* dflash_status_str(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_E_NULL: return "null pointer";
    case DFLASH_E_CONFIG: return "invalid configuration";
    case DFLASH_E_SHAPE: return "size out of range";
    case DFLASH_E_CAPACITY: return "capacity exceeded";
    case DFLASH_E_ALIGN: return "misaligned pointer or stride";
    case DFLASH_E_DEVICE: return "device error";
    case DFLASH_E_STATE: return "invalid state";
  }
  return "unknown status";
}

const char* dflash_last_error(void) { return g_err.c_str(); }

dflash_status dflash_target_layer_ids(int32_t n_target_layers, int32_t n_feat, int32_t* out) {
  if (!out) return fail(DFLASH_E_NULL, "out is NULL");
  if (n_feat < 1 || n_target_layers < 4 || (n_feat > 1 && n_target_layers - 4 < n_feat - 1))
    return fail(DFLASH_E_SHAPE, "cannot pick %d distinct layers of %d", n_feat, n_target_layers);
  if (n_feat == 1) {
    out[0] = n_target_layers / 2;
    return DFLASH_OK;
  }
  const double lo = 1.0, hi = (double)(n_target_layers - 3);
  for (int i = 0; i < n_feat; ++i)
    out[i] = (int32_t)std::floor(lo + (hi - lo) * i / (n_feat - 1) + 0.5);
  return DFLASH_OK;
}

size_t dflash_kv_bytes(const dflash_config* cfg, int32_t max_ctx) {
  if (!cfg || max_ctx < 0) return 0;
  const dflash_config c = normalized(*cfg);
  if (check_config(c) != DFLASH_OK) return 0;
  return (size_t)c.n_layers * 2 * c.n_kv_heads * (size_t)row_capacity(c, max_ctx) * c.head_dim * 2;
}

int32_t dflash_kv_row_capacity(const dflash_config* cfg, int32_t max_ctx) {
  if (!cfg || max_ctx < 0) return 0;
  const dflash_config c = normalized(*cfg);
  if (check_config(c) != DFLASH_OK) return 0;
  return row_capacity(c, max_ctx);
}

size_t dflash_workspace_bytes(const dflash_config* cfg, int32_t max_seqs, int32_t max_tokens) {
  if (!cfg || max_seqs < 1 || max_seqs > kMaxSeqs || max_tokens < 0) return 0;
  const dflash_config c = normalized(*cfg);
  if (check_config(c) != DFLASH_OK) return 0;
  return make_layout(c, max_seqs, max_tokens).total;
}

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w, void* stream,
                            dflash_handle** out) {
  if (!cfg || !w || !out) return fail(DFLASH_E_NULL, "cfg, weights and out are required");
  const dflash_config c = normalized(*cfg);
  dflash_status st = check_config(c);
  if (st != DFLASH_OK) return st;
  const void* mats[] = {w->w_c, w->ctx_norm, w->embed, w->lm_head, w->final_norm};
  for (const void* p : mats) {
    if (!p) return fail(DFLASH_E_NULL, "a model-level weight pointer is NULL");
    if (!aligned(p, 16)) return fail(DFLASH_E_ALIGN, "weights must be 16-byte aligned");
  }
  if (!w->layers) return fail(DFLASH_E_NULL, "layers is NULL");
  for (int i = 0; i < c.n_layers; ++i) {
    const dflash_layer_weights& l = w->layers[i];
    const void* lp[] = {l.wq, l.wk, l.wv, l.wo, l.w_gate, l.w_up, l.w_down, l.attn_norm, l.mlp_norm};
    for (const void* p : lp) {
      if (!p) return fail(DFLASH_E_NULL, "layer %d has a NULL weight", i);
      if (!aligned(p, 16)) return fail(DFLASH_E_ALIGN, "layer %d weight not 16-byte aligned", i);
    }
  }
  dflash_handle* h = new dflash_handle();
  h->cfg = c;
  h->w = *w;
  h->layers.assign(w->layers, w->layers + c.n_layers);
  h->w.layers = h->layers.data();
  h->stream = (hipStream_t)stream;
  *out = h;
  return DFLASH_OK;
}

dflash_status dflash_destroy(dflash_handle* h) {
  if (!h) return fail(DFLASH_E_NULL, "handle is NULL");
  profiler_release(h->prof);
  delete h;
  return DFLASH_OK;
}

dflash_status dflash_set_stream(dflash_handle* h, void* stream) {
  if (!h) return fail(DFLASH_E_NULL, "handle is NULL");
  h->stream = (hipStream_t)stream;
  return DFLASH_OK;
}

dflash_status dflash_set_workspace(dflash_handle* h, void* ws, size_t bytes, int32_t max_seqs,
                                   int32_t max_tokens) {
  if (!h || !ws) return fail(DFLASH_E_NULL, "handle and workspace are required");
  if (!aligned(ws, 256)) return fail(DFLASH_E_ALIGN, "workspace must be 256-byte aligned");
  if (max_seqs < 1 || max_seqs > kMaxSeqs || max_tokens < 0)
    return fail(DFLASH_E_SHAPE, "max_seqs=%d outside 1..%d or max_tokens=%d < 0", max_seqs, kMaxSeqs, max_tokens);
  const Layout L = make_layout(h->cfg, max_seqs, max_tokens);
  if (bytes < L.total)
    return fail(DFLASH_E_CAPACITY, "workspace of %zu bytes, %zu needed", bytes, L.total);
  if (max_tokens > kContextRowsStreaming) {
    // the split-K arrival counters start at zero; every launch leaves them so
    hipError_t e = hipMemsetAsync((unsigned char*)ws + L.gemm_ctr, 0, (size_t)kGemmMaxCounters * 4,
                                  h->stream);
    if (e != hipSuccess) return dev_fail(e, "hipMemsetAsync");
  }
  h->ws = (unsigned char*)ws;
  h->ws_bytes = bytes;
  h->max_seqs = max_seqs;
  h->max_tokens = max_tokens;
  h->lay = L;
  return DFLASH_OK;
}

dflash_status dflash_fuse_context(dflash_handle* h, const void* const* feats, int64_t ld,
                                  int32_t n_tokens, void* ctx_out) {
  if (!h || !feats || !ctx_out) return fail(DFLASH_E_NULL, "handle, feats and ctx_out are required");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  const dflash_config& c = h->cfg;
  if (n_tokens < 1 || n_tokens > h->max_tokens)
    return fail(DFLASH_E_SHAPE, "n_tokens=%d outside 1..%d", n_tokens, h->max_tokens);
  if (ld < c.hidden || ld % 8) return fail(DFLASH_E_ALIGN, "ld=%lld must be >= hidden and a multiple of 8", (long long)ld);
  FuseLaunch F{};
  for (int i = 0; i < c.n_feat_layers; ++i) {
    if (!feats[i]) return fail(DFLASH_E_NULL, "feats[%d] is NULL", i);
    if (!aligned(feats[i], 16)) return fail(DFLASH_E_ALIGN, "feats[%d] not 16-byte aligned", i);
    F.feats[i] = (const bf16_t*)feats[i];
  }
  if (!aligned(ctx_out, 16)) return fail(DFLASH_E_ALIGN, "ctx_out not 16-byte aligned");
  F.n_feat = c.n_feat_layers;
  F.ld = ld;
  F.T = n_tokens;
  F.D = c.hidden;
  F.w_c = (const bf16_t*)h->w.w_c;
  F.gain = (const bf16_t*)h->w.ctx_norm;
  F.eps = c.rms_eps;
  F.out = (bf16_t*)ctx_out;
  F.ssq = (float*)(h->ws + h->lay.fuse_ssq);
  F.y = (float*)(h->ws + h->lay.fuse_y);
  F.split = split_ws(h);
  F.gemm = gemm_ws(h);
  const bool rows = n_tokens <= kContextRowsStreaming;
  hipError_t e = timed(h, ST_FUSE, [&] {
    return rows ? launch_fuse_rows(F, h->stream) : launch_fuse(F, h->stream);
  });
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "fuse_context");
}

static dflash_status check_kv(const dflash_handle* h, const dflash_kv* kv, const char* name) {
  if (!kv || !kv->base) return fail(DFLASH_E_NULL, "%s: kv or kv->base is NULL", name);
  if (!aligned(kv->base, 256)) return fail(DFLASH_E_ALIGN, "%s: kv->base not 256-byte aligned", name);
  if (kv->max_ctx < 0 || kv->len < 0 || kv->len > kv->max_ctx)
    return fail(DFLASH_E_SHAPE, "%s: len=%d max_ctx=%d", name, kv->len, kv->max_ctx);
  (void)h;
  return DFLASH_OK;
}

dflash_status dflash_inject_kv(dflash_handle* h, dflash_kv* kv, const void* ctx_feat,
                               int32_t n_tokens, int32_t pos0) {
  if (!h || !ctx_feat) return fail(DFLASH_E_NULL, "handle and ctx_feat are required");
  dflash_status st = check_kv(h, kv, "inject_kv");
  if (st != DFLASH_OK) return st;
  const dflash_config& c = h->cfg;
  if (n_tokens < 1 || n_tokens > h->max_tokens)
    return fail(DFLASH_E_SHAPE, "n_tokens=%d outside 1..%d", n_tokens, h->max_tokens);
  if (pos0 < 0 || pos0 > kv->len)
    return fail(DFLASH_E_SHAPE, "pos0=%d must lie in 0..len=%d", pos0, kv->len);
  if ((int64_t)pos0 + n_tokens > kv->max_ctx)
    return fail(DFLASH_E_CAPACITY, "pos0+n_tokens=%lld exceeds max_ctx=%d", (long long)pos0 + n_tokens, kv->max_ctx);
  if (!aligned(ctx_feat, 16)) return fail(DFLASH_E_ALIGN, "ctx_feat not 16-byte aligned");
  InjectLaunch I{};
  I.ctx = (const bf16_t*)ctx_feat;
  I.T = n_tokens; I.D = c.hidden; I.L = c.n_layers; I.Hkv = c.n_kv_heads; I.hd = c.head_dim;
  I.pos0 = pos0; I.cap = row_capacity(c, kv->max_ctx);
  I.log2_theta = std::log2((double)c.rope_theta);
  for (int i = 0; i < c.n_layers; ++i) {
    I.wk[i] = (const bf16_t*)h->layers[i].wk;
    I.wv[i] = (const bf16_t*)h->layers[i].wv;
  }
  I.kv = (bf16_t*)kv->base;
  I.split = split_ws(h);
  I.gemm = gemm_ws(h);
  const bool rows = n_tokens <= kContextRowsStreaming;
  hipError_t e = timed(h, ST_INJECT, [&] {
    return rows ? launch_inject_rows(I, h->stream) : launch_inject(I, h->stream);
  });
  if (e != hipSuccess) return dev_fail(e, "inject_kv");
  kv->len = pos0 + n_tokens;
  return DFLASH_OK;
}

dflash_status dflash_kv_trim(dflash_handle* h, dflash_kv* kv, int32_t keep_len) {
  if (!h) return fail(DFLASH_E_NULL, "handle is NULL");
  dflash_status st = check_kv(h, kv, "kv_trim");
  if (st != DFLASH_OK) return st;
  if (keep_len < 0 || keep_len > kv->len)
    return fail(DFLASH_E_SHAPE, "keep_len=%d must lie in 0..len=%d", keep_len, kv->len);
  kv->len = keep_len;
  return DFLASH_OK;
}

}  // extern "C"

// The draft forward; len_dev == NULL: the host lengths kvs[s]->len, else the
// device lengths len_dev[s] (attention is then planned for the buffers' full
// capacity, the kernels skip key ranges past the actual length).
static dflash_status draft_impl(dflash_handle* h, int32_t n_seqs, dflash_kv* const* kvs,
                                const int32_t* len_dev, const int32_t* anchor_ids,
                                int32_t block_len, int32_t* block_out, float* hidden_out,
                                float* logits_out) {
  if (!h || !kvs || !anchor_ids || !block_out)
    return fail(DFLASH_E_NULL, "handle, kvs, anchor_ids and block_out are required");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  const dflash_config& c = h->cfg;
  if (n_seqs < 1 || n_seqs > h->max_seqs)
    return fail(DFLASH_E_SHAPE, "n_seqs=%d outside 1..%d", n_seqs, h->max_seqs);
  if (block_len < 1 || block_len > c.block_size)
    return fail(DFLASH_E_SHAPE, "block_len=%d outside 1..%d", block_len, c.block_size);
  if ((hidden_out && !aligned(hidden_out, 4)) || (logits_out && !aligned(logits_out, 4)))
    return fail(DFLASH_E_ALIGN, "optional outputs must be 4-byte aligned");
  SeqTable seqs{};
  int max_keys = 0;
  for (int s = 0; s < n_seqs; ++s) {
    dflash_status st = check_kv(h, kvs[s], "draft_block");
    if (st != DFLASH_OK) return st;
    seqs.s[s].kv = (bf16_t*)kvs[s]->base;
    seqs.s[s].cap = row_capacity(c, kvs[s]->max_ctx);
    seqs.s[s].len = kvs[s]->len;
    seqs.s[s].max_ctx = kvs[s]->max_ctx;
    // context keys: the block's own keys are added by the merge kernel
    max_keys = std::max(max_keys, len_dev ? kvs[s]->max_ctx : kvs[s]->len);
  }
  seqs.len_dev = len_dev;
  const Layout& Ly = h->lay;
  unsigned char* ws = h->ws;
  DraftLaunch L{};
  L.M = n_seqs * block_len; L.n_seqs = n_seqs; L.Bl = block_len;
  L.D = c.hidden; L.Hq = c.n_heads; L.Hkv = c.n_kv_heads; L.hd = c.head_dim; L.F = c.ffn;
  L.V = c.vocab; L.mask_id = c.mask_token_id; L.eps = c.rms_eps;
  L.log2_theta = std::log2((double)c.rope_theta);
  L.embed = (const bf16_t*)h->w.embed;
  L.gain0 = (const bf16_t*)h->layers[0].attn_norm;
  L.anchors = anchor_ids; L.block_out = block_out; L.seqs = &seqs;
  L.x = (float*)(ws + Ly.x); L.xh = (bf16_t*)(ws + Ly.xh); L.xl = (bf16_t*)(ws + Ly.xl);
  L.ssq = (float*)(ws + Ly.ssq); L.q = (bf16_t*)(ws + Ly.q); L.q_lo = (bf16_t*)(ws + Ly.q_lo);
  L.blk_k = (float*)(ws + Ly.blk_k); L.blk_v = (float*)(ws + Ly.blk_v);
  L.ob_h = (bf16_t*)(ws + Ly.ob_h); L.ob_l = (bf16_t*)(ws + Ly.ob_l);
  L.act_h = (bf16_t*)(ws + Ly.act_h); L.act_l = (bf16_t*)(ws + Ly.act_l);
  L.lm_part = (uint64_t*)(ws + Ly.lm_part);
  L.att_acc = (float*)(ws + Ly.att_acc); L.att_ml = (float*)(ws + Ly.att_ml);
  L.split = split_ws(h);
  L.gemm = gemm_ws(h);
  const bool conv = !h->conv.empty();
  L.conv_gs = conv ? h->conv_gs : 0;
  L.conv_h = (float*)(ws + Ly.conv_h); L.conv_y = (float*)(ws + Ly.conv_y);
  L.conv_ah = (bf16_t*)(ws + Ly.conv_ah); L.conv_al = (bf16_t*)(ws + Ly.conv_al);
  L.conv_xh = (bf16_t*)(ws + Ly.conv_xh); L.conv_xl = (bf16_t*)(ws + Ly.conv_xl);
  L.conv_o = (float*)(ws + Ly.conv_o);
  L.conv_corr_a = (float*)(ws + Ly.conv_corr_a); L.conv_corr_m = (float*)(ws + Ly.conv_corr_m);
  // split each sequence's keys so that the grid holds ~1024 waves (one per
  // SIMD) where the context allows, in whole 32-key chunks; each workgroup
  // runs G query-head waves, times 2 key columns when G <= 2
  const int pairs = n_seqs * c.n_kv_heads;
  const int G = c.n_heads / c.n_kv_heads;
  const int WG_waves = G <= 2 ? 2 * G : G;
  const int max_splits =
      std::max(1, std::min(kAttnMaxSplits, attn_slots(h->max_seqs, c.n_kv_heads) / pairs - 1));
  // (the last split also takes the remainder); long key ranges are split further when the
  // grid is full already (many sequences), since a wave's chunks are serial
  int splits = std::max(1, (1024 + pairs * WG_waves - 1) / (pairs * WG_waves));
  splits = std::max(splits, (max_keys + kAttnMaxKeysPerSplit - 1) / kAttnMaxKeysPerSplit);
  splits = std::min(max_splits, splits);
  // at least two chunks per split: with one, the merge's extra splits cost
  // more than the shorter chains save (D = 2048: 64 splits of 32 keys ->
  // 32 of 64, merge 5.3 -> 4.4 us a layer)
  int kps = std::max(64, max_keys / splits / 32 * 32);
  if (max_keys / kps > max_splits) kps = (int)align_up((size_t)((max_keys + max_splits - 1) / max_splits), 32);
  // never more workgroups than the target: with device-resident lengths
  // max_keys covers the whole cache, and the last split absorbs the rest
  splits = std::max(1, std::min(splits, max_keys / kps));
  L.att_splits = splits; L.att_keys_per_split = kps;
  L.att_blk_wg = kps >= kAttnBlockWgKeys && (int64_t)splits * pairs > kAttnBlockWgMinWGs;

  hipStream_t st = h->stream;
  hipError_t e = timed(h, ST_EMBED, [&] { return launch_embed(L, st); });
  if (e != hipSuccess) return dev_fail(e, "embed");
  for (int i = 0; i < c.n_layers; ++i) {
    const dflash_layer_weights& lw = h->layers[i];
    const bf16_t* gnext = (const bf16_t*)(i + 1 < c.n_layers ? h->layers[i + 1].attn_norm
                                                              : h->w.final_norm);
    float* hid = hidden_out ? hidden_out + (size_t)i * L.M * c.hidden : nullptr;
    if (conv && conv_fused(L)) {
      // the layer with its two convs ([Code] sections 13-14), fused into the
      // GEMMs' finishers: prepare on the sublayer's normed input (the
      // projection's finisher forms the norm and the conv), finish on the
      // sublayer's output before the residual add (in its finisher)
      const dflash_conv_layer& cw = h->conv[i];
      e = timed(h, ST_CONV, [&] {
        return launch_conv_prepare_fused(L, (const bf16_t*)lw.attn_norm, (const bf16_t*)cw.attn_base,
                                         (const bf16_t*)cw.attn_proj, L.conv_corr_a, st);
      });
      if (e != hipSuccess) return dev_fail(e, "conv (attention, prepare)");
      e = timed(h, ST_QKV, [&] {
        return launch_qkv(L, i, (const bf16_t*)lw.wq, (const bf16_t*)lw.wk, (const bf16_t*)lw.wv, st,
                          L.conv_ah, L.conv_al);
      });
      if (e != hipSuccess) return dev_fail(e, "qkv");
      e = timed(h, ST_ATTN, [&] { return launch_attention(L, i, st); });
      if (e != hipSuccess) return dev_fail(e, "attention");
      e = timed(h, ST_OPROJ, [&] {
        return launch_conv_resid_fused(L, (const bf16_t*)lw.wo, L.ob_h, L.ob_l, c.n_heads * c.head_dim,
                                       (const bf16_t*)cw.attn_base, L.conv_corr_a,
                                       (const bf16_t*)lw.mlp_norm, nullptr, st);
      });
      if (e != hipSuccess) return dev_fail(e, "o_proj + conv finish");
      e = timed(h, ST_CONV, [&] {
        return launch_conv_prepare_fused(L, (const bf16_t*)lw.mlp_norm, (const bf16_t*)cw.mlp_base,
                                         (const bf16_t*)cw.mlp_proj, L.conv_corr_m, st);
      });
      if (e != hipSuccess) return dev_fail(e, "conv (MLP, prepare)");
      e = timed(h, ST_GATEUP, [&] {
        return launch_swiglu(L, (const bf16_t*)lw.w_gate, (const bf16_t*)lw.w_up, st, L.conv_ah,
                             L.conv_al);
      });
      if (e != hipSuccess) return dev_fail(e, "gate_up");
      e = timed(h, ST_DOWN, [&] {
        return launch_conv_resid_fused(L, (const bf16_t*)lw.w_down, L.act_h, L.act_l, c.ffn,
                                       (const bf16_t*)cw.mlp_base, L.conv_corr_m, gnext, hid, st);
      });
      if (e != hipSuccess) return dev_fail(e, "down_proj + conv finish");
      continue;
    }
    if (conv) {
      // the layer with its two convs ([Code] sections 13-14): prepare on the
      // sublayer's normed input, finish on its output before the residual add
      // (separate kernels: more rows than one tile)
      const dflash_conv_layer& cw = h->conv[i];
      e = timed(h, ST_CONV, [&] {
        hipError_t r = launch_norm_rows(L, (const bf16_t*)lw.attn_norm, st);
        return r != hipSuccess ? r
                               : launch_conv_prepare_draft(L, (const bf16_t*)cw.attn_base,
                                                           (const bf16_t*)cw.attn_proj, L.conv_corr_a, st);
      });
      if (e != hipSuccess) return dev_fail(e, "conv (attention, prepare)");
      e = timed(h, ST_QKV, [&] {
        return launch_qkv(L, i, (const bf16_t*)lw.wq, (const bf16_t*)lw.wk, (const bf16_t*)lw.wv, st,
                          L.conv_ah, L.conv_al);
      });
      if (e != hipSuccess) return dev_fail(e, "qkv");
      e = timed(h, ST_ATTN, [&] { return launch_attention(L, i, st); });
      if (e != hipSuccess) return dev_fail(e, "attention");
      e = timed(h, ST_OPROJ, [&] {
        return launch_store(L, (const bf16_t*)lw.wo, L.ob_h, L.ob_l, c.n_heads * c.head_dim, L.conv_o, st);
      });
      if (e != hipSuccess) return dev_fail(e, "o_proj");
      e = timed(h, ST_CONV, [&] {
        hipError_t r = launch_conv_finish_resid(L, (const bf16_t*)cw.attn_base, L.conv_corr_a,
                                                (const bf16_t*)lw.mlp_norm, nullptr, st);
        if (r != hipSuccess) return r;
        r = launch_norm_rows(L, (const bf16_t*)lw.mlp_norm, st);
        return r != hipSuccess ? r
                               : launch_conv_prepare_draft(L, (const bf16_t*)cw.mlp_base,
                                                           (const bf16_t*)cw.mlp_proj, L.conv_corr_m, st);
      });
      if (e != hipSuccess) return dev_fail(e, "conv (attention finish, MLP prepare)");
      e = timed(h, ST_GATEUP, [&] {
        return launch_swiglu(L, (const bf16_t*)lw.w_gate, (const bf16_t*)lw.w_up, st, L.conv_ah,
                             L.conv_al);
      });
      if (e != hipSuccess) return dev_fail(e, "gate_up");
      e = timed(h, ST_DOWN, [&] {
        return launch_store(L, (const bf16_t*)lw.w_down, L.act_h, L.act_l, c.ffn, L.conv_o, st);
      });
      if (e != hipSuccess) return dev_fail(e, "down_proj");
      e = timed(h, ST_CONV, [&] {
        return launch_conv_finish_resid(L, (const bf16_t*)cw.mlp_base, L.conv_corr_m, gnext, hid, st);
      });
      if (e != hipSuccess) return dev_fail(e, "conv (MLP finish)");
      continue;
    }
    e = timed(h, ST_QKV, [&] {
      return launch_qkv(L, i, (const bf16_t*)lw.wq, (const bf16_t*)lw.wk, (const bf16_t*)lw.wv, st);
    });
    if (e != hipSuccess) return dev_fail(e, "qkv");
    e = timed(h, ST_ATTN, [&] { return launch_attention(L, i, st); });
    if (e != hipSuccess) return dev_fail(e, "attention");
    e = timed(h, ST_OPROJ, [&] {
      return launch_resid(L, (const bf16_t*)lw.wo, L.ob_h, L.ob_l, c.n_heads * c.head_dim,
                          (const bf16_t*)lw.mlp_norm, nullptr, st);
    });
    if (e != hipSuccess) return dev_fail(e, "o_proj");
    e = timed(h, ST_GATEUP, [&] {
      return launch_swiglu(L, (const bf16_t*)lw.w_gate, (const bf16_t*)lw.w_up, st);
    });
    if (e != hipSuccess) return dev_fail(e, "gate_up");
    e = timed(h, ST_DOWN, [&] {
      return launch_resid(L, (const bf16_t*)lw.w_down, L.act_h, L.act_l, c.ffn, gnext, hid, st);
    });
    if (e != hipSuccess) return dev_fail(e, "down_proj");
  }
  if (block_len > 1) {
    e = timed(h, ST_LM, [&] { return launch_lm(L, (const bf16_t*)h->w.lm_head, logits_out, st); });
    if (e != hipSuccess) return dev_fail(e, "lm_head");
    e = timed(h, ST_LM_ARGMAX, [&] {
      return launch_lm_argmax(L, (const bf16_t*)h->w.lm_head, logits_out, st);
    });
    if (e != hipSuccess) return dev_fail(e, "lm_argmax");
  }
  return DFLASH_OK;
}

extern "C" {

dflash_status dflash_draft_block(dflash_handle* h, int32_t n_seqs, dflash_kv* const* kvs,
                                 const int32_t* anchor_ids, int32_t block_len, int32_t* block_out,
                                 float* hidden_out, float* logits_out) {
  return draft_impl(h, n_seqs, kvs, nullptr, anchor_ids, block_len, block_out, hidden_out,
                    logits_out);
}

dflash_status dflash_draft_block_dev(dflash_handle* h, int32_t n_seqs, dflash_kv* const* kvs,
                                     const int32_t* len_dev, const int32_t* anchor_ids,
                                     int32_t block_len, int32_t* block_out, float* hidden_out,
                                     float* logits_out) {
  if (!len_dev) return fail(DFLASH_E_NULL, "len_dev is required");
  if (!aligned(len_dev, 4)) return fail(DFLASH_E_ALIGN, "len_dev not 4-byte aligned");
  return draft_impl(h, n_seqs, kvs, len_dev, anchor_ids, block_len, block_out, hidden_out,
                    logits_out);
}

dflash_status dflash_append_dev(dflash_handle* h, int32_t n_seqs, dflash_kv* const* kvs,
                                int32_t* len_dev, const int32_t* tau_dev,
                                const void* const* feats, int64_t ld, int32_t rows_per_seq) {
  if (!h || !kvs || !len_dev || !tau_dev || !feats)
    return fail(DFLASH_E_NULL, "handle, kvs, len_dev, tau_dev and feats are required");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  const dflash_config& c = h->cfg;
  if (n_seqs < 1 || n_seqs > h->max_seqs)
    return fail(DFLASH_E_SHAPE, "n_seqs=%d outside 1..%d", n_seqs, h->max_seqs);
  if (rows_per_seq < 1 || rows_per_seq > c.block_size)
    return fail(DFLASH_E_SHAPE, "rows_per_seq=%d outside 1..%d", rows_per_seq, c.block_size);
  const int T = n_seqs * rows_per_seq;
  if (T > h->max_tokens)
    return fail(DFLASH_E_SHAPE, "n_seqs*rows_per_seq=%d exceeds max_tokens=%d", T, h->max_tokens);
  if (ld < c.hidden || ld % 8) return fail(DFLASH_E_ALIGN, "ld=%lld must be >= hidden and a multiple of 8", (long long)ld);
  if (!aligned(len_dev, 4) || !aligned(tau_dev, 4)) return fail(DFLASH_E_ALIGN, "len_dev/tau_dev not 4-byte aligned");
  FuseLaunch F{};
  for (int i = 0; i < c.n_feat_layers; ++i) {
    if (!feats[i]) return fail(DFLASH_E_NULL, "feats[%d] is NULL", i);
    if (!aligned(feats[i], 16)) return fail(DFLASH_E_ALIGN, "feats[%d] not 16-byte aligned", i);
    F.feats[i] = (const bf16_t*)feats[i];
  }
  SeqTable seqs{};
  for (int s = 0; s < n_seqs; ++s) {
    dflash_status st = check_kv(h, kvs[s], "append_dev");
    if (st != DFLASH_OK) return st;
    seqs.s[s].kv = (bf16_t*)kvs[s]->base;
    seqs.s[s].cap = row_capacity(c, kvs[s]->max_ctx);
    seqs.s[s].len = kvs[s]->len;
    seqs.s[s].max_ctx = kvs[s]->max_ctx;
  }
  seqs.len_dev = len_dev;
  // the fused rows stay a bf16 hi/lo pair (~16 significant bits) until the
  // injection: they never leave the call, and the injection's weight stream
  // is HBM-bound either way
  bf16_t* ctx = (bf16_t*)(h->ws + h->lay.app_ctx);
  bf16_t* ctx_lo = (bf16_t*)(h->ws + h->lay.app_ctx_lo);
  F.n_feat = c.n_feat_layers; F.ld = ld; F.T = T; F.D = c.hidden;
  F.w_c = (const bf16_t*)h->w.w_c; F.gain = (const bf16_t*)h->w.ctx_norm; F.eps = c.rms_eps;
  F.out = ctx; F.out_lo = ctx_lo; F.ssq = (float*)(h->ws + h->lay.fuse_ssq); F.y = (float*)(h->ws + h->lay.fuse_y);
  F.split = split_ws(h); F.gemm = gemm_ws(h);
  // few rows: the fusion's norm moves into the injection's epilogue (the row
  // scale commutes with the products), which saves the normalisation pass
  F.norm_in_consumer = T <= kContextRowsStreaming;
  AppendLaunch A{};
  A.ctx = ctx; A.ctx_lo = ctx_lo; A.T = T; A.rps = rows_per_seq; A.D = c.hidden; A.L = c.n_layers;
  A.Hkv = c.n_kv_heads; A.hd = c.head_dim; A.log2_theta = std::log2((double)c.rope_theta);
  for (int i = 0; i < c.n_layers; ++i) {
    A.wk[i] = (const bf16_t*)h->layers[i].wk;
    A.wv[i] = (const bf16_t*)h->layers[i].wv;
  }
  A.tau = tau_dev; A.seqs = &seqs; A.split = split_ws(h);
  if (F.norm_in_consumer) {
    A.ssq = F.ssq;
    A.eps = c.rms_eps;
  }
  hipStream_t st = h->stream;
  hipError_t e = timed(h, ST_FUSE, [&] {
    return T <= kContextRowsStreaming ? launch_fuse_rows(F, st) : launch_fuse(F, st);
  });
  if (e != hipSuccess) return dev_fail(e, "append_dev fuse");
  e = timed(h, ST_INJECT, [&] { return launch_append_inject(A, st); });
  if (e != hipSuccess) return dev_fail(e, "append_dev inject");
  e = launch_advance_len(len_dev, tau_dev, seqs, n_seqs, st);
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "append_dev lengths");
}

dflash_status dflash_kv_trim_dev(dflash_handle* h, int32_t n_seqs, int32_t* len_dev,
                                 int32_t keep_len) {
  if (!h || !len_dev) return fail(DFLASH_E_NULL, "handle and len_dev are required");
  if (n_seqs < 1 || n_seqs > kMaxSeqs) return fail(DFLASH_E_SHAPE, "n_seqs=%d outside 1..%d", n_seqs, kMaxSeqs);
  if (keep_len < 0) return fail(DFLASH_E_SHAPE, "keep_len=%d < 0", keep_len);
  if (!aligned(len_dev, 4)) return fail(DFLASH_E_ALIGN, "len_dev not 4-byte aligned");
  hipError_t e = launch_trim_len(len_dev, n_seqs, keep_len, h->stream);
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "kv_trim_dev");
}

}  // extern "C"

// The checks and launches of dflash_verify; the partials go to part / part2
// (max_rows rows of merged statistics, then the slice sums).
static dflash_status verify_impl(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                 const int32_t* block_ids, const float* target_logits,
                                 const float* draft_logits, float temperature, uint64_t seed,
                                 uint64_t philox_offset, int32_t* tau_out, int32_t* bonus_out,
                                 void* part, void* part2, int max_rows, int seq_cap,
                                 const char* name) {
  const dflash_config& c = h->cfg;
  if (n_seqs < 1 || n_seqs > seq_cap)
    return fail(DFLASH_E_SHAPE, "%s: n_seqs=%d outside 1..%d", name, n_seqs, seq_cap);
  if (block_len < 1 || block_len > c.block_size)
    return fail(DFLASH_E_SHAPE, "%s: block_len=%d outside 1..%d", name, block_len, c.block_size);
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(DFLASH_E_SHAPE, "%s: temperature must be finite and >= 0", name);
  const bool greedy = temperature == 0.f;
  if (!greedy && block_len > 1 && !draft_logits)
    return fail(DFLASH_E_NULL, "%s: draft_logits are required when temperature > 0", name);
  if (greedy && draft_logits)
    return fail(DFLASH_E_SHAPE, "%s: draft_logits must be NULL when temperature == 0", name);
  if (c.vocab % 4 == 0 && !aligned(target_logits, 16))
    return fail(DFLASH_E_ALIGN, "%s: target_logits not 16-byte aligned", name);
  const int rows = greedy ? n_seqs * block_len : n_seqs * (2 * block_len - 1);
  if (rows > max_rows)
    return fail(DFLASH_E_CAPACITY, "%s: %d verification rows exceed the scratch's %d", name, rows,
                max_rows);
  VerifyLaunch P{};
  P.n_seqs = n_seqs; P.Bl = block_len; P.V = c.vocab;
  P.block_ids = block_ids; P.target = target_logits; P.draft = draft_logits;
  P.temperature = (double)temperature; P.seed = seed; P.offset = philox_offset;
  P.tau = tau_out; P.bonus = bonus_out;
  P.part = part;
  P.part2 = part2;
  P.max_rows = max_rows;
  P.splits = std::max(1, std::min(kVerifyMaxSplits, (1024 + rows - 1) / rows));
  hipError_t e = timed(h, ST_VERIFY, [&] {
    return greedy ? launch_verify_greedy(P, h->stream) : launch_verify_pq(P, h->stream);
  });
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, name);
}

extern "C" {

dflash_status dflash_verify(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                            const int32_t* block_ids, const float* target_logits,
                            const float* draft_logits, float temperature, uint64_t seed,
                            uint64_t philox_offset, int32_t* tau_out, int32_t* bonus_out) {
  if (!h || !block_ids || !target_logits || !tau_out || !bonus_out)
    return fail(DFLASH_E_NULL, "handle, block_ids, target_logits, tau_out and bonus_out are required");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  return verify_impl(h, n_seqs, block_len, block_ids, target_logits, draft_logits, temperature,
                     seed, philox_offset, tau_out, bonus_out, h->ws + h->lay.vpart,
                     h->ws + h->lay.vcdf, 2 * h->max_seqs * h->cfg.block_size, h->max_seqs,
                     "verify");
}

dflash_status dflash_verify_noalloc(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                    const int32_t* block_ids, const float* target_logits,
                                    const float* draft_logits, float temperature, uint64_t seed,
                                    uint64_t philox_offset, int32_t* tau_out, int32_t* bonus_out) {
  if (!h || !block_ids || !target_logits || !tau_out || !bonus_out)
    return fail(DFLASH_E_NULL, "handle, block_ids, target_logits, tau_out and bonus_out are required");
  // the fixed scratch of the current device (its address is looked up on
  // the first call on each device and kept)
  void* scratch = nullptr;
  hipError_t e = verify_scratch_ptr(&scratch);
  if (e != hipSuccess) return dev_fail(e, "verify_noalloc: scratch address");
  unsigned char* base = static_cast<unsigned char*>(scratch);
  return verify_impl(h, n_seqs, block_len, block_ids, target_logits, draft_logits, temperature,
                     seed, philox_offset, tau_out, bonus_out, base, base + kVerifyScratchPart,
                     kVerifyScratchRows, kMaxSeqs, "verify_noalloc");
}

dflash_status dflash_verify_candidates(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                      const int32_t* block_ids, const float* target_logits,
                                      const int32_t* cand, const float* q_rows, int32_t top_k,
                                      float temperature, uint64_t seed, uint64_t philox_offset,
                                      int32_t* tau_out, int32_t* bonus_out) {
  if (!h || !block_ids || !target_logits || !tau_out || !bonus_out)
    return fail(DFLASH_E_NULL, "handle, block_ids, target_logits, tau_out and bonus_out are required");
  if (block_len > 1 && (!cand || !q_rows))
    return fail(DFLASH_E_NULL, "cand and q_rows are required when block_len > 1");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  const dflash_config& c = h->cfg;
  if (n_seqs < 1 || n_seqs > h->max_seqs)
    return fail(DFLASH_E_SHAPE, "n_seqs=%d outside 1..%d", n_seqs, h->max_seqs);
  if (block_len < 1 || block_len > c.block_size)
    return fail(DFLASH_E_SHAPE, "block_len=%d outside 1..%d", block_len, c.block_size);
  if (top_k < 1 || top_k > kSelMaxK)
    return fail(DFLASH_E_SHAPE, "top_k=%d outside 1..%d", top_k, kSelMaxK);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DFLASH_E_SHAPE, "temperature must be finite and > 0");
  if (c.vocab % 4 == 0 && !aligned(target_logits, 16))
    return fail(DFLASH_E_ALIGN, "target_logits not 16-byte aligned");
  if (!aligned(cand, 4) || !aligned(q_rows, 4) || !aligned(block_ids, 4))
    return fail(DFLASH_E_ALIGN, "cand, q_rows and block_ids must be 4-byte aligned");
  VerifyLaunch P{};
  P.n_seqs = n_seqs; P.Bl = block_len; P.V = c.vocab;
  P.block_ids = block_ids; P.target = target_logits;
  P.cand = cand; P.qc = q_rows; P.k = top_k;
  P.temperature = (double)temperature; P.seed = seed; P.offset = philox_offset;
  P.tau = tau_out; P.bonus = bonus_out;
  P.part = h->ws + h->lay.vpart;
  P.part2 = h->ws + h->lay.vcdf;
  P.max_rows = 2 * h->max_seqs * c.block_size;
  const int rows = n_seqs * block_len;
  P.splits = std::max(1, std::min(kVerifyMaxSplits, (1024 + rows - 1) / rows));
  hipError_t e = timed(h, ST_VERIFY, [&] { return launch_verify_pq_cand(P, h->stream); });
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "verify_candidates");
}

dflash_status dflash_sample_draft(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                  const float* draft_logits, float temperature, uint64_t seed,
                                  uint64_t philox_offset, int32_t* block_ids) {
  if (!h || !draft_logits || !block_ids)
    return fail(DFLASH_E_NULL, "handle, draft_logits and block_ids are required");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  const dflash_config& c = h->cfg;
  if (n_seqs < 1 || n_seqs > h->max_seqs)
    return fail(DFLASH_E_SHAPE, "n_seqs=%d outside 1..%d", n_seqs, h->max_seqs);
  if (block_len < 1 || block_len > c.block_size)
    return fail(DFLASH_E_SHAPE, "block_len=%d outside 1..%d", block_len, c.block_size);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DFLASH_E_SHAPE, "temperature must be finite and > 0 (use argmax drafting at 0)");
  if (block_len == 1) return DFLASH_OK;  // nothing drafted
  VerifyLaunch P{};
  P.n_seqs = n_seqs; P.Bl = block_len - 1; P.V = c.vocab;
  P.target = draft_logits; P.temperature = (double)temperature;
  P.seed = seed; P.offset = philox_offset;
  P.part = h->ws + h->lay.vpart;
  P.part2 = h->ws + h->lay.vcdf;
  P.max_rows = 2 * h->max_seqs * c.block_size;
  const int rows = n_seqs * (block_len - 1);
  P.splits = std::max(1, std::min(kVerifyMaxSplits, (1024 + rows - 1) / rows));
  hipError_t e = timed(h, ST_SAMPLE, [&] {
    return launch_sample_draft(P, block_ids, block_len, h->stream);
  });
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "sample_draft");
}

dflash_status dflash_set_selector(dflash_handle* h, const dflash_selector* sel) {
  if (!h) return fail(DFLASH_E_NULL, "handle is required");
  if (!sel) {
    h->sel = dflash_selector{};
    return DFLASH_OK;
  }
  if (!sel->hidden_proj || !sel->pred_codebook || !sel->succ_codebook)
    return fail(DFLASH_E_NULL, "hidden_proj, pred_codebook and succ_codebook are required");
  if (sel->top_k < 1 || sel->top_k > kSelMaxK || sel->top_k > h->cfg.vocab)
    return fail(DFLASH_E_SHAPE, "top_k=%d outside 1..%d (and at most the vocabulary)", sel->top_k,
                kSelMaxK);
  if (sel->rank < 64 || sel->rank > kSelMaxRank || sel->rank % 64)
    return fail(DFLASH_E_SHAPE, "rank=%d: 64..%d in steps of 64", sel->rank, kSelMaxRank);
  if (sel_slices(h->cfg.vocab) > sel_max_slices())
    return fail(DFLASH_E_SHAPE, "vocab=%d exceeds the selector's %d vocab slices", h->cfg.vocab,
                sel_max_slices());
  if (h->cfg.hidden % 64)
    return fail(DFLASH_E_SHAPE, "the selector needs hidden %% 64 == 0 (hidden=%d)", h->cfg.hidden);
  if (!aligned(sel->hidden_proj, 16) || !aligned(sel->pred_codebook, 16) ||
      !aligned(sel->succ_codebook, 16))
    return fail(DFLASH_E_ALIGN, "selector tables must be 16-byte aligned");
  h->sel = *sel;
  return DFLASH_OK;
}

dflash_status dflash_set_conv(dflash_handle* h, const dflash_conv_layer* layers, int32_t group_size) {
  if (!h) return fail(DFLASH_E_NULL, "handle is required");
  if (!layers) {
    h->conv.clear();
    h->conv_gs = 0;
    return DFLASH_OK;
  }
  const dflash_config& c = h->cfg;
  if (group_size < 1 || c.hidden % (16 * group_size))
    return fail(DFLASH_E_SHAPE, "group_size=%d: hidden=%d must be a multiple of 16 * group_size",
                group_size, c.hidden);
  for (int i = 0; i < c.n_layers; ++i) {
    const dflash_conv_layer& l = layers[i];
    const void* ps[] = {l.attn_base, l.attn_proj, l.mlp_base, l.mlp_proj};
    for (const void* p : ps) {
      if (!p) return fail(DFLASH_E_NULL, "conv layer %d has a NULL table", i);
      if (!aligned(p, 16)) return fail(DFLASH_E_ALIGN, "conv layer %d table not 16-byte aligned", i);
    }
  }
  h->conv.assign(layers, layers + c.n_layers);
  h->conv_gs = group_size;
  return DFLASH_OK;
}

dflash_status dflash_select_block(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                  const float* last_hidden, const float* draft_logits,
                                  const int32_t* anchor_ids, float temperature, uint64_t seed,
                                  uint64_t philox_offset, int32_t* block_ids, int32_t* cand_out,
                                  float* q_out) {
  if (!h || !last_hidden || !draft_logits || !anchor_ids || !block_ids)
    return fail(DFLASH_E_NULL, "handle, last_hidden, draft_logits, anchor_ids and block_ids are required");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  if (!h->sel.rank) return fail(DFLASH_E_STATE, "no selector set (dflash_set_selector)");
  const dflash_config& c = h->cfg;
  if (n_seqs < 1 || n_seqs > h->max_seqs)
    return fail(DFLASH_E_SHAPE, "n_seqs=%d outside 1..%d", n_seqs, h->max_seqs);
  if (block_len < 1 || block_len > c.block_size)
    return fail(DFLASH_E_SHAPE, "block_len=%d outside 1..%d", block_len, c.block_size);
  if (block_len - 1 > sel_max_walk_rows())
    return fail(DFLASH_E_SHAPE, "block_len-1=%d exceeds the selector's %d rows", block_len - 1,
                sel_max_walk_rows());
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(DFLASH_E_SHAPE, "temperature must be finite and >= 0");
  if (!aligned(last_hidden, 16) || !aligned(draft_logits, 4) || !aligned(anchor_ids, 4) ||
      !aligned(block_ids, 4) || !aligned(cand_out, 4) || !aligned(q_out, 4))
    return fail(DFLASH_E_ALIGN, "last_hidden must be 16-byte aligned, the other arrays 4-byte");
  if (block_len == 1) return DFLASH_OK;  // nothing drafted
  SelectLaunch L{};
  L.n_seqs = n_seqs; L.Bl = block_len; L.P = block_len - 1;
  L.V = c.vocab; L.D = c.hidden; L.k = h->sel.top_k; L.rank = h->sel.rank; L.eps = c.rms_eps;
  L.logits = draft_logits; L.last_hidden = last_hidden;
  L.gain = (const bf16_t*)h->w.final_norm;
  L.w_proj = (const bf16_t*)h->sel.hidden_proj;
  L.pred = (const bf16_t*)h->sel.pred_codebook;
  L.succ = (const bf16_t*)h->sel.succ_codebook;
  L.anchors = anchor_ids;
  L.temperature = (double)temperature; L.seed = seed; L.offset = philox_offset;
  L.block = block_ids; L.cand_out = cand_out; L.q_out = q_out;
  L.keys = (uint64_t*)(h->ws + h->lay.sel_keys);
  L.gpart = (float*)(h->ws + h->lay.sel_gpart);
  L.spart = (float*)(h->ws + h->lay.sel_spart);
  L.S = (float*)(h->ws + h->lay.sel_S);
  L.cand = (int32_t*)(h->ws + h->lay.sel_cand);
  hipError_t e = timed(h, ST_SELECT, [&] { return launch_select(L, h->stream); });
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "select_block");
}

}  // extern "C"

namespace {
dflash_status conv_check(dflash_handle* h, int32_t n_seqs, int32_t block_len, int32_t group_size,
                         const void* base, const float* x, const float* prev, const float* corr,
                         const float* y) {
  if (!h || !base || !x || !prev || !corr || !y)
    return fail(DFLASH_E_NULL, "handle, base, inputs, prev, corrections and y are required");
  if (!h->ws) return fail(DFLASH_E_STATE, "no workspace set");
  const dflash_config& c = h->cfg;
  if (n_seqs < 1 || n_seqs > h->max_seqs)
    return fail(DFLASH_E_SHAPE, "n_seqs=%d outside 1..%d", n_seqs, h->max_seqs);
  if (block_len < 1 || block_len > c.block_size)
    return fail(DFLASH_E_SHAPE, "block_len=%d outside 1..%d", block_len, c.block_size);
  if (group_size < 1 || c.hidden % (16 * group_size))
    return fail(DFLASH_E_SHAPE, "group_size=%d: hidden=%d must be a multiple of 16 * group_size",
                group_size, c.hidden);
  if (!aligned(base, 16) || !aligned(x, 16) || !aligned(prev, 4) || !aligned(corr, 4) ||
      !aligned(y, 4))
    return fail(DFLASH_E_ALIGN, "base and the input rows must be 16-byte aligned, the rest 4-byte");
  const size_t rows = (size_t)n_seqs * block_len, D = c.hidden, G = D / group_size;
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
  };
  const size_t ny = rows * D * 4;
  if (overlap(y, ny, x, ny) || overlap(y, ny, prev, (size_t)n_seqs * D * 4) ||
      overlap(y, ny, corr, rows * 2 * G * 4))
    return fail(DFLASH_E_SHAPE, "y must not overlap the inputs or the corrections");
  return DFLASH_OK;
}
}  // namespace

extern "C" {

dflash_status dflash_conv_prepare(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                  int32_t group_size, const void* base, const void* proj,
                                  const float* x, const float* prev, float* y, float* corr_out) {
  if (!proj) return fail(DFLASH_E_NULL, "proj is required");
  dflash_status st = conv_check(h, n_seqs, block_len, group_size, base, x, prev, corr_out, y);
  if (st != DFLASH_OK) return st;
  if (!aligned(proj, 16)) return fail(DFLASH_E_ALIGN, "proj must be 16-byte aligned");
  const size_t rows = (size_t)n_seqs * block_len, D = h->cfg.hidden;
  if ((uintptr_t)corr_out < (uintptr_t)x + rows * D * 4 &&
      (uintptr_t)x < (uintptr_t)corr_out + rows * 2 * (D / group_size) * 4)
    return fail(DFLASH_E_SHAPE, "corr_out must not overlap x");
  ConvLaunch C{};
  C.n_seqs = n_seqs; C.Bl = block_len; C.D = (int)D; C.gs = group_size;
  C.base = (const bf16_t*)base; C.proj = (const bf16_t*)proj;
  C.x = x; C.prev = prev; C.y = y; C.corr = corr_out;
  C.xh = (bf16_t*)(h->ws + h->lay.conv_xh);
  C.xl = (bf16_t*)(h->ws + h->lay.conv_xl);
  C.split = split_ws(h);
  hipError_t e = timed(h, ST_CONV, [&] { return launch_conv_prepare(C, h->stream); });
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "conv_prepare");
}

dflash_status dflash_conv_finish(dflash_handle* h, int32_t n_seqs, int32_t block_len,
                                 int32_t group_size, const void* base, const float* z,
                                 const float* prev, const float* corr, float* y) {
  dflash_status st = conv_check(h, n_seqs, block_len, group_size, base, z, prev, corr, y);
  if (st != DFLASH_OK) return st;
  ConvLaunch C{};
  C.n_seqs = n_seqs; C.Bl = block_len; C.D = h->cfg.hidden; C.gs = group_size;
  C.base = (const bf16_t*)base; C.x = z; C.prev = prev; C.y = y; C.corr = (float*)corr;
  hipError_t e = timed(h, ST_CONV, [&] { return launch_conv_finish(C, h->stream); });
  return e == hipSuccess ? DFLASH_OK : dev_fail(e, "conv_finish");
}

}  // extern "C"
