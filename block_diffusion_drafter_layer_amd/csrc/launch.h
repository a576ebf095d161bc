// Internal launch interface between the host ABI (api.cpp) and the kernels.
// Every launcher only enqueues on the given stream and returns the launch
// status; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dfl {

constexpr int kMaxLayers = 16;
constexpr int kMaxFeat = 8;
constexpr int kAttnMaxSplits = 128;
constexpr int kAttnSlotCap = 1024;   // (sequence, kv head, split) partial slots, at least
// slots per (sequence, kv head) the workspace keeps: up to 8 context splits
// and the block's own keys
constexpr int kAttnMinSplitsPerPair = 9;
constexpr int kAttnMaxKeysPerSplit = 512; // longer key ranges are split when slots allow
// The block's own keys get a workgroup of their own per (sequence, kv head)
// when the splits hold at least kAttnBlockWgKeys keys and the context's
// workgroups already fill more than a round of the GPU (kAttnBlockWgMinWGs:
// two per CU); otherwise the extra workgroups would share CUs with context
// splits and lengthen the launch, and the merge takes the block keys.
constexpr int kAttnBlockWgKeys = 128;
constexpr int kAttnBlockWgMinWGs = 512;
inline int attn_slots(int max_seqs, int n_kv_heads) {
  const int s = max_seqs * n_kv_heads * kAttnMinSplitsPerPair;
  return s > kAttnSlotCap ? s : kAttnSlotCap;
}
constexpr int kVerifyMaxSplits = 64;
constexpr int kFuseTileN = 256;     // output columns per fusion GEMM tile
constexpr int kGemmMaxSplit = 4;    // workgroups sharing one context-GEMM tile
constexpr int kGemmMaxCounters = 1024;
constexpr int kTiledK = 64;        // k per stage of the tiled MFMA GEMM (K must be a multiple)

// Split-K scratch of the context GEMMs: fp32 partial tiles and the tiles'
// arrival counters (zero between launches).
struct GemmWs {
  float* part;
  size_t part_floats;
  int32_t* ctr;
  int n_ctr;
};
size_t ctx_gemm_part_floats();

// Split-K scratch of the streaming GEMMs: fp32 partial tiles.
constexpr int kSplitMaxWG = 1024;     // capacity: partial tiles of <= 32 x 64
constexpr int kSplitTargetWG = 512;   // split narrow matrices up to this grid
struct SplitWs {
  float* part;
  size_t part_floats;
};

// Workspace pointers and shapes of one draft forward.
struct DraftLaunch {
  int M, n_seqs, Bl;
  int D, Hq, Hkv, hd, F, V, mask_id;
  float eps;
  double log2_theta;
  const bf16_t* embed;
  const bf16_t* gain0;      // attn_norm of layer 0
  const int32_t* anchors;
  int32_t* block_out;
  const SeqTable* seqs;
  // workspace
  float* x;                 // [M][D]
  bf16_t *xh, *xl;          // [M][D]
  float* ssq;               // [M][D/32]
  bf16_t *q, *q_lo;         // [M][Hq*hd] query after RoPE, hi/lo
  float *blk_k, *blk_v;     // [M][Hkv*hd] the block's own K (after RoPE) and V, fp32
  bf16_t *ob_h, *ob_l;      // [M][Hq*hd]
  bf16_t *act_h, *act_l;    // [M][F]
  uint64_t* lm_part;        // [ceil(V/32)][M] argmax keys per column block and row
  float* att_acc;           // [slots*G][16][hd]
  float* att_ml;            // [slots*G][16][2]
  int att_splits, att_keys_per_split;
  bool att_blk_wg;          // a workgroup of its own for the block's keys (else the merge)
  SplitWs split;
  GemmWs gemm;              // the tiled GEMM's split-K scratch (batches of more than 64 rows)
  // DFlash 2 convs in every layer (conv_gs == 0: none)
  int conv_gs;
  float* conv_h;            // [M][D] a sublayer's normed input
  float* conv_y;            // [M][D] its conv (prepare call)
  bf16_t *conv_ah, *conv_al;  // [M][D] conv_y as the sublayer GEMM's hi/lo input
  bf16_t *conv_xh, *conv_xl;  // [M][D] split scratch of the prepare projection
  float* conv_o;            // [M][D] a sublayer's output before the finish call
  float *conv_corr_a, *conv_corr_m;  // [M][2 * D / conv_gs] finish corrections
};

int skinny_tile_cols();
int skinny_max_rows();
// split-buffer floats the LDS-staged streaming GEMM needs for [rows<=16] x [K] -> [n_vcols]
size_t stream_part_floats(int n_vcols, int K);

hipError_t launch_embed(const DraftLaunch& L, hipStream_t st);
// ah/al: the layer's input rows as a bf16 hi/lo pair with no norm to apply
// (the conv's output); null: the residual's next-norm input and its row scale
hipError_t launch_qkv(const DraftLaunch& L, int layer, const bf16_t* wq,
                      const bf16_t* wk, const bf16_t* wv, hipStream_t st,
                      const bf16_t* ah = nullptr, const bf16_t* al = nullptr);
hipError_t launch_attention(const DraftLaunch& L, int layer, hipStream_t st);
hipError_t launch_resid(const DraftLaunch& L, const bf16_t* w, const bf16_t* ah,
                        const bf16_t* al, int K, const bf16_t* gain_next,
                        float* hidden, hipStream_t st);
hipError_t launch_swiglu(const DraftLaunch& L, const bf16_t* wg, const bf16_t* wu,
                         hipStream_t st, const bf16_t* ah = nullptr, const bf16_t* al = nullptr);
// DFlash 2 convs in the layer: the fp32 norm of the residual rows into conv_h,
// the prepare call on conv_h (conv_y, its hi/lo copy, the finish corrections
// into corr), the plain product into out, and the finish call + residual add
// + next-norm input
hipError_t launch_norm_rows(const DraftLaunch& L, const bf16_t* gain, hipStream_t st);
hipError_t launch_conv_prepare_draft(const DraftLaunch& L, const bf16_t* base, const bf16_t* proj,
                                     float* corr, hipStream_t st);
hipError_t launch_store(const DraftLaunch& L, const bf16_t* w, const bf16_t* ah, const bf16_t* al,
                        int K, float* out, hipStream_t st);
hipError_t launch_conv_finish_resid(const DraftLaunch& L, const bf16_t* base, const float* corr,
                                    const bf16_t* gain_next, float* hidden, hipStream_t st);
// the same two steps fused into the GEMMs' finishers, when every row fits one
// 16-row tile: the prepare call's projection with the norm and the conv in its
// finisher (the conv output straight to conv_ah / conv_al), and the
// sublayer's output product with the finish call and the residual add in its
// finisher
bool conv_fused(const DraftLaunch& L);
hipError_t launch_conv_prepare_fused(const DraftLaunch& L, const bf16_t* gain, const bf16_t* base,
                                     const bf16_t* proj, float* corr, hipStream_t st);
hipError_t launch_conv_resid_fused(const DraftLaunch& L, const bf16_t* w, const bf16_t* ah,
                                   const bf16_t* al, int K, const bf16_t* base, const float* corr,
                                   const bf16_t* gain_next, float* hidden, hipStream_t st);
hipError_t launch_lm(const DraftLaunch& L, const bf16_t* w_lm, float* logits,
                     hipStream_t st);
// drafted tokens from the LM head's output (split sums, logits, argmax)
hipError_t launch_lm_argmax(const DraftLaunch& L, const bf16_t* w_lm, float* logits,
                            hipStream_t st);

// Context fusion: y = [f_0 .. f_{n-1}] W_c^T (bf16 into out), then RMSNorm.
struct FuseLaunch {
  const bf16_t* feats[kMaxFeat];
  int n_feat;
  int64_t ld;
  int T, D;
  const bf16_t* w_c;
  const bf16_t* gain;
  float eps;
  bf16_t* out;        // [T][D] H_t, the one rounding to bf16
  bf16_t* out_lo;     // optional [T][D]: H_t - out rounded to bf16 (out then is the hi half)
  float* y;           // [T][D] fp32 projection before the norm (workspace)
  float* ssq;         // [T][ceil(D/256)] (tiled) or [T][D/32] (few rows)
  SplitWs split;
  GemmWs gemm;
  // few rows only: leave the norm to the consumer - out/out_lo receive the
  // bf16 hi/lo halves of y * gain (not normalised) and ssq the per-32-column
  // sums of y^2, from which the consumer's epilogue applies the row scale
  bool norm_in_consumer = false;
};
hipError_t launch_fuse(const FuseLaunch& F, hipStream_t st);        // tiled MFMA GEMM
hipError_t launch_fuse_rows(const FuseLaunch& F, hipStream_t st);   // few rows: streaming
hipError_t launch_fuse_normalize(bf16_t* out, bf16_t* out_lo, const float* y, const float* ssq,
                                 int n_parts, int T, int D, const bf16_t* gain, float eps,
                                 hipStream_t st);

// KV injection of T context rows at positions pos0.. into every layer.
struct InjectLaunch {
  const bf16_t* ctx;  // [T][D]
  int T, D, L, Hkv, hd, pos0, cap;
  double log2_theta;
  const bf16_t* wk[kMaxLayers];
  const bf16_t* wv[kMaxLayers];
  bf16_t* kv;
  SplitWs split;
  GemmWs gemm;
};
hipError_t launch_inject(const InjectLaunch& I, hipStream_t st);       // tiled MFMA GEMM
hipError_t launch_inject_rows(const InjectLaunch& I, hipStream_t st);  // few rows: streaming
constexpr int kContextRowsStreaming = 64;  // row counts up to this use the streaming kernels

// Device-resident rounds: fused accepted rows of several sequences injected
// at their device lengths, then the lengths advanced by tau.
struct AppendLaunch {
  const bf16_t* ctx;   // [T][D] fused rows, sequence s at rows s*rps .. (bf16 hi)
  const bf16_t* ctx_lo;  // [T][D] their lo halves
  int T, rps, D, L, Hkv, hd;
  double log2_theta;
  const bf16_t* wk[kMaxLayers];
  const bf16_t* wv[kMaxLayers];
  const int32_t* tau;  // [n_seqs] device
  const SeqTable* seqs;  // kv bases, capacities, len_dev
  SplitWs split;
  const float* ssq = nullptr;  // optional [T][D/32] sums of y^2: ctx holds y * gain, not yet normalised
  float eps = 0.f;
};
hipError_t launch_append_inject(const AppendLaunch& A, hipStream_t st);
// len[s] = min(len[s] + tau[s], max_ctx[s]) for s < n_seqs
hipError_t launch_advance_len(int32_t* len, const int32_t* tau, const SeqTable& seqs, int n_seqs,
                              hipStream_t st);
// len[s] = min(len[s], keep) for s < n
hipError_t launch_trim_len(int32_t* len, int n, int32_t keep, hipStream_t st);

// Verification.
struct VerifyLaunch {
  int n_seqs, Bl, V;
  const int32_t* block_ids;
  const float* target;
  const float* draft;
  double temperature;
  uint64_t seed, offset;
  int32_t *tau, *bonus;
  void* part;          // workspace for per-split partials
  int splits;
  void* part2;         // merged row statistics [max_rows] then slice sums [max_rows / 2][splits]
  int max_rows;
  // draft distribution on candidate sets (instead of draft logits): row
  // s * (Bl - 1) + j holds k candidates and their probabilities
  const int32_t* cand;
  const float* qc;
  int k;
};
hipError_t launch_verify_greedy(const VerifyLaunch& P, hipStream_t st);
// Fixed verification scratch for callers without a workspace: row partials
// of up to kVerifyScratchRows rows x kVerifyMaxSplits splits (16 B each),
// kVerifyScratchRows merged row statistics (16 B) and kVerifyScratchRows / 2
// x kVerifyMaxSplits slice sums (8 B). verify_scratch_ptr returns the
// current device's copy (looked up once per device).
constexpr int kVerifyScratchRows = 2048;
constexpr size_t kVerifyScratchPart = (size_t)kVerifyScratchRows * kVerifyMaxSplits * 16;
constexpr size_t kVerifyScratchBytes =
    kVerifyScratchPart + (size_t)kVerifyScratchRows * 16 + (size_t)kVerifyScratchRows / 2 * kVerifyMaxSplits * 8;
constexpr int kVerifyScratchDevices = 64;
hipError_t verify_scratch_ptr(void** out);
hipError_t launch_verify_pq(const VerifyLaunch& P, hipStream_t st);
// p/q with P.cand / P.qc (P.draft unused)
hipError_t launch_verify_pq_cand(const VerifyLaunch& P, hipStream_t st);
// draft tokens sampled from softmax(rows / T): P.target = the draft logits,
// P.n_seqs * P.Bl rows (P.Bl = drafted rows per sequence); writes
// block[s * Bl + 1 + j]
hipError_t launch_sample_draft(const VerifyLaunch& P, int32_t* block, int Bl, hipStream_t st);

// DFlash 2 candidate selector over drafted blocks.
constexpr int kSelMaxK = 16;       // candidates per row
constexpr int kSelMaxRank = 256;   // code width
struct SelectLaunch {
  int n_seqs, Bl, P;               // P = Bl - 1 drafted rows per sequence
  int V, D, k, rank;
  float eps;
  const float* logits;             // [n_seqs * P][V]
  const float* last_hidden;        // [n_seqs * Bl][D] residual after the last layer
  const bf16_t* gain;              // final norm gain [D]
  const bf16_t* w_proj;            // [rank][D]
  const bf16_t* pred;              // [V][rank]
  const bf16_t* succ;              // [V][rank]
  const int32_t* anchors;          // [n_seqs]
  double temperature;
  uint64_t seed, offset;
  int32_t* block;                  // [n_seqs][Bl], columns 1..
  int32_t* cand_out;               // optional [n_seqs * P][k]
  float* q_out;                    // optional [n_seqs * P][k]
  // workspace
  uint64_t* keys;                  // [rows][slices][k]
  float* gpart;                    // [kz][rows][rank]
  float* spart;                    // [kz][rows]
  float* S;                        // [rows][16][16]
  int32_t* cand;                   // [rows][16]
};
int sel_slices(int V);
int sel_kz(int D);
int sel_max_walk_rows();
int sel_max_slices();
hipError_t launch_select(const SelectLaunch& L, hipStream_t st);

// DFlash 2 grouped dynamic two-tap conv over n_seqs blocks of Bl rows.
struct ConvLaunch {
  int n_seqs, Bl, D, gs;
  const bf16_t* base;   // [2][2][D]
  const bf16_t* proj;   // [4 * D / gs][D] (prepare only)
  const float* x;       // [n_seqs * Bl][D] input (z for the finish call)
  const float* prev;    // [n_seqs][D]
  float* y;             // [n_seqs * Bl][D]
  float* corr;          // [n_seqs * Bl][2 * D / gs]: written by prepare, read by finish
  bf16_t *xh, *xl;      // workspace [n_seqs * Bl][D] (prepare only)
  SplitWs split;
};
hipError_t launch_conv_prepare(const ConvLaunch& C, hipStream_t st);
hipError_t launch_conv_finish(const ConvLaunch& C, hipStream_t st);

// reference copy for byte-counter calibration (16-byte aligned, bytes % 16 == 0)
hipError_t launch_copy_bytes(void* dst, const void* src, size_t bytes, hipStream_t st);
// read-ceiling reference: reads bytes (a multiple of 128 KiB, 16-byte
// aligned) in the weight streams' access pattern; sink: >= 256 words
hipError_t launch_read_bytes(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace dfl
