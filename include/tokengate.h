/*
 * tokengate.h -- C ABI of the TokenGate gated-prefill library (MI355X, gfx950).
 *
 * The library implements the inference hot path of TokenGate ("TokenGate:
 * Adapting LLMs for Fast and Memory-Efficient Prefill with Learned Token
 * Pruning", Section 4): at gate layer L every prunable token is scored by a
 * small MLP over its RMS-normalised post-attention residual, the scores are
 * RMS-normalised along the sequence, the top-K prunable tokens plus every
 * non-prunable token are kept, the residual stream is compacted to the kept
 * set, and the layers above L run token-gated causal GQA attention whose
 * logits carry each kept key's score through a per-head gain and a
 * temperature.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them.  Tensors are dense, row-major and
 *    contiguous in the order the shapes are written.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL means the default stream).  Nothing synchronises and nothing is
 *    copied device -> host.
 *  - Return value: TG_OK (0) or a tg_status code.  Arguments are validated
 *    before anything is enqueued; on any error nothing is enqueued and
 *    tg_last_error() describes the problem.  No C++ exception crosses the ABI.
 *  - Results are deterministic: the same inputs give the same output bits.
 *  - Batch rows are independent; every batch row has the same N, r and K,
 *    except in the _varlen entry points, which take per-row values.
 *  - The non-prunable tokens (the question x_R of the prompt x = [x_R, x_D])
 *    are the first r tokens of each sequence; tokens r..N-1 are prunable.
 *    The _span entry points take the prunable span [span_begin, span_end)
 *    instead, with non-prunable text on both sides.
 *  - Sizes and the cu_seqlens offsets of the attention _varlen entry points
 *    are host values; every tensor is a device pointer.
 *  - bf16 is IEEE bfloat16 stored in 16 bits; fp32 is IEEE binary32.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TG_OK = 0,
  TG_EINVAL = 1,        /* null pointer, bad size, bad alignment */
  TG_EUNSUPPORTED = 2,  /* a valid request the library does not implement */
  TG_EHIP = 3           /* a HIP launch or runtime error */
} tg_status;

typedef enum { TG_F32 = 0, TG_BF16 = 1 } tg_dtype;

typedef enum {
  TG_OP_GATE_SCORE = 0,
  TG_OP_SEQ_RMSNORM = 1,
  TG_OP_TOPK_SELECT = 2,
  TG_OP_COMPACT = 3,
  TG_OP_GATED_ATTENTION = 4,
  TG_OP_GATE_SELECT = 5,
  TG_OP_GATED_ATTENTION_ROPE = 6,
  TG_OP_GATED_ATTENTION_BACKWARD = 7,
  TG_OP_GATED_ATTENTION_ROPE_BACKWARD = 8
} tg_op;

/*
 * tg_gate_score -- row RMSNorm of the post-attention residual followed by the
 * scoring MLP (paper Section 4, "Scoring Network", Eq. 1 and the first half
 * of Eq. 3; Appendix C.4 for the residual after layer L's mixer).
 *
 * For every batch row and every prunable token j in [r, N):
 *     a~_j  = a_j * norm_w / sqrt(mean_c(a_j[c]^2) + eps_row)
 *     u     = W1 a~_j + b1                      (h values)
 *     out_j = sum_k w2[k] * silu(u[k]) + b2[0]  silu(x) = x / (1 + exp(-x))
 * and out_j = 0 for j < r.
 *
 *   resid     [B, N, d]  dtype `dt` (TG_BF16 or TG_F32), 16-byte aligned
 *   norm_w    [d]        dtype `dt`   RMSNorm weight
 *   W1        [h, d]     dtype `dt`   first linear layer (PyTorch Linear layout)
 *   b1        [h]        fp32
 *   w2        [h]        dtype `dt`   second linear layer (one output)
 *   b2        [1]        fp32
 *   score_raw [B, N]     fp32 output (the raw score b~)
 *   ws, ws_bytes         workspace of at least tg_workspace_size(TG_OP_GATE_SCORE,
 *                        B, N, d, h, K) = h * d * 2 bytes, 16-byte aligned (holds
 *                        W1 with the RMSNorm weight folded in; bf16 path only,
 *                        may be NULL for TG_F32)
 * Supported: TG_BF16 with d % 64 == 0, h in {64, 128, 256} and at most 2 GiB
 * per batch row (bf16 MFMA, fp32 accumulation; the product W1 * norm_w is
 * rounded to bf16, exact when norm_w is 1); TG_F32 with d % 4 == 0,
 * d <= 4096 and h <= 1024 (fp32 FMA).  Other shapes return TG_EUNSUPPORTED.
 */
int tg_gate_score(const void* resid, int dt, int B, int N, int d, int r,
                  const void* norm_w, float eps_row,
                  const void* W1, const float* b1, int h,
                  const void* w2, const float* b2,
                  float* score_raw, void* ws, size_t ws_bytes, void* stream);

/*
 * tg_gate_score splits into a weight preparation and the scorer proper, so
 * that a caller whose weights do not change folds them once (at load time)
 * instead of on every call:
 *
 * tg_gate_fold_weights -- writes W1 with the RMSNorm weight folded in,
 * bf16(W1[n][c] * norm_w[c]), in the order the scorer's kernels read it
 * (an opaque layout of h * d bf16 values), to W1_folded.  W1, norm_w as for
 * tg_gate_score; dt must be TG_BF16; folded_bytes >= h * d * 2
 * (= tg_workspace_size(TG_OP_GATE_SCORE, ...)); W1_folded 16-byte aligned.
 *
 * tg_gate_score_folded -- tg_gate_score with the folded weights in place of
 * W1 and norm_w; no workspace.  For the same inputs the scores equal
 * tg_gate_score's bit for bit.  Same shapes and errors as tg_gate_score's
 * bf16 path.
 */
int tg_gate_fold_weights(const void* W1, const void* norm_w, int dt, int h,
                         int d, void* W1_folded, size_t folded_bytes,
                         void* stream);
int tg_gate_score_folded(const void* resid, int dt, int B, int N, int d, int r,
                         const void* W1_folded, float eps_row, const float* b1,
                         int h, const void* w2, const float* b2,
                         float* score_raw, void* stream);

/*
 * tg_gate -- the whole gate in one call: the scoring network on folded
 * weights (tg_gate_score_folded), then the sequence RMSNorm, the top-K
 * selector and the compaction of tg_gate_select (paper, Section 4: "Scoring
 * Network" Eq. 1 and Eq. 3, "Top-K Selector" Eq. 4; App. C.4).  Two
 * launches: the scorer, in which the last workgroup of each batch row to
 * finish its scores runs that row's selection (found by counting the row's
 * finished workgroups, so no workgroup waits for another), then the gather
 * of the kept residual rows.  Every output equals tg_gate_score_folded
 * followed by tg_gate_select bit for bit.
 *
 *   resid, dt (TG_BF16 only), B, N (<= 32768), d, r, W1_folded, eps_row,
 *   b1, h, w2, b2    as tg_gate_score_folded (score_raw [B, N] fp32 receives
 *                    the raw scores)
 *   eps_seq, K, score, keep, kept_idx, resid_out, score_out
 *                    as tg_gate_select (score may be score_raw: in place)
 *   ws, ws_bytes     B 32-bit words of ZEROS, 4-byte aligned: the row
 *                    counters.  The call leaves them zero, so one buffer
 *                    zeroed once serves every later call.  Calls that share
 *                    a counter buffer must not overlap in time.
 */
int tg_gate(const void* resid, int dt, int B, int N, int d, int r,
            const void* W1_folded, float eps_row, const float* b1, int h,
            const void* w2, const float* b2, float eps_seq, int K,
            float* score_raw, float* score, uint8_t* keep, int32_t* kept_idx,
            void* resid_out, float* score_out, void* ws, size_t ws_bytes,
            void* stream);

/*
 * tg_gate_score_noalloc -- tg_gate_score for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same computation and the same result bits,
 * with no workspace argument.  The folded W1 goes to a fixed scratch array
 * of 4 MiB inside the library instead (one per device, held until the
 * process ends), so h * d * 2 must not exceed 4194304 bytes (h = 256 allows
 * d up to 8192); larger sizes return TG_EINVAL.  Nothing is allocated, on
 * the device or by any library routine.  The first call on a device looks
 * up that device's scratch address (no allocation, no enqueue).  Every call
 * on one device shares that device's scratch: calls on one stream are
 * ordered, but calls that may overlap on one device (other streams, other
 * threads) race on it and must be serialised by the caller.  The fp32 path
 * needs no scratch.  Arguments, supported shapes and errors are otherwise
 * those of tg_gate_score.
 */
int tg_gate_score_noalloc(const void* resid, int dt, int B, int N, int d, int r,
                          const void* norm_w, float eps_row,
                          const void* W1, const float* b1, int h,
                          const void* w2, const float* b2,
                          float* score_raw, void* stream);

/*
 * tg_seq_rmsnorm -- RMSNorm of the scalar scores along the sequence (paper
 * Section 4, "Scoring Network", second half of Eq. 3; scores of
 * non-prunable tokens are fixed to zero).
 *
 * For every batch row, with P = N - r:
 *     ms    = (1/P) * sum_{j in [r,N)} score_raw[j]^2
 *     out_j = score_raw[j] / sqrt(ms + eps_seq)   for j >= r,   0 for j < r.
 * With P == 0 every output is 0.  The reduction order is fixed.
 *
 *   score_raw [B, N] fp32 in;  score [B, N] fp32 out (may alias score_raw)
 *   ws, ws_bytes     workspace of tg_workspace_size(TG_OP_SEQ_RMSNORM, B, N,
 *                    ...) bytes, 16-byte aligned: none for N <= 32768, else
 *                    8 * B * ceil(N / 8192) (fp64 partial sums; contents need
 *                    no initialisation)
 */
int tg_seq_rmsnorm(const float* score_raw, int B, int N, int r, float eps_seq,
                   float* score, void* ws, size_t ws_bytes, void* stream);

/*
 * tg_topk_select -- top-K selector (paper Section 4, "Top-K Selector", Eq. 4):
 * keep the K' = min(K, N - r) highest-scoring prunable tokens and every
 * non-prunable token.
 *
 * Order: higher score first; equal scores go to the lower index; -0.0 and
 * +0.0 are equal; NaN ranks below every number, -inf included.  The order is
 * total, so exactly r + K' tokens are kept per batch row.
 *
 *   score [B, N] fp32 in;   keep [B, N] uint8 out (1 = kept, 0 = pruned)
 *   K >= 0 (K >= N - r keeps everything)
 *   ws, ws_bytes     workspace of tg_workspace_size(TG_OP_TOPK_SELECT, B, N,
 *                    ...) bytes, 16-byte aligned: none for N <= 32768, else
 *                    20496 * B (digit histograms, cleared by the call itself)
 */
int tg_topk_select(const float* score, int B, int N, int r, int K,
                   uint8_t* keep, void* ws, size_t ws_bytes, void* stream);

/*
 * tg_compact -- compaction of the residual stream to the kept set (paper
 * Section 4, "Top-K Selector": pruned tokens stop at layer L and the kept set
 * continues; Appendix C.4: kept tokens keep their original positions).
 *
 * Kept tokens are listed in ascending original order:
 *     kept_idx[m]   = j, the m-th kept token (also its original position)
 *     resid_out[m]  = resid[j]     (bit copy of the un-normalised residual)
 *     score_out[m]  = score[j]
 *
 *   resid     [B, N, d] dtype `dt`, 16-byte aligned; keep [B, N] uint8
 *   score     [B, N] fp32
 *   M         number of ones in every batch row of keep (the caller knows it:
 *             M = r + min(K, N - r) after tg_topk_select).  The library cannot
 *             check the count without a device->host read; a wrong M leaves
 *             rows unwritten or writes past M.
 *   kept_idx  [B, M] int32 out; resid_out [B, M, d] dtype `dt` out;
 *   score_out [B, M] fp32 out
 * Requires d * sizeof(dt) % 16 == 0.
 */
int tg_compact(const void* resid, int dt, int B, int N, int d, const uint8_t* keep,
               const float* score, int M, int32_t* kept_idx, void* resid_out,
               float* score_out, void* ws, size_t ws_bytes, void* stream);

/*
 * tg_gate_select -- tg_seq_rmsnorm, tg_topk_select and tg_compact in one call
 * (paper Section 4: the sequence RMSNorm of the scores, second half of Eq. 3;
 * the Top-K Selector, Eq. 4; compaction to the kept set, Appendix C.4).
 *
 * Every output is bit-identical to the three calls in sequence with
 * M = r + min(K, N - r):
 *     score     = tg_seq_rmsnorm(score_raw)
 *     keep      = tg_topk_select(score, K)
 *     kept_idx, resid_out, score_out = tg_compact(resid, keep, score, M)
 * Rows of up to 32768 tokens take two launches (one workgroup per batch row
 * normalises, selects and writes the kept indices and scores; then the row
 * gather); longer rows run the three calls.
 *
 *   score_raw [B, N] fp32 in;  score [B, N] fp32 out (may alias score_raw)
 *   keep [B, N] uint8 out;  resid [B, N, d] dtype `dt`, 16-byte aligned
 *   kept_idx [B, M] int32, resid_out [B, M, d] dtype `dt`, score_out [B, M]
 *   fp32 out
 *   ws, ws_bytes     workspace of tg_workspace_size(TG_OP_GATE_SELECT, B, N,
 *                    ...) bytes, 16-byte aligned: none for N <= 32768, else
 *                    the larger of the TG_OP_SEQ_RMSNORM and TG_OP_TOPK_SELECT
 *                    workspaces (contents need no initialisation)
 * Requires d * sizeof(dt) % 16 == 0 and K >= 0.
 */
int tg_gate_select(const float* score_raw, int B, int N, int r, float eps_seq, int K,
                   const void* resid, int dt, int d, float* score, uint8_t* keep,
                   int32_t* kept_idx, void* resid_out, float* score_out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * The same four steps with the prunable document anywhere in the prompt.
 * The paper's prompt is x = [x_R, x_D] (Section 3); its public interface
 * marks the prunable document with a placeholder inside the prompt (page 3),
 * so text may also follow the document.  These entry points take the
 * prunable span [span_begin, span_end) of every batch row in place of r.
 * Every token outside the span is non-prunable: its score is 0 and it is
 * always kept.  The kept set holds N - P + min(K, P) tokens, P = span_end -
 * span_begin, in ascending original order: first the tokens before the span,
 * then the kept span tokens, then the tokens after it.  The tokens after the
 * span occupy the last N - span_end ranks of kept_idx and score_out.
 * Arguments, workspaces and errors are otherwise those of the entry point
 * without the suffix.  The plain entry points are the case span_end == N,
 * bit for bit.  Requires 0 <= span_begin <= span_end <= N.
 */
int tg_gate_score_span(const void* resid, int dt, int B, int N, int d,
                       int span_begin, int span_end, const void* norm_w,
                       float eps_row, const void* W1, const float* b1, int h,
                       const void* w2, const float* b2, float* score_raw,
                       void* ws, size_t ws_bytes, void* stream);
int tg_seq_rmsnorm_span(const float* score_raw, int B, int N, int span_begin,
                        int span_end, float eps_seq, float* score, void* ws,
                        size_t ws_bytes, void* stream);
int tg_topk_select_span(const float* score, int B, int N, int span_begin,
                        int span_end, int K, uint8_t* keep, void* ws,
                        size_t ws_bytes, void* stream);
int tg_gate_select_span(const float* score_raw, int B, int N, int span_begin,
                        int span_end, float eps_seq, int K, const void* resid,
                        int dt, int d, float* score, uint8_t* keep,
                        int32_t* kept_idx, void* resid_out, float* score_out,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * tg_gate_score_varlen -- tg_gate_score for a varying-length batch: row b is
 * scored on its own prunable span [span_begin[b], span_end[b]) (int32 DEVICE
 * arrays of B entries, clamped into [0, N]); every other token of the row,
 * padding included, scores 0.  max_span (host) must be at least every span's
 * length: it sizes the grid, and a longer span is cut to max_span tokens.
 * Otherwise as tg_gate_score (same workspace).
 */
int tg_gate_score_varlen(const void* resid, int dt, int B, int N, int d,
                         const int32_t* span_begin, const int32_t* span_end,
                         int max_span, const void* norm_w, float eps_row,
                         const void* W1, const float* b1, int h,
                         const void* w2, const float* b2, float* score_raw,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * tg_gate_select_varlen -- tg_gate_select_span for a batch whose sequences
 * differ in length, in the position of the prunable document and in the
 * budget (serving batches several prompts; page 3's interface marks each
 * prompt's document and takes a kept-token budget).  Row b of the padded
 * [B, N] inputs holds a sequence of seq_len[b] tokens whose prunable span is
 * [span_begin[b], span_end[b]) with budget K[b]; its tokens at or past
 * seq_len[b] are padding: score 0, keep 0, never kept.  The row keeps
 *     M_b = seq_len[b] - P_b + min(K[b], P_b)   tokens, P_b = span_end[b] - span_begin[b],
 * written packed at rows cu_kept[b] .. cu_kept[b+1]-1 of kept_idx (indices
 * within the row), resid_out and score_out, in the order of the span
 * entry points.
 *
 *   seq_len, span_begin, span_end, K [B] and cu_kept [B + 1]: int32 DEVICE
 *                    arrays (cu_kept[0] = 0, cu_kept[b+1] = cu_kept[b] + M_b);
 *                    values are clamped into 0 <= span_begin <= span_end <=
 *                    seq_len <= N and K >= 0, and a row never writes more
 *                    than cu_kept[b+1] - cu_kept[b] kept tokens
 *   max_kept         host int, at least every M_b (sizes the gather's grid)
 *   score [B, N], keep [B, N]: as tg_gate_select (per row)
 *   kept_idx [cu_kept[B]] int32, resid_out [cu_kept[B], d], score_out
 *                    [cu_kept[B]] fp32: packed outputs
 *   ws, ws_bytes     tg_workspace_size(TG_OP_GATE_SELECT, B, N, 0, 0, 0)
 *                    bytes (none, ws may be NULL, when N <= 32768)
 * A row of up to 32768 tokens is selected by one workgroup; a longer one
 * (rows of any length <= N) by the sliced normalisation, the chunked
 * selection and the compaction scan of the separate calls.  Either way each
 * row's results equal tg_gate_select_span's on that row alone (its first
 * seq_len[b] tokens), bit for bit.
 */
int tg_gate_select_varlen(const float* score_raw, int B, int N,
                          const int32_t* seq_len, const int32_t* span_begin,
                          const int32_t* span_end, const int32_t* K,
                          const int32_t* cu_kept, int max_kept, float eps_seq,
                          const void* resid, int dt, int d, float* score,
                          uint8_t* keep, int32_t* kept_idx, void* resid_out,
                          float* score_out, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * tg_gated_attention -- token-gated causal GQA attention over the kept set
 * (paper Section 4: token-gated attention Eq. 5, head-wise gain Eq. 6,
 * temperature Eq. 7, combined as the key-bias form Eq. 8; Appendix C.4).
 *
 * For batch row b, query head h (kv head g = h / (Hq / Hkv)), kept rank i and
 * key rank j <= i:
 *     ratio_i = 1 if pos[i] == i, else ln(max(pos[i]+1, 2)) / ln(max(i+1, 2))
 *     z_ij    = (q_i . k_j) * sm_scale / (temp[h] * ratio_i) + gain[h] * key_score[j]
 *     out_i   = sum_j softmax_j(z_i) v_j
 *     lse_i   = ln sum_j exp(z_ij)
 * gain and temp are the effective (already positive) values; pos holds the
 * original positions of the kept tokens (kept_idx), or 0..M-1 for full-context
 * behaviour (ratio 1).
 *
 *   q   [B, M, Hq, d_h] bf16,   k, v [B, M, Hkv, d_h] bf16  (16-byte aligned)
 *   key_score [B, M] fp32,  pos [B, M] int32,  gain [Hq] fp32,  temp [Hq] fp32
 *   out [B, M, Hq, d_h] bf16 (fp32 accumulate, round to nearest even)
 *   lse [B, Hq, M] fp32, or NULL to skip it
 *   ws, ws_bytes  workspace of at least tg_workspace_size(TG_OP_GATED_ATTENTION,
 *                 B, M, Hkv * d_h, Hq, d_h) bytes, 16-byte aligned (holds an
 *                 fp16 transposed copy of V, the per-head key-score term
 *                 gain[h] * key_score[j] and the scale of each 64-key tile of
 *                 V; contents need no initialisation)
 * Precision: Q.K^T runs on bf16 MFMA; the softmax numerator and V enter the
 * P.V product as fp16, fp32 accumulation.  Each 64-key tile of a KV head's V
 * is scaled by a power of two that puts its largest |v| in [2^14, 2^15)
 * (for tile maxima in [2^-36, 2^65)), so every value within a factor 2^28
 * of its tile's largest converts exactly; the factor is taken out of the
 * softmax numerator, which therefore keeps fp16's 11 significant bits
 * relative to the row's largest contribution.
 * Supported: d_h in {64, 128}; Hq / Hkv in {1, 2, 4}.  M == 0 is a no-op.
 */
int tg_gated_attention(const void* q, const void* k, const void* v,
                       int B, int M, int Hq, int Hkv, int d_h,
                       const float* key_score, const int32_t* pos,
                       const float* gain, const float* temp, float sm_scale,
                       void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * The pruned forward replayed as one captured graph per padded length (paper
 * Section 5, "Implementation and timing": the forward after pruning is
 * captured as one CUDA graph per padded length).  The two entry points below
 * read the budget and the kept length from device memory, and size their
 * launches by a padded length M_pad fixed at capture time, so one captured
 * graph serves every budget whose kept set fits M_pad: the caller writes the
 * budget K into device memory before each replay.
 *
 * tg_gate_select_padded -- tg_gate_select with the budget of row b read from
 * K[b] (device int32; negative values count as 0) and the kept set written
 * into M_pad rows per batch row.  The budget is cut to M_pad - r, so row b
 * keeps M_b = r + min(K[b], N - r, M_pad - r) <= M_pad tokens, written to
 * kept_count[b] (device int32), and its outputs fill the first M_b rows of
 * kept_idx [B, M_pad], resid_out [B, M_pad, d] and score_out [B, M_pad];
 * rows M_b .. M_pad - 1 are left untouched.  score and keep are as in
 * tg_gate_select.  For the same K every output equals tg_gate_select's bit
 * for bit.  Requires r <= M_pad <= N <= 32768; no workspace.
 */
int tg_gate_select_padded(const float* score_raw, int B, int N, int r,
                          float eps_seq, const int32_t* K, int M_pad,
                          const void* resid, int dt, int d, float* score,
                          uint8_t* keep, int32_t* kept_idx, void* resid_out,
                          float* score_out, int32_t* kept_count, void* stream);

/*
 * tg_gated_attention_padded -- tg_gated_attention where batch row b uses the
 * first M_b = kept_count[b] (device int32, clamped to [0, M_pad]) rows of
 * tensors laid out with the padded length M_pad: q [B, M_pad, Hq, d_h],
 * k, v [B, M_pad, Hkv, d_h], key_score and pos [B, M_pad], out [B, M_pad,
 * Hq, d_h], lse [B, Hq, M_pad] (or NULL).  Rows M_b .. M_pad - 1 are neither
 * read nor written.  Each row's results equal tg_gated_attention's for M =
 * M_b bit for bit.  The workspace is tg_gated_attention's for M = M_pad.
 */
int tg_gated_attention_padded(const void* q, const void* k, const void* v,
                              int B, int M_pad, const int32_t* kept_count,
                              int Hq, int Hkv, int d_h, const float* key_score,
                              const int32_t* pos, const float* gain,
                              const float* temp, float sm_scale, void* out,
                              float* lse, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * tg_gated_attention_varlen -- tg_gated_attention over the packed kept rows of
 * a varying-length batch (the output layout of tg_gate_select_varlen).
 * Sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of q [T, Hq, d_h],
 * k and v [T, Hkv, d_h], key_score [T], pos [T] and out [T, Hq, d_h]; lse,
 * when given, holds sequence b's [Hq, M_b] block (head-major, as the batched
 * entry point's [B, Hq, M] for B = 1) at offset cu_seqlens[b] * Hq.
 * Causality and the temperature's ranks run within each sequence.
 *
 *   cu_seqlens [B + 1] int32 HOST array (cu_seqlens[0] = 0, non-decreasing)
 *   ws, ws_bytes     workspace of at least tg_workspace_size(
 *                    TG_OP_GATED_ATTENTION, 1, T + 63 * B, Hkv * d_h, Hq, d_h)
 *                    bytes, T = cu_seqlens[B] (every sequence's fp16 V^T copy
 *                    and key-score terms, each padded to 64 rows, side by
 *                    side), 16-byte aligned
 * Every sequence is validated as tg_gated_attention (a batch of one) before
 * anything is launched.  Up to 64 non-empty sequences share one launch of
 * each kernel (longest first); empty sequences are skipped.
 */
int tg_gated_attention_varlen(const void* q, const void* k, const void* v,
                              int B, const int32_t* cu_seqlens, int Hq,
                              int Hkv, int d_h, const float* key_score,
                              const int32_t* pos, const float* gain,
                              const float* temp, float sm_scale, void* out,
                              float* lse, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * tg_gated_attention_rope -- tg_gated_attention on rotary-embedded queries and
 * keys.  The paper keeps every kept token's original position for the
 * position encoding of the layers above the gate (Appendix C.4); this entry
 * point applies the rotate-half rotary embedding at those positions (`pos`)
 * before the attention, so q and k can be passed un-rotated:
 *     for each head vector x (width d_h) of q and k at kept rank i,
 *     pair (x_j, x_{j + d_h/2}), j < d_h/2, turns by the angle
 *     pos[i] * rope_base^(-2 j / d_h):
 *       x'_j          = x_j cos a - x_{j+d_h/2} sin a
 *       x'_{j+d_h/2}  = x_{j+d_h/2} cos a + x_j sin a
 * and the rotated q', k' (rounded to bf16, nearest even) replace q, k in the
 * definition of tg_gated_attention (pos also keeps its role in the
 * temperature).  The angle is formed and reduced modulo 2 pi in fp64; its
 * sine and cosine and the rotation are fp32.
 *
 *   arguments as tg_gated_attention, plus rope_base (> 1, e.g. 1e6)
 *   ws, ws_bytes     workspace of at least tg_workspace_size(
 *                    TG_OP_GATED_ATTENTION_ROPE, B, M, Hkv * d_h, Hq, d_h) bytes,
 *                    16-byte aligned (tg_gated_attention's workspace followed
 *                    by the rotated k and the cosines and sines of every
 *                    row's angles; q is rotated inside the attention kernel
 *                    from those; contents need no initialisation)
 */
int tg_gated_attention_rope(const void* q, const void* k, const void* v,
                            int B, int M, int Hq, int Hkv, int d_h,
                            const float* key_score, const int32_t* pos,
                            const float* gain, const float* temp, float sm_scale,
                            double rope_base, void* out, float* lse, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * tg_gated_attention_rope_varlen -- tg_gated_attention_varlen with the rotary
 * embedding of tg_gated_attention_rope: every packed row of q and k turns by
 * its own original position pos[t] (Appendix C.4: kept tokens keep their
 * positions in every prompt of the batch).  Each sequence's results equal
 * tg_gated_attention_rope's for that sequence alone, bit for bit.  The
 * workspace is at least tg_workspace_size(TG_OP_GATED_ATTENTION_ROPE, 1,
 * T + 63 * B, Hkv * d_h, Hq, d_h) bytes, T = cu_seqlens[B].  Otherwise as
 * tg_gated_attention_varlen.
 */
int tg_gated_attention_rope_varlen(const void* q, const void* k, const void* v,
                                   int B, const int32_t* cu_seqlens, int Hq,
                                   int Hkv, int d_h, const float* key_score,
                                   const int32_t* pos, const float* gain,
                                   const float* temp, float sm_scale,
                                   double rope_base, void* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * tg_gated_attention_backward -- gradients of tg_gated_attention.  In the
 * paper the key score reaches the loss only through the gain_h * b_j term of
 * the token-gated attention logits (Section 4, token-gated attention, Eq. 8):
 * that term is what trains the scorer despite the non-differentiable top-K,
 * and the per-head gain and the temperature are trainable as well ("Putting
 * everything together").  With z, c_i and lse as in tg_gated_attention,
 * P_ij = exp(z_ij - lse_i) (j <= i) and the upstream gradient dO:
 *     D_i      = dO_i . O_i
 *     dZ_ij    = P_ij (dO_i . v_j - D_i)
 *     d_q_i    = c_i sum_j dZ_ij k_j                 (per query head)
 *     d_k_j    = sum_{h of the group} sum_i c_i dZ_ij q_i
 *     d_v_j    = sum_{h of the group} sum_i P_ij dO_i
 *     d_key_score_j = sum_h gain_h sum_i dZ_{h,ij}
 *     d_gain_h = sum_{b,i,j} dZ_{h,ij} key_score_j
 *     d_temp_h = -(1 / temp_h) sum_{b,i,j} dZ_{h,ij} (q_i . k_j) c_i
 * P and D are formed from the forward's own outputs `out` and `lse`, as in
 * the usual flash-attention backward.
 *
 *   q, k, v, key_score, pos, gain, temp, sm_scale, B, M, Hq, Hkv, d_h
 *                    as passed to tg_gated_attention
 *   out [B, M, Hq, d_h] bf16 and lse [B, Hq, M] fp32: that call's outputs
 *   d_out [B, M, Hq, d_h] bf16: the gradient of the loss with respect to out
 *   d_q [B, M, Hq, d_h], d_k and d_v [B, M, Hkv, d_h] bf16 (nearest even)
 *   d_key_score [B, M] fp32; d_gain [Hq] and d_temp [Hq] fp32, summed over
 *                    the batch.  Every output is overwritten, not accumulated.
 *   ws, ws_bytes     workspace of at least tg_workspace_size(
 *                    TG_OP_GATED_ATTENTION_BACKWARD, B, M, Hkv * d_h, Hq, d_h)
 *                    bytes, 16-byte aligned, contents need no initialisation
 *   d_h in {64, 128}; Hq / Hkv in {1, 2, 4}; B <= 65535.  With M == 0 only
 *   d_gain and d_temp are written (zeros) and the other pointers may be NULL.
 *   Products run on bf16 MFMA with fp32 accumulation (P and dZ c are rounded
 *   to bf16 for the second products); the softmax terms are fp32; d_gain and
 *   d_temp add their fp32 per-block partials in fp64.
 */
int tg_gated_attention_backward(const void* q, const void* k, const void* v,
                                const void* out, const float* lse,
                                const void* d_out, int B, int M, int Hq,
                                int Hkv, int d_h, const float* key_score,
                                const int32_t* pos, const float* gain,
                                const float* temp, float sm_scale, void* d_q,
                                void* d_k, void* d_v, float* d_key_score,
                                float* d_gain, float* d_temp, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * tg_gated_attention_rope_backward -- gradients of tg_gated_attention_rope.
 * q and k are rotated exactly as the forward rotates them (bf16 copies, so
 * the products see the forward's operands), the gradients of
 * tg_gated_attention_backward are formed with respect to the rotated q' and
 * k' in fp32, and the transposed rotation maps them back:
 *     d_q_j         = d_q'_j c + d_q'_{j+d_h/2} s
 *     d_q_{j+d_h/2} = d_q'_{j+d_h/2} c - d_q'_j s        (and the same for k)
 * with c, s the cosine and sine of the same angle, rounded once to bf16.  The
 * rounding of q', k' to bf16 is passed through as the identity.  d_v,
 * d_key_score, d_gain and d_temp are those of the rotated problem.
 *
 *   arguments as tg_gated_attention_backward, plus rope_base (> 1) as given
 *   to the forward; out and lse are that forward's outputs
 *   ws, ws_bytes     workspace of at least tg_workspace_size(
 *                    TG_OP_GATED_ATTENTION_ROPE_BACKWARD, B, M, Hkv * d_h, Hq,
 *                    d_h) bytes, 16-byte aligned: the backward's workspace
 *                    rounded up to 16 bytes, then 6 * B * M * (Hq + Hkv) * d_h
 */
int tg_gated_attention_rope_backward(const void* q, const void* k,
                                     const void* v, const void* out,
                                     const float* lse, const void* d_out,
                                     int B, int M, int Hq, int Hkv, int d_h,
                                     const float* key_score,
                                     const int32_t* pos, const float* gain,
                                     const float* temp, float sm_scale,
                                     double rope_base, void* d_q, void* d_k,
                                     void* d_v, float* d_key_score,
                                     float* d_gain, float* d_temp, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * tg_gated_attention_backward_varlen -- tg_gated_attention_backward over the
 * packed sequences of tg_gated_attention_varlen (same layouts: rows
 * cu_seqlens[b] .. cu_seqlens[b+1]-1; out and lse as that call wrote them).
 * d_gain and d_temp are [B, Hq]: sequence b's gradients in row b (sum the
 * rows for the batch's gradient; an empty sequence's rows are 0).
 * cu_seqlens is a HOST array; the workspace is at least tg_workspace_size(
 * TG_OP_GATED_ATTENTION_BACKWARD, 1, T + 63 * B, Hkv * d_h, Hq, d_h) bytes,
 * T = cu_seqlens[B] (every sequence's row constants and partials, each
 * padded to 64 rows, side by side).  Every sequence is validated as
 * tg_gated_attention_backward (a batch of one) before anything is launched;
 * up to 64 sequences share one launch of each kernel (longest first), and
 * each sequence's results equal that batch-of-one call's bit for bit.
 */
int tg_gated_attention_backward_varlen(const void* q, const void* k,
                                       const void* v, const void* out,
                                       const float* lse, const void* d_out,
                                       int B, const int32_t* cu_seqlens,
                                       int Hq, int Hkv, int d_h,
                                       const float* key_score,
                                       const int32_t* pos, const float* gain,
                                       const float* temp, float sm_scale,
                                       void* d_q, void* d_k, void* d_v,
                                       float* d_key_score, float* d_gain,
                                       float* d_temp, void* ws,
                                       size_t ws_bytes, void* stream);

/*
 * tg_gated_attention_rope_backward_varlen -- gradients of
 * tg_gated_attention_rope_varlen (q and k passed un-rotated, as to that
 * call; every packed row turned by its own original position pos[t],
 * Appendix C.4).  d_q and d_k are with respect to the un-rotated q and k
 * (the transposed rotation of the gradients with respect to the rotated
 * ones, as tg_gated_attention_rope_backward).  The workspace is at least
 * tg_workspace_size(TG_OP_GATED_ATTENTION_ROPE_BACKWARD, 1, T + 63 * B,
 * Hkv * d_h, Hq, d_h) bytes, T = cu_seqlens[B].  Each sequence's results
 * equal tg_gated_attention_rope_backward's for that sequence alone (a batch
 * of one), bit for bit.  Otherwise as tg_gated_attention_backward_varlen.
 */
int tg_gated_attention_rope_backward_varlen(const void* q, const void* k,
                                            const void* v, const void* out,
                                            const float* lse,
                                            const void* d_out, int B,
                                            const int32_t* cu_seqlens, int Hq,
                                            int Hkv, int d_h,
                                            const float* key_score,
                                            const int32_t* pos,
                                            const float* gain,
                                            const float* temp, float sm_scale,
                                            double rope_base, void* d_q,
                                            void* d_k, void* d_v,
                                            float* d_key_score, float* d_gain,
                                            float* d_temp, void* ws,
                                            size_t ws_bytes, void* stream);

/*
 * tg_kv_cache_prune -- post-prefill pruning of the KV cache of the layers at
 * and below the gate (paper, Section 5, "Implementation and timing", and
 * Appendix B: optionally, once prefill completes, those layers keep only the
 * selected tokens, so that decoding holds the same kept entries at every
 * layer).  For every layer l < n_layers and batch row b:
 *     k_out[l, b, m] = k_cache[l, b, kept_idx[b, m]]   (and the same for v)
 *
 *   k_cache, v_cache [n_layers, B, N, Hkv, d_h] two-byte values (bf16)
 *   kept_idx [B, M] int32: the kept set of tg_compact / tg_gate_select,
 *                    ascending original indices (any order is accepted)
 *   k_out, v_out [n_layers, B, M, Hkv, d_h]: the caller's buffers (they may
 *                    not overlap the caches); rows are copied bit for bit
 *   M in [0, N]; d_h a multiple of 8.  An index outside [0, N) leaves its
 *   output row unwritten.  n_layers == 0 or M == 0 enqueue nothing.
 */
int tg_kv_cache_prune(const void* k_cache, const void* v_cache, int n_layers,
                      int B, int N, int Hkv, int d_h, const int32_t* kept_idx,
                      int M, void* k_out, void* v_out, void* stream);

/* Workspace bytes an entry point needs for the given sizes (0 when none).
 * For TG_OP_GATED_ATTENTION pass N = M (kept length), d = Hkv * d_h, h = Hq
 * and K = d_h; the size is B * round_up(M, 64) * (2 * Hkv * d_h + 4 * (Hq +
 * Hkv)).  K = 0 gives the size for the largest Hkv (= Hq), an upper bound.
 * For TG_OP_GATED_ATTENTION_ROPE pass the same and K = d_h; the size adds
 * B * M * d_h * 2 * Hkv (the rotated k) + B * round_up(M, 64) * d_h * 4
 * (the angle table).
 * For TG_OP_GATED_ATTENTION_BACKWARD pass the same as for
 * TG_OP_GATED_ATTENTION_ROPE; with Mp = round_up(M, 64) the size is
 * B * Mp * (12 Hq + 4 Hkv) + 8 * B * (Mp / 64) * Hq.
 * TG_OP_SEQ_RMSNORM and TG_OP_TOPK_SELECT depend on B and N only. */
size_t tg_workspace_size(int op, int B, int N, int d, int h, int K);

/* Message describing the last non-zero status returned on this thread. */
const char* tg_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int tg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
