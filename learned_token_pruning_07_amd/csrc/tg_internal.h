// Host-side launchers of the TokenGate kernels.  Arguments are validated by the
// C-ABI front end (tg_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tg {

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();

// Rows [r, p1) of each batch row are the prunable span (p1 = N for a prompt
// [x_R, x_D]); every other row scores 0.
// With span_begin/span_end (device [B] arrays) set, row b's span comes from
// them (clamped into [0, N]) and [r, p1) only sizes the grid (p1 - r = the
// longest span).
hipError_t launch_gate_score_bf16(const uint16_t* resid, int B, int N, int d, int r, int p1,
                                  const int32_t* span_begin, const int32_t* span_end,
                                  const uint16_t* norm_w, float eps_row, const uint16_t* W1,
                                  const float* b1, int h, const uint16_t* w2, const float* b2,
                                  float* out, void* ws, hipStream_t s);

// Workspace bytes of launch_gate_score_bf16: the norm-weight-folded W1.
size_t gate_score_workspace(int h, int d);
// Its two halves: W1 with the norm weight folded in (fragment order, h * d
// bf16 values), and the scorer on an already folded W1.
hipError_t launch_gate_fold(const uint16_t* W1, const uint16_t* norm_w, int h, int d, void* W1f, hipStream_t s);
hipError_t launch_gate_score_folded(const uint16_t* resid, int B, int N, int d, int r, int p1,
                                    const int32_t* span_begin, const int32_t* span_end, float eps_row,
                                    const uint16_t* W1f, const float* b1, int h, const uint16_t* w2,
                                    const float* b2, float* out, hipStream_t s);

// The scorer's static scratch (for callers that cannot allocate): its size,
// and its device address on the current device (looked up on the first call
// per device, then cached).
constexpr size_t kGateScoreScratchBytes = size_t(4) << 20;
hipError_t gate_score_scratch(void** ptr);

hipError_t launch_gate_score_f32(const float* resid, int B, int N, int d, int r, int p1,
                                 const int32_t* span_begin, const int32_t* span_end,
                                 const float* norm_w, float eps_row, const float* W1,
                                 const float* b1, int h, const float* w2, const float* b2,
                                 float* out, hipStream_t s);

// Per-row lengths, spans, budgets and output offsets of a varying-length
// batch (device arrays of B, B, B, B and B + 1 entries); all null for a
// uniform batch.  With len null but K set, the rows are uniform in length
// and span but take their budgets from K (device), write their kept tokens
// at rows b * pad of the outputs and their kept counts to kept_count[b].
struct VarlenRows {
  const int32_t* len;
  const int32_t* span_begin;
  const int32_t* span_end;
  const int32_t* K;
  const int32_t* cu_kept;
  int pad = 0;
  int32_t* kept_count = nullptr;
};

// Row b of a varying-length batch: its length, prunable span [r, p1) and
// budget, clamped into 0 <= r <= p1 <= len <= N and K >= 0.
struct RowSpec {
  int len, r, p1, K;
};
__device__ __forceinline__ RowSpec varlen_row(const VarlenRows& vr, int b, int N) {
  RowSpec rs;
  rs.len = min(max(vr.len[b], 0), N);
  rs.p1 = min(max(vr.span_end[b], 0), rs.len);
  rs.r = min(max(vr.span_begin[b], 0), rs.p1);
  rs.K = max(vr.K[b], 0);
  return rs;
}
// A varying-length row of up to this many tokens is selected by one
// workgroup; the kernels of the longer rows skip it.
constexpr int kVarlenOneGroupRow = 32768;

// The whole gate in two launches (bf16 residual, N <= 32768): the folded
// scorer, whose last workgroup of each row runs that row's selection
// (count: B zeroed words, left zeroed), then the kept rows' gather.  The
// results equal launch_gate_score_folded + launch_gate_select bit for bit.
hipError_t launch_gate_fused(const uint16_t* resid, int B, int N, int d, int r, const uint16_t* W1w, float eps_row,
                             const float* b1, int h, const uint16_t* w2, const float* b2, float eps_seq, int K,
                             float* score_raw, float* score, uint8_t* keep, int32_t* kept_idx, uint16_t* resid_out,
                             float* score_kept, uint32_t* count, hipStream_t s);

size_t seq_rmsnorm_workspace(int B, int N);
hipError_t launch_seq_rmsnorm(const float* in, int B, int N, int r, int p1, float eps, float* out, void* ws,
                              hipStream_t s);
// the sliced normalisation of the rows of a varying-length batch longer than
// kVarlenOneGroupRow tokens (N > kVarlenOneGroupRow; the others are untouched)
hipError_t launch_seq_rmsnorm_long_rows(const float* in, int B, int N, VarlenRows vr, float eps, float* out,
                                        void* ws, hipStream_t s);

size_t topk_select_workspace(int B, int N);
hipError_t launch_topk_select(const float* score, int B, int N, int r, int p1, int K, uint8_t* keep, void* ws,
                              hipStream_t s);
// the chunked selection of those long rows (every budget, trivial ones
// included; keep 0 past a row's length)
hipError_t launch_topk_select_long_rows(const float* score, int B, int N, VarlenRows vr, uint8_t* keep, void* ws,
                                        hipStream_t s);

hipError_t launch_compact(const void* resid, size_t row_bytes, int B, int N, const uint8_t* keep,
                          const float* score, int M, int32_t* kept_idx, void* resid_out,
                          float* score_out, hipStream_t s);

// kept_idx and score_out of those long rows from their keep masks, at rows
// cu_kept[b] .. cu_kept[b + 1] - 1
hipError_t launch_compact_scan_long_rows(const uint8_t* keep, const float* score, int B, int N, VarlenRows vr,
                                         int32_t* kept_idx, float* score_out, hipStream_t s);

// resid_out[m] = resid[kept_idx[m]] for m < M (the row gather of launch_compact)
hipError_t launch_compact_gather(const void* resid, size_t row_bytes, int B, int N, int M,
                                 const int32_t* kept_idx, void* resid_out, hipStream_t s);

// out[cu_kept[b] + m] = resid[b, kept_idx[cu_kept[b] + m]] for m < cu_kept[b + 1] - cu_kept[b] <= max_kept
hipError_t launch_compact_gather_varlen(const void* resid, size_t row_bytes, int B, int N, const int32_t* cu_kept,
                                        int max_kept, const int32_t* kept_idx, void* resid_out, hipStream_t s);

// out[b * pad + m] = resid[b, kept_idx[b * pad + m]] for m < count[b] (clamped to [0, pad])
hipError_t launch_compact_gather_padded(const void* resid, size_t row_bytes, int B, int N, const int32_t* count,
                                        int pad, const int32_t* kept_idx, void* resid_out, hipStream_t s);

// gate selection of a varying-length batch: rows of up to 32768 tokens in
// one workgroup each, longer ones (N > 32768) through the sliced
// normalisation, the chunked selection and the compaction scan, with
// gate_select_workspace(B, N) bytes of workspace
hipError_t launch_gate_select_varlen(const float* score_raw, int B, int N, VarlenRows vr, int max_kept, float eps,
                                     const void* resid, size_t row_bytes, float* score, uint8_t* keep,
                                     int32_t* kept_idx, void* resid_out, float* score_kept, void* ws,
                                     hipStream_t s);

// gate selection with per-row budgets from a device array and outputs padded
// to pad rows per batch row (rows of up to 32768 tokens); the kept counts go
// to kept_count (device) and the gather reads them from there
hipError_t launch_gate_select_padded(const float* score_raw, int B, int N, int r, float eps, const int32_t* K,
                                     int pad, const void* resid, size_t row_bytes, float* score, uint8_t* keep,
                                     int32_t* kept_idx, void* resid_out, float* score_kept, int32_t* kept_count,
                                     hipStream_t s);

// launch_seq_rmsnorm + launch_topk_select + launch_compact in sequence, bit
// for bit (M = N - P + min(K, P), P = p1 - r); two launches for rows of up to
// 32768 tokens.
size_t gate_select_workspace(int B, int N);
hipError_t launch_gate_select(const float* score_raw, int B, int N, int r, int p1, float eps, int K,
                              const void* resid, size_t row_bytes, float* score, uint8_t* keep, int32_t* kept_idx,
                              void* resid_out, float* score_kept, void* ws, hipStream_t s);

// rope_base > 0: q and k are first rotated (rotary embedding at the positions
// pos, base rope_base) into the workspace, and the attention reads the copies.
// m_dev (may be null): per-row kept lengths [B] on the device, each clamped
// to [0, M]; the tensors keep their [B, M, ...] layout (M the padded length)
// and row b uses only its first m_dev[b] rows.
hipError_t launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B,
                                  int M, int Hq, int Hkv, int dh, const float* key_score,
                                  const int32_t* pos, const float* gain, const float* temp,
                                  float sm_scale, double rope_base, uint16_t* out, float* lse, void* ws,
                                  hipStream_t s, const int32_t* m_dev = nullptr);

// Packed sequences of a varying-length batch (cu_seqlens a host array of B + 1
// row offsets): one prepass and one attention launch per 64 non-empty
// sequences, all sequences' V^T copies and key-score terms side by side in
// the workspace (gated_attention_workspace(1, slots) bytes, slots from
// gated_attention_varlen_slots).
hipError_t launch_gated_attention_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B,
                                         const int32_t* cu_seqlens, int Hq, int Hkv, int dh, const float* key_score,
                                         const int32_t* pos, const float* gain, const float* temp, float sm_scale, double rope_base,
                                         uint16_t* out, float* lse, void* ws, hipStream_t s);
// sum over the sequences of the length rounded up to 64 key slots
size_t gated_attention_varlen_slots(int B, const int32_t* cu_seqlens);

// Workspace bytes of launch_gated_attention: the fp16 V^T copy and the
// key-score terms; with the rotary embedding also the rotated q and k.
size_t gated_attention_workspace(int B, int M, int Hq, int Hkv, int dh);
size_t gated_attention_rope_workspace(int B, int M, int Hq, int Hkv, int dh);
// the rotary varying-length call's workspace (rope_base > 0)
size_t gated_attention_rope_varlen_workspace(int B, const int32_t* cu_seqlens, int Hq, int Hkv, int dh);

// Backward of the token-gated attention: dq, dk, dv (bf16), the key-score
// gradient [B, M] and the gain and temperature gradients [Hq] (fp32).
hipError_t launch_gated_attention_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                           const uint16_t* out, const float* lse, const uint16_t* d_out, int B, int M,
                                           int Hq, int Hkv, int dh, const float* key_score, const int32_t* pos,
                                           const float* gain, const float* temp, float sm_scale, double rope_base,
                                           uint16_t* dq,
                                           uint16_t* dk, uint16_t* dv, float* d_key_score, float* d_gain,
                                           float* d_temp, void* ws, hipStream_t s);
size_t gated_attention_backward_workspace(int B, int M, int Hq, int Hkv, int dh);
// Packed sequences (host cu_seqlens, B + 1 offsets): one launch of each kernel
// per 64 sequences, every sequence's row constants and partials side by side
// in the workspace (gated_attention_backward_varlen_workspace bytes); d_gain
// and d_temp [B, Hq].  rope_base > 0: q and k rotated by their positions
// first (gated_attention_rope_backward_varlen_workspace bytes).
hipError_t launch_gated_attention_backward_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                                  const uint16_t* out, const float* lse, const uint16_t* d_out, int B,
                                                  const int32_t* cu_seqlens, int Hq, int Hkv, int dh,
                                                  const float* key_score, const int32_t* pos, const float* gain,
                                                  const float* temp, float sm_scale, double rope_base, uint16_t* dq,
                                                  uint16_t* dk, uint16_t* dv, float* d_key_score, float* d_gain,
                                                  float* d_temp, void* ws, hipStream_t s);
size_t gated_attention_backward_varlen_workspace(int B, const int32_t* cu_seqlens, int Hq, int Hkv);
size_t gated_attention_rope_backward_varlen_workspace(int B, const int32_t* cu_seqlens, int Hq, int Hkv, int dh);
size_t gated_attention_rope_backward_workspace(int B, int M, int Hq, int Hkv, int dh);

// Row gather of the K and V caches of n_layers layers to the kept set.
hipError_t launch_kv_cache_prune(const void* k_cache, const void* v_cache, int n_layers, int B, int N, int Hkv,
                                 int dh, const int32_t* kept_idx, int M, void* k_out, void* v_out, hipStream_t s);

}  // namespace tg
