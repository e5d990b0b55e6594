// C-ABI front end of the TokenGate library: argument validation, dispatch,
// error reporting.  Every check runs before anything is enqueued; no HIP call
// is made on a path that returns an error status.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/tokengate.h"
#include "tg_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TG_OK;
  return fail(TG_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t dt_size(int dt) { return dt == TG_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int tg_version(void) { return 10000; }

const char* tg_last_error(void) { return g_err; }

size_t tg_workspace_size(int op, int B, int N, int d, int h, int K) {
  if (op == TG_OP_GATE_SCORE) {
    if (d <= 0 || h <= 0) return 0;
    return tg::gate_score_workspace(h, d);  // the RMSNorm weight folded into W1 (bf16)
  }
  if (op == TG_OP_TOPK_SELECT) {
    if (B <= 0 || N <= 0) return 0;
    return tg::topk_select_workspace(B, N);  // digit histograms, rows longer than 32768 only
  }
  if (op == TG_OP_SEQ_RMSNORM) {
    if (B <= 0 || N <= 0) return 0;
    return tg::seq_rmsnorm_workspace(B, N);  // fp64 partial sums, rows longer than 32768 only
  }
  if (op == TG_OP_GATE_SELECT) {
    if (B <= 0 || N <= 0) return 0;
    return tg::gate_select_workspace(B, N);  // rows longer than 32768 only
  }
  if (op == TG_OP_GATED_ATTENTION) {
    if (B <= 0 || N <= 0 || d <= 0 || h <= 0 || K < 0) return 0;
    // d = Hkv * d_h, h = Hq, K = d_h: an fp16 V^T copy (B * Hkv * d_h *
    // round_up(M, 64) values), the fp32 key-score term of every query head and
    // the V^T tile scales of every KV head (B * (Hq + Hkv) * round_up(M, 64)).
    // K = 0 sizes for the largest Hkv (= Hq).
    if (K > 0) return d % K == 0 ? tg::gated_attention_workspace(B, N, h, d / K, K) : 0;
    const size_t Mp = (size_t)(N + 63) / 64 * 64;
    return (size_t)B * Mp * ((size_t)d * 2 + (size_t)h * 8);
  }
  if (op == TG_OP_GATED_ATTENTION_ROPE) {
    // as TG_OP_GATED_ATTENTION with K = d_h, plus the rotated q and k (bf16)
    if (B <= 0 || N <= 0 || d <= 0 || h <= 0 || K <= 0 || d % K != 0) return 0;
    return tg::gated_attention_rope_workspace(B, N, h, d / K, K);
  }
  if (op == TG_OP_GATED_ATTENTION_BACKWARD) {
    // N = M, d = Hkv * d_h, h = Hq, K = d_h: per-row constants and the
    // partial sums of the key-score, gain and temperature gradients
    if (B <= 0 || N <= 0 || d <= 0 || h <= 0 || K <= 0 || d % K != 0) return 0;
    return tg::gated_attention_backward_workspace(B, N, h, d / K, K);
  }
  if (op == TG_OP_GATED_ATTENTION_ROPE_BACKWARD) {
    // as TG_OP_GATED_ATTENTION_BACKWARD, then the rotated q and k (bf16) and
    // the fp32 gradients with respect to them
    if (B <= 0 || N <= 0 || d <= 0 || h <= 0 || K <= 0 || d % K != 0) return 0;
    return tg::gated_attention_rope_backward_workspace(B, N, h, d / K, K);
  }
  return 0;
}

static int gate_score_common(const char* name, const void* resid, int dt, int B, int N, int d, int r, int p1,
                             const int32_t* sb, const int32_t* se,
                             const void* norm_w, float eps_row, const void* W1, const float* b1, int h,
                             const void* w2, const float* b2, float* score_raw, void* ws, size_t ws_bytes,
                             void* stream, bool static_scratch = false) {
  if (dt != TG_BF16 && dt != TG_F32) return fail(TG_EINVAL, "%s: unknown dtype %d", name, dt);
  if (B <= 0 || N <= 0 || d <= 0 || h <= 0) return fail(TG_EINVAL, "%s: B, N, d, h must be > 0", name);
  if (r < 0 || r > p1 || p1 > N)
    return fail(TG_EINVAL, "%s: prunable span [%d, %d) outside [0, N=%d]", name, r, p1, N);
  if (!resid || !norm_w || !W1 || !b1 || !w2 || !b2 || !score_raw)
    return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!(eps_row >= 0.0f)) return fail(TG_EINVAL, "%s: eps_row must be >= 0", name);
  if ((long long)B * N * d > (1LL << 40)) return fail(TG_EINVAL, "%s: tensor too large", name);
  if (!aligned16(resid) || !aligned16(W1) || !aligned16(norm_w) || !aligned4(score_raw) || !aligned4(b1) ||
      !aligned4(b2))
    return fail(TG_EINVAL, "%s: resid, W1 and norm_w must be 16-byte aligned", name);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dt == TG_BF16) {
    if (d % 64 != 0) return fail(TG_EUNSUPPORTED, "%s: bf16 needs d %% 64 == 0 (d=%d)", name, d);
    if (h != 64 && h != 128 && h != 256)
      return fail(TG_EUNSUPPORTED, "%s: bf16 supports h in {64,128,256} (h=%d)", name, h);
    const size_t need = tg::gate_score_workspace(h, d);
    if (static_scratch) {
      if (need > tg::kGateScoreScratchBytes)
        return fail(TG_EINVAL, "%s: h * d * 2 = %zu bytes exceeds the %zu-byte static scratch", name, need,
                    tg::kGateScoreScratchBytes);
    } else {
      if (!ws || ws_bytes < need)
        return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
      if (!aligned16(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
    }
    if ((size_t)(p1 - r) * d * 2 > 0x7FFFFFFFull)
      return fail(TG_EUNSUPPORTED, "%s: a batch row above 2 GiB", name);
    if (static_scratch) {  // every argument is valid: look up this device's scratch
      const int rc = hip_status(tg::gate_score_scratch(&ws), name);
      if (rc != TG_OK) return rc;
    }
    return hip_status(tg::launch_gate_score_bf16(static_cast<const uint16_t*>(resid), B, N, d, r, p1, sb, se,
                                                 static_cast<const uint16_t*>(norm_w), eps_row,
                                                 static_cast<const uint16_t*>(W1), b1, h,
                                                 static_cast<const uint16_t*>(w2), b2, score_raw, ws, s),
                      name);
  }
  if (d % 4 != 0 || d > 4096 || h > 1024)
    return fail(TG_EUNSUPPORTED, "%s: fp32 needs d %% 4 == 0, d <= 4096, h <= 1024", name);
  return hip_status(tg::launch_gate_score_f32(static_cast<const float*>(resid), B, N, d, r, p1, sb, se,
                                              static_cast<const float*>(norm_w), eps_row,
                                              static_cast<const float*>(W1), b1, h, static_cast<const float*>(w2),
                                              b2, score_raw, s),
                    name);
}

static int seq_rmsnorm_common(const char* name, const float* score_raw, int B, int N, int r, int p1, float eps_seq,
                              float* score, void* ws, size_t ws_bytes, void* stream) {
  if (B <= 0 || N <= 0) return fail(TG_EINVAL, "%s: B, N must be > 0", name);
  if (r < 0 || r > p1 || p1 > N)
    return fail(TG_EINVAL, "%s: prunable span [%d, %d) outside [0, N=%d]", name, r, p1, N);
  if (!score_raw || !score) return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!aligned4(score_raw) || !aligned4(score)) return fail(TG_EINVAL, "%s: misaligned pointer", name);
  if (!(eps_seq >= 0.0f)) return fail(TG_EINVAL, "%s: eps_seq must be >= 0", name);
  const size_t need = tg::seq_rmsnorm_workspace(B, N);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
  }
  return hip_status(tg::launch_seq_rmsnorm(score_raw, B, N, r, p1, eps_seq, score, ws,
                                           reinterpret_cast<hipStream_t>(stream)),
                    name);
}

static int topk_select_common(const char* name, const float* score, int B, int N, int r, int p1, int K, uint8_t* keep,
                              void* ws, size_t ws_bytes, void* stream) {
  if (B <= 0 || N <= 0) return fail(TG_EINVAL, "%s: B, N must be > 0", name);
  if (r < 0 || r > p1 || p1 > N)
    return fail(TG_EINVAL, "%s: prunable span [%d, %d) outside [0, N=%d]", name, r, p1, N);
  if (K < 0) return fail(TG_EINVAL, "%s: K=%d must be >= 0", name, K);
  if (!score || !keep) return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!aligned4(score)) return fail(TG_EINVAL, "%s: misaligned score", name);
  const size_t need = tg::topk_select_workspace(B, N);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
  }
  return hip_status(tg::launch_topk_select(score, B, N, r, p1, K, keep, ws, reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_compact(const void* resid, int dt, int B, int N, int d, const uint8_t* keep, const float* score, int M,
               int32_t* kept_idx, void* resid_out, float* score_out, void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  if (dt != TG_BF16 && dt != TG_F32) return fail(TG_EINVAL, "tg_compact: unknown dtype %d", dt);
  if (B <= 0 || N <= 0 || d <= 0) return fail(TG_EINVAL, "tg_compact: B, N, d must be > 0");
  if (M < 0 || M > N) return fail(TG_EINVAL, "tg_compact: M=%d outside [0, N=%d]", M, N);
  if (!resid || !keep || !score || (M > 0 && (!kept_idx || !resid_out || !score_out)))
    return fail(TG_EINVAL, "tg_compact: null pointer argument");
  const size_t row_bytes = (size_t)d * dt_size(dt);
  if (row_bytes % 16 != 0) return fail(TG_EUNSUPPORTED, "tg_compact: row bytes must be a multiple of 16");
  if (!aligned16(resid) || (M > 0 && !aligned16(resid_out)) || !aligned4(score) ||
      (M > 0 && (!aligned4(kept_idx) || !aligned4(score_out))))
    return fail(TG_EINVAL, "tg_compact: misaligned pointer");
  return hip_status(tg::launch_compact(resid, row_bytes, B, N, keep, score, M, kept_idx, resid_out, score_out,
                                       reinterpret_cast<hipStream_t>(stream)),
                    "tg_compact");
}

static int gate_select_common(const char* name, const float* score_raw, int B, int N, int r, int p1, float eps_seq,
                              int K, const void* resid, int dt, int d, float* score, uint8_t* keep, int32_t* kept_idx,
                              void* resid_out, float* score_out, void* ws, size_t ws_bytes, void* stream) {
  if (dt != TG_BF16 && dt != TG_F32) return fail(TG_EINVAL, "%s: unknown dtype %d", name, dt);
  if (B <= 0 || N <= 0 || d <= 0) return fail(TG_EINVAL, "%s: B, N, d must be > 0", name);
  if (r < 0 || r > p1 || p1 > N)
    return fail(TG_EINVAL, "%s: prunable span [%d, %d) outside [0, N=%d]", name, r, p1, N);
  if (K < 0) return fail(TG_EINVAL, "%s: K=%d must be >= 0", name, K);
  if (!(eps_seq >= 0.0f)) return fail(TG_EINVAL, "%s: eps_seq must be >= 0", name);
  const int P = p1 - r;
  const int M = N - P + (K < P ? K : P);
  if (!score_raw || !score || !keep || !resid || (M > 0 && (!kept_idx || !resid_out || !score_out)))
    return fail(TG_EINVAL, "%s: null pointer argument", name);
  const size_t row_bytes = (size_t)d * dt_size(dt);
  if (row_bytes % 16 != 0) return fail(TG_EUNSUPPORTED, "%s: row bytes must be a multiple of 16", name);
  if (!aligned4(score_raw) || !aligned4(score) || !aligned16(resid) ||
      (M > 0 && (!aligned16(resid_out) || !aligned4(kept_idx) || !aligned4(score_out))))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  const size_t need = tg::gate_select_workspace(B, N);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
  }
  return hip_status(tg::launch_gate_select(score_raw, B, N, r, p1, eps_seq, K, resid, row_bytes, score, keep, kept_idx,
                                           resid_out, score_out, ws, reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_gate_score(const void* resid, int dt, int B, int N, int d, int r, const void* norm_w, float eps_row,
                  const void* W1, const float* b1, int h, const void* w2, const float* b2, float* score_raw,
                  void* ws, size_t ws_bytes, void* stream) {
  return gate_score_common("tg_gate_score", resid, dt, B, N, d, r, N, nullptr, nullptr, norm_w, eps_row, W1, b1, h, w2, b2, score_raw,
                           ws, ws_bytes, stream);
}

int tg_gate_fold_weights(const void* W1, const void* norm_w, int dt, int h, int d, void* W1_folded,
                         size_t folded_bytes, void* stream) {
  const char* name = "tg_gate_fold_weights";
  if (dt != TG_BF16) return fail(TG_EUNSUPPORTED, "%s: only the bf16 scorer takes folded weights", name);
  if (d <= 0 || h <= 0) return fail(TG_EINVAL, "%s: d, h must be > 0", name);
  if (d % 64 != 0) return fail(TG_EUNSUPPORTED, "%s: bf16 needs d %% 64 == 0 (d=%d)", name, d);
  if (h != 64 && h != 128 && h != 256)
    return fail(TG_EUNSUPPORTED, "%s: bf16 supports h in {64,128,256} (h=%d)", name, h);
  if (!W1 || !norm_w || !W1_folded) return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!aligned16(W1) || !aligned16(norm_w) || !aligned16(W1_folded))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  const size_t need = tg::gate_score_workspace(h, d);
  if (folded_bytes < need) return fail(TG_EINVAL, "%s: %zu bytes needed, %zu given", name, need, folded_bytes);
  return hip_status(tg::launch_gate_fold(static_cast<const uint16_t*>(W1), static_cast<const uint16_t*>(norm_w), h,
                                         d, W1_folded, reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_gate_score_folded(const void* resid, int dt, int B, int N, int d, int r, const void* W1_folded,
                         float eps_row, const float* b1, int h, const void* w2, const float* b2, float* score_raw,
                         void* stream) {
  const char* name = "tg_gate_score_folded";
  if (dt != TG_BF16) return fail(TG_EUNSUPPORTED, "%s: only the bf16 scorer takes folded weights", name);
  if (B <= 0 || N <= 0 || d <= 0 || h <= 0) return fail(TG_EINVAL, "%s: B, N, d, h must be > 0", name);
  if (r < 0 || r > N) return fail(TG_EINVAL, "%s: r=%d outside [0, N=%d]", name, r, N);
  if (!resid || !W1_folded || !b1 || !w2 || !b2 || !score_raw) return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!(eps_row >= 0.0f)) return fail(TG_EINVAL, "%s: eps_row must be >= 0", name);
  if ((long long)B * N * d > (1LL << 40)) return fail(TG_EINVAL, "%s: tensor too large", name);
  if (!aligned16(resid) || !aligned16(W1_folded) || !aligned4(score_raw) || !aligned4(b1) || !aligned4(b2))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  if (d % 64 != 0) return fail(TG_EUNSUPPORTED, "%s: bf16 needs d %% 64 == 0 (d=%d)", name, d);
  if (h != 64 && h != 128 && h != 256)
    return fail(TG_EUNSUPPORTED, "%s: bf16 supports h in {64,128,256} (h=%d)", name, h);
  if ((size_t)(N - r) * d * 2 > 0x7FFFFFFFull) return fail(TG_EUNSUPPORTED, "%s: a batch row above 2 GiB", name);
  return hip_status(tg::launch_gate_score_folded(static_cast<const uint16_t*>(resid), B, N, d, r, N, nullptr,
                                                 nullptr, eps_row, static_cast<const uint16_t*>(W1_folded), b1, h,
                                                 static_cast<const uint16_t*>(w2), b2, score_raw,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_gate_score_noalloc(const void* resid, int dt, int B, int N, int d, int r, const void* norm_w, float eps_row,
                          const void* W1, const float* b1, int h, const void* w2, const float* b2, float* score_raw,
                          void* stream) {
  return gate_score_common("tg_gate_score_noalloc", resid, dt, B, N, d, r, N, nullptr, nullptr, norm_w, eps_row, W1,
                           b1, h, w2, b2, score_raw, nullptr, 0, stream, true);
}

int tg_gate(const void* resid, int dt, int B, int N, int d, int r, const void* W1_folded, float eps_row,
            const float* b1, int h, const void* w2, const float* b2, float eps_seq, int K, float* score_raw,
            float* score, uint8_t* keep, int32_t* kept_idx, void* resid_out, float* score_out, void* ws,
            size_t ws_bytes, void* stream) {
  const char* name = "tg_gate";
  if (dt != TG_BF16) return fail(TG_EUNSUPPORTED, "%s: the fused gate takes a bf16 residual", name);
  if (B <= 0 || B > 65535 || N <= 0 || d <= 0 || h <= 0) return fail(TG_EINVAL, "%s: bad sizes", name);
  if (N > 32768) return fail(TG_EUNSUPPORTED, "%s: rows of up to 32768 tokens (N=%d)", name, N);
  if (r < 0 || r > N) return fail(TG_EINVAL, "%s: r=%d outside [0, N=%d]", name, r, N);
  if (K < 0) return fail(TG_EINVAL, "%s: K=%d must be >= 0", name, K);
  if (!(eps_row >= 0.0f) || !(eps_seq >= 0.0f)) return fail(TG_EINVAL, "%s: eps_row and eps_seq must be >= 0", name);
  const int P = N - r;
  const int M = N - P + (K < P ? K : P);
  if (!resid || !W1_folded || !b1 || !w2 || !b2 || !score_raw || !score || !keep ||
      (M > 0 && (!kept_idx || !resid_out || !score_out)))
    return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!aligned16(resid) || !aligned16(W1_folded) || !aligned4(b1) || !aligned4(b2) || !aligned4(score_raw) ||
      !aligned4(score) || (M > 0 && (!aligned16(resid_out) || !aligned4(kept_idx) || !aligned4(score_out))))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  if (d % 64 != 0) return fail(TG_EUNSUPPORTED, "%s: needs d %% 64 == 0 (d=%d)", name, d);
  if (h != 64 && h != 128 && h != 256) return fail(TG_EUNSUPPORTED, "%s: h in {64,128,256} (h=%d)", name, h);
  // one counting word per batch row, zero on entry and left zero
  if (!ws || ws_bytes < (size_t)B * 4) return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name,
                                                   (size_t)B * 4, ws_bytes);
  if (!aligned4(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
  return hip_status(tg::launch_gate_fused(static_cast<const uint16_t*>(resid), B, N, d, r,
                                          static_cast<const uint16_t*>(W1_folded), eps_row, b1, h,
                                          static_cast<const uint16_t*>(w2), b2, eps_seq, K, score_raw, score, keep,
                                          kept_idx, static_cast<uint16_t*>(resid_out), score_out,
                                          static_cast<uint32_t*>(ws), reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_gate_score_span(const void* resid, int dt, int B, int N, int d, int span_begin, int span_end,
                       const void* norm_w, float eps_row, const void* W1, const float* b1, int h, const void* w2,
                       const float* b2, float* score_raw, void* ws, size_t ws_bytes, void* stream) {
  return gate_score_common("tg_gate_score_span", resid, dt, B, N, d, span_begin, span_end, nullptr, nullptr, norm_w, eps_row, W1, b1,
                           h, w2, b2, score_raw, ws, ws_bytes, stream);
}

int tg_seq_rmsnorm(const float* score_raw, int B, int N, int r, float eps_seq, float* score, void* ws,
                   size_t ws_bytes, void* stream) {
  return seq_rmsnorm_common("tg_seq_rmsnorm", score_raw, B, N, r, N, eps_seq, score, ws, ws_bytes, stream);
}

int tg_seq_rmsnorm_span(const float* score_raw, int B, int N, int span_begin, int span_end, float eps_seq,
                        float* score, void* ws, size_t ws_bytes, void* stream) {
  return seq_rmsnorm_common("tg_seq_rmsnorm_span", score_raw, B, N, span_begin, span_end, eps_seq, score, ws,
                            ws_bytes, stream);
}

int tg_topk_select(const float* score, int B, int N, int r, int K, uint8_t* keep, void* ws, size_t ws_bytes,
                   void* stream) {
  return topk_select_common("tg_topk_select", score, B, N, r, N, K, keep, ws, ws_bytes, stream);
}

int tg_topk_select_span(const float* score, int B, int N, int span_begin, int span_end, int K, uint8_t* keep,
                        void* ws, size_t ws_bytes, void* stream) {
  return topk_select_common("tg_topk_select_span", score, B, N, span_begin, span_end, K, keep, ws, ws_bytes, stream);
}

int tg_gate_select(const float* score_raw, int B, int N, int r, float eps_seq, int K, const void* resid, int dt,
                   int d, float* score, uint8_t* keep, int32_t* kept_idx, void* resid_out, float* score_out,
                   void* ws, size_t ws_bytes, void* stream) {
  return gate_select_common("tg_gate_select", score_raw, B, N, r, N, eps_seq, K, resid, dt, d, score, keep, kept_idx,
                            resid_out, score_out, ws, ws_bytes, stream);
}

int tg_gate_select_span(const float* score_raw, int B, int N, int span_begin, int span_end, float eps_seq, int K,
                        const void* resid, int dt, int d, float* score, uint8_t* keep, int32_t* kept_idx,
                        void* resid_out, float* score_out, void* ws, size_t ws_bytes, void* stream) {
  return gate_select_common("tg_gate_select_span", score_raw, B, N, span_begin, span_end, eps_seq, K, resid, dt, d,
                            score, keep, kept_idx, resid_out, score_out, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

int gated_attention_common(const char* name, const void* q, const void* k, const void* v, int B, int M, int Hq,
                           int Hkv, int d_h, const float* key_score, const int32_t* pos, const float* gain,
                           const float* temp, float sm_scale, double rope_base, void* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream,
                           bool launch = true, const int32_t* m_dev = nullptr) {
  if (B <= 0 || M < 0 || Hq <= 0 || Hkv <= 0) return fail(TG_EINVAL, "%s: bad sizes", name);
  if (Hq % Hkv != 0) return fail(TG_EINVAL, "%s: Hq=%d not a multiple of Hkv=%d", name, Hq, Hkv);
  if (M == 0) return TG_OK;
  if (!q || !k || !v || !key_score || !pos || !gain || !temp || !out)
    return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(key_score) ||
      !aligned4(pos) || !aligned4(gain) || !aligned4(temp) || (lse && !aligned4(lse)) || !aligned4(m_dev))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  if (!(sm_scale > 0.0f)) return fail(TG_EINVAL, "%s: sm_scale must be > 0", name);
  if (d_h != 64 && d_h != 128) return fail(TG_EUNSUPPORTED, "%s: d_h=%d not in {64,128}", name, d_h);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4) return fail(TG_EUNSUPPORTED, "%s: Hq/Hkv=%d not in {1,2,4}", name, G);
  const size_t need = rope_base > 0.0 ? tg::gated_attention_rope_workspace(B, M, Hq, Hkv, d_h)
                                      : tg::gated_attention_workspace(B, M, Hq, Hkv, d_h);
  if (!ws || ws_bytes < need)
    return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
  if (!aligned16(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
  if (!launch) return TG_OK;
  return hip_status(tg::launch_gated_attention(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                               static_cast<const uint16_t*>(v), B, M, Hq, Hkv, d_h, key_score,
                                               pos, gain, temp, sm_scale, rope_base, static_cast<uint16_t*>(out),
                                               lse, ws, reinterpret_cast<hipStream_t>(stream), m_dev),
                    name);
}

}  // namespace

extern "C" {

int tg_gated_attention(const void* q, const void* k, const void* v, int B, int M, int Hq, int Hkv, int d_h,
                       const float* key_score, const int32_t* pos, const float* gain, const float* temp,
                       float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return gated_attention_common("tg_gated_attention", q, k, v, B, M, Hq, Hkv, d_h, key_score, pos, gain, temp,
                                sm_scale, 0.0, out, lse, ws, ws_bytes, stream);
}

int tg_gated_attention_padded(const void* q, const void* k, const void* v, int B, int M_pad,
                              const int32_t* kept_count, int Hq, int Hkv, int d_h, const float* key_score,
                              const int32_t* pos, const float* gain, const float* temp, float sm_scale, void* out,
                              float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!kept_count) return fail(TG_EINVAL, "tg_gated_attention_padded: null pointer argument");
  return gated_attention_common("tg_gated_attention_padded", q, k, v, B, M_pad, Hq, Hkv, d_h, key_score, pos, gain,
                                temp, sm_scale, 0.0, out, lse, ws, ws_bytes, stream, true, kept_count);
}

int tg_gated_attention_rope(const void* q, const void* k, const void* v, int B, int M, int Hq, int Hkv, int d_h,
                            const float* key_score, const int32_t* pos, const float* gain, const float* temp,
                            float sm_scale, double rope_base, void* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!(rope_base > 1.0) || !(rope_base < 1e300))
    return fail(TG_EINVAL, "tg_gated_attention_rope: rope_base must be finite and > 1");
  return gated_attention_common("tg_gated_attention_rope", q, k, v, B, M, Hq, Hkv, d_h, key_score, pos, gain,
                                temp, sm_scale, rope_base, out, lse, ws, ws_bytes, stream);
}

static int attention_backward_common(const char* name, const void* q, const void* k, const void* v, const void* out,
                                     const float* lse, const void* d_out, int B, int M, int Hq, int Hkv, int d_h,
                                     const float* key_score, const int32_t* pos, const float* gain, const float* temp,
                                     float sm_scale, double rope_base, void* d_q, void* d_k, void* d_v,
                                     float* d_key_score, float* d_gain, float* d_temp, void* ws, size_t ws_bytes,
                                     void* stream, bool launch = true) {
  if (B <= 0 || B > 65535 || M < 0 || Hq <= 0 || Hkv <= 0) return fail(TG_EINVAL, "%s: bad sizes", name);
  if (Hq % Hkv != 0) return fail(TG_EINVAL, "%s: Hq=%d not a multiple of Hkv=%d", name, Hq, Hkv);
  if (!gain || !temp || !d_gain || !d_temp) return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!aligned4(gain) || !aligned4(temp) || !aligned4(d_gain) || !aligned4(d_temp))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  if (d_h != 64 && d_h != 128) return fail(TG_EUNSUPPORTED, "%s: d_h=%d not in {64,128}", name, d_h);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4) return fail(TG_EUNSUPPORTED, "%s: Hq/Hkv=%d not in {1,2,4}", name, G);
  if (M > 0) {
    if (!q || !k || !v || !out || !lse || !d_out || !key_score || !pos || !d_q || !d_k || !d_v || !d_key_score)
      return fail(TG_EINVAL, "%s: null pointer argument", name);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(d_out) ||
        !aligned16(d_q) || !aligned16(d_k) || !aligned16(d_v) || !aligned4(lse) || !aligned4(key_score) ||
        !aligned4(pos) || !aligned4(d_key_score))
      return fail(TG_EINVAL, "%s: misaligned pointer", name);
    if (!(sm_scale > 0.0f)) return fail(TG_EINVAL, "%s: sm_scale must be > 0", name);
    // buffer-resource ranges are 32-bit: every per-head plane must stay below 2 GiB
    const long long Mp = (M + 63LL) / 64 * 64;
    if ((long long)M * Hq * d_h * 2 >= (1LL << 31) || Mp * d_h * 2 >= (1LL << 31) ||
        (long long)B * Hq * Mp * 4 >= (1LL << 31))
      return fail(TG_EUNSUPPORTED, "%s: M=%d too large", name, M);
    const size_t need = rope_base > 0.0 ? tg::gated_attention_rope_backward_workspace(B, M, Hq, Hkv, d_h)
                                        : tg::gated_attention_backward_workspace(B, M, Hq, Hkv, d_h);
    if (!ws || ws_bytes < need)
      return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
  }
  if (!launch) return TG_OK;
  return hip_status(
      tg::launch_gated_attention_backward(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
          static_cast<const uint16_t*>(out), lse, static_cast<const uint16_t*>(d_out), B, M, Hq, Hkv, d_h, key_score,
          pos, gain, temp, sm_scale, rope_base, static_cast<uint16_t*>(d_q), static_cast<uint16_t*>(d_k),
          static_cast<uint16_t*>(d_v), d_key_score, d_gain, d_temp, ws, reinterpret_cast<hipStream_t>(stream)),
      name);
}

int tg_gated_attention_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                                const void* d_out, int B, int M, int Hq, int Hkv, int d_h, const float* key_score,
                                const int32_t* pos, const float* gain, const float* temp, float sm_scale, void* d_q,
                                void* d_k, void* d_v, float* d_key_score, float* d_gain, float* d_temp, void* ws,
                                size_t ws_bytes, void* stream) {
  return attention_backward_common("tg_gated_attention_backward", q, k, v, out, lse, d_out, B, M, Hq, Hkv, d_h,
                                   key_score, pos, gain, temp, sm_scale, 0.0, d_q, d_k, d_v, d_key_score, d_gain,
                                   d_temp, ws, ws_bytes, stream);
}

int tg_gated_attention_rope_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                                     const void* d_out, int B, int M, int Hq, int Hkv, int d_h,
                                     const float* key_score, const int32_t* pos, const float* gain,
                                     const float* temp, float sm_scale, double rope_base, void* d_q, void* d_k,
                                     void* d_v, float* d_key_score, float* d_gain, float* d_temp, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (!(rope_base > 1.0) || !(rope_base < 1e300))
    return fail(TG_EINVAL, "tg_gated_attention_rope_backward: rope_base must be finite and > 1");
  return attention_backward_common("tg_gated_attention_rope_backward", q, k, v, out, lse, d_out, B, M, Hq, Hkv, d_h,
                                   key_score, pos, gain, temp, sm_scale, rope_base, d_q, d_k, d_v, d_key_score,
                                   d_gain, d_temp, ws, ws_bytes, stream);
}

int tg_kv_cache_prune(const void* k_cache, const void* v_cache, int n_layers, int B, int N, int Hkv, int d_h,
                      const int32_t* kept_idx, int M, void* k_out, void* v_out, void* stream) {
  const char* name = "tg_kv_cache_prune";
  if (n_layers < 0 || n_layers > 32767 || B <= 0 || B > 65535 || N <= 0 || Hkv <= 0 || d_h <= 0)
    return fail(TG_EINVAL, "%s: bad sizes", name);
  if (d_h % 8 != 0) return fail(TG_EUNSUPPORTED, "%s: d_h=%d not a multiple of 8", name, d_h);
  if (M < 0 || M > N) return fail(TG_EINVAL, "%s: M=%d outside [0, N=%d]", name, M, N);
  if (M == 0 || n_layers == 0) return TG_OK;
  if (!k_cache || !v_cache || !kept_idx || !k_out || !v_out) return fail(TG_EINVAL, "%s: null pointer argument", name);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out) || !aligned4(kept_idx))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  return hip_status(tg::launch_kv_cache_prune(k_cache, v_cache, n_layers, B, N, Hkv, d_h, kept_idx, M, k_out, v_out,
                                              reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_gate_select_varlen(const float* score_raw, int B, int N, const int32_t* seq_len, const int32_t* span_begin,
                          const int32_t* span_end, const int32_t* K, const int32_t* cu_kept, int max_kept,
                          float eps_seq, const void* resid, int dt, int d, float* score, uint8_t* keep,
                          int32_t* kept_idx, void* resid_out, float* score_out, void* ws, size_t ws_bytes,
                          void* stream) {
  const char* name = "tg_gate_select_varlen";
  if (dt != TG_BF16 && dt != TG_F32) return fail(TG_EINVAL, "%s: unknown dtype %d", name, dt);
  if (B <= 0 || B > 65535 || N <= 0 || d <= 0) return fail(TG_EINVAL, "%s: B, N, d must be > 0", name);
  // rows longer than 32768 tokens take the sliced kernels and their workspace
  const size_t need = tg::gate_select_workspace(B, N);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
  if (need > 0 && !aligned16(ws)) return fail(TG_EINVAL, "%s: misaligned workspace", name);
  if (max_kept < 0 || max_kept > N) return fail(TG_EINVAL, "%s: max_kept=%d outside [0, N=%d]", name, max_kept, N);
  if (!(eps_seq >= 0.0f)) return fail(TG_EINVAL, "%s: eps_seq must be >= 0", name);
  if (!score_raw || !seq_len || !span_begin || !span_end || !K || !cu_kept || !resid || !score || !keep ||
      !kept_idx || !resid_out || !score_out)
    return fail(TG_EINVAL, "%s: null pointer argument", name);
  const size_t row_bytes = (size_t)d * dt_size(dt);
  if (row_bytes % 16 != 0) return fail(TG_EUNSUPPORTED, "%s: row bytes must be a multiple of 16", name);
  if (!aligned4(score_raw) || !aligned4(score) || !aligned16(resid) || !aligned16(resid_out) ||
      !aligned4(kept_idx) || !aligned4(score_out) || !aligned4(seq_len) || !aligned4(span_begin) ||
      !aligned4(span_end) || !aligned4(K) || !aligned4(cu_kept))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  return hip_status(tg::launch_gate_select_varlen(score_raw, B, N,
                                                  tg::VarlenRows{seq_len, span_begin, span_end, K, cu_kept}, max_kept,
                                                  eps_seq, resid, row_bytes, score, keep, kept_idx, resid_out,
                                                  score_out, ws, reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_gate_select_padded(const float* score_raw, int B, int N, int r, float eps_seq, const int32_t* K, int M_pad,
                          const void* resid, int dt, int d, float* score, uint8_t* keep, int32_t* kept_idx,
                          void* resid_out, float* score_out, int32_t* kept_count, void* stream) {
  const char* name = "tg_gate_select_padded";
  if (dt != TG_BF16 && dt != TG_F32) return fail(TG_EINVAL, "%s: unknown dtype %d", name, dt);
  if (B <= 0 || B > 65535 || N <= 0 || d <= 0) return fail(TG_EINVAL, "%s: B, N, d must be > 0", name);
  if (N > 32768) return fail(TG_EUNSUPPORTED, "%s: rows of up to 32768 tokens (N=%d)", name, N);
  if (r < 0 || r > N) return fail(TG_EINVAL, "%s: r=%d outside [0, N=%d]", name, r, N);
  if (M_pad < r || M_pad > N)
    return fail(TG_EINVAL, "%s: M_pad=%d outside [r=%d, N=%d]", name, M_pad, r, N);
  if (!(eps_seq >= 0.0f)) return fail(TG_EINVAL, "%s: eps_seq must be >= 0", name);
  if (!score_raw || !K || !resid || !score || !keep || !kept_idx || !resid_out || !score_out || !kept_count)
    return fail(TG_EINVAL, "%s: null pointer argument", name);
  const size_t row_bytes = (size_t)d * dt_size(dt);
  if (row_bytes % 16 != 0) return fail(TG_EUNSUPPORTED, "%s: row bytes must be a multiple of 16", name);
  if (!aligned4(score_raw) || !aligned4(score) || !aligned16(resid) || !aligned16(resid_out) ||
      !aligned4(kept_idx) || !aligned4(score_out) || !aligned4(K) || !aligned4(kept_count))
    return fail(TG_EINVAL, "%s: misaligned pointer", name);
  return hip_status(tg::launch_gate_select_padded(score_raw, B, N, r, eps_seq, K, M_pad, resid, row_bytes, score,
                                                  keep, kept_idx, resid_out, score_out, kept_count,
                                                  reinterpret_cast<hipStream_t>(stream)),
                    name);
}

int tg_gate_score_varlen(const void* resid, int dt, int B, int N, int d, const int32_t* span_begin,
                         const int32_t* span_end, int max_span, const void* norm_w, float eps_row, const void* W1,
                         const float* b1, int h, const void* w2, const float* b2, float* score_raw, void* ws,
                         size_t ws_bytes, void* stream) {
  if (max_span < 0 || max_span > N)
    return fail(TG_EINVAL, "tg_gate_score_varlen: max_span=%d outside [0, N=%d]", max_span, N);
  if (!span_begin || !span_end || !aligned4(span_begin) || !aligned4(span_end))
    return fail(TG_EINVAL, "tg_gate_score_varlen: span arrays must be 4-byte aligned device pointers");
  return gate_score_common("tg_gate_score_varlen", resid, dt, B, N, d, 0, max_span, span_begin, span_end, norm_w,
                           eps_row, W1, b1, h, w2, b2, score_raw, ws, ws_bytes, stream);
}

static int attention_varlen_common(const char* name, const void* q, const void* k, const void* v, int B,
                                   const int32_t* cu_seqlens, int Hq, int Hkv, int d_h, const float* key_score,
                                   const int32_t* pos, const float* gain, const float* temp, float sm_scale,
                                   double rope_base, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (B <= 0 || !cu_seqlens) return fail(TG_EINVAL, "%s: B must be > 0 and cu_seqlens given", name);
  if (cu_seqlens[0] != 0) return fail(TG_EINVAL, "%s: cu_seqlens[0] must be 0", name);
  for (int b = 0; b < B; ++b)
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return fail(TG_EINVAL, "%s: cu_seqlens must be non-decreasing", name);
  if (Hq <= 0 || Hkv <= 0) return fail(TG_EINVAL, "%s: bad sizes", name);
  if (Hq % Hkv != 0) return fail(TG_EINVAL, "%s: Hq=%d not a multiple of Hkv=%d", name, Hq, Hkv);
  if (d_h != 64 && d_h != 128) return fail(TG_EUNSUPPORTED, "%s: d_h=%d not in {64,128}", name, d_h);
  const size_t slots = tg::gated_attention_varlen_slots(B, cu_seqlens);
  if (slots == 0) return TG_OK;
  if (slots > 0x7FFFFFFF) return fail(TG_EINVAL, "%s: %zu padded rows exceed the 32-bit index range", name, slots);
  // all sequences' V^T copies and key-score terms sit side by side (then,
  // with the rotary embedding, the rotated k by packed row and the angle
  // table by padded slot)
  const size_t need = rope_base > 0.0 ? tg::gated_attention_rope_varlen_workspace(B, cu_seqlens, Hq, Hkv, d_h)
                                      : tg::gated_attention_workspace(1, (int)slots, Hq, Hkv, d_h);
  if (!ws || ws_bytes < need) return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
  // each sequence is validated as a batch of one; then the batch is launched
  for (int b = 0; b < B; ++b) {
    const size_t t0 = (size_t)cu_seqlens[b];
    const int m = cu_seqlens[b + 1] - cu_seqlens[b];
    if (m == 0) continue;
    const int rc = gated_attention_common(
        name, static_cast<const uint16_t*>(q) + t0 * Hq * d_h, static_cast<const uint16_t*>(k) + t0 * Hkv * d_h,
        static_cast<const uint16_t*>(v) + t0 * Hkv * d_h, 1, m, Hq, Hkv, d_h, key_score + t0, pos + t0, gain, temp,
        sm_scale, rope_base, static_cast<uint16_t*>(out) + t0 * Hq * d_h, lse ? lse + t0 * Hq : nullptr, ws,
        ws_bytes, stream, false);
    if (rc != TG_OK) return rc;
  }
  return hip_status(tg::launch_gated_attention_varlen(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), B,
      cu_seqlens, Hq, Hkv, d_h, key_score, pos, gain, temp, sm_scale, rope_base, static_cast<uint16_t*>(out), lse,
      ws, static_cast<hipStream_t>(stream)), name);
}

int tg_gated_attention_varlen(const void* q, const void* k, const void* v, int B, const int32_t* cu_seqlens, int Hq,
                              int Hkv, int d_h, const float* key_score, const int32_t* pos, const float* gain,
                              const float* temp, float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                              void* stream) {
  return attention_varlen_common("tg_gated_attention_varlen", q, k, v, B, cu_seqlens, Hq, Hkv, d_h, key_score, pos,
                                 gain, temp, sm_scale, 0.0, out, lse, ws, ws_bytes, stream);
}

int tg_gated_attention_rope_varlen(const void* q, const void* k, const void* v, int B, const int32_t* cu_seqlens,
                                   int Hq, int Hkv, int d_h, const float* key_score, const int32_t* pos,
                                   const float* gain, const float* temp, float sm_scale, double rope_base, void* out,
                                   float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!(rope_base > 1.0) || !(rope_base < 1e300))
    return fail(TG_EINVAL, "tg_gated_attention_rope_varlen: rope_base must be finite and > 1");
  return attention_varlen_common("tg_gated_attention_rope_varlen", q, k, v, B, cu_seqlens, Hq, Hkv, d_h, key_score,
                                 pos, gain, temp, sm_scale, rope_base, out, lse, ws, ws_bytes, stream);
}

static int attention_backward_varlen_common(const char* name, const void* q, const void* k, const void* v,
                                            const void* out, const float* lse, const void* d_out, int B,
                                            const int32_t* cu_seqlens, int Hq, int Hkv, int d_h,
                                            const float* key_score, const int32_t* pos, const float* gain,
                                            const float* temp, float sm_scale, double rope_base, void* d_q,
                                            void* d_k, void* d_v, float* d_key_score, float* d_gain, float* d_temp,
                                            void* ws, size_t ws_bytes, void* stream) {
  if (B <= 0 || !cu_seqlens) return fail(TG_EINVAL, "%s: B must be > 0 and cu_seqlens given", name);
  if (cu_seqlens[0] != 0) return fail(TG_EINVAL, "%s: cu_seqlens[0] must be 0", name);
  for (int b = 0; b < B; ++b)
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return fail(TG_EINVAL, "%s: cu_seqlens must be non-decreasing", name);
  if ((size_t)cu_seqlens[B] + 63 * (size_t)B > 0x7FFFFFFF)
    return fail(TG_EINVAL, "%s: the padded rows exceed the 32-bit index range", name);
  if (Hq <= 0 || Hkv <= 0) return fail(TG_EINVAL, "%s: bad sizes", name);  // (before any size is derived from them)
  if (Hq % Hkv != 0) return fail(TG_EINVAL, "%s: Hq=%d not a multiple of Hkv=%d", name, Hq, Hkv);
  if (d_h != 64 && d_h != 128) return fail(TG_EUNSUPPORTED, "%s: d_h=%d not in {64,128}", name, d_h);
  // every sequence's row constants and partials sit side by side (then, for
  // the rotary variant, the rotated q and k and their fp32 gradients)
  const size_t need = rope_base > 0.0 && cu_seqlens[B] > 0
                          ? tg::gated_attention_rope_backward_varlen_workspace(B, cu_seqlens, Hq, Hkv, d_h)
                          : tg::gated_attention_backward_varlen_workspace(B, cu_seqlens, Hq, Hkv);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TG_EINVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, ws_bytes);
  if (!d_gain || !d_temp) return fail(TG_EINVAL, "%s: null pointer argument", name);
  // each sequence is validated as a batch of one; then the batch is launched
  // (sequence b's gain and temperature gradients go to row b)
  for (int b = 0; b < B; ++b) {
    const size_t t0 = (size_t)cu_seqlens[b];
    const int m = cu_seqlens[b + 1] - cu_seqlens[b];
    const size_t qo = t0 * Hq * d_h, ko = t0 * Hkv * d_h;
    const int rc = attention_backward_common(
        name, static_cast<const uint16_t*>(q) + qo, static_cast<const uint16_t*>(k) + ko,
        static_cast<const uint16_t*>(v) + ko, static_cast<const uint16_t*>(out) + qo, lse ? lse + t0 * Hq : nullptr,
        static_cast<const uint16_t*>(d_out) + qo, 1, m, Hq, Hkv, d_h, key_score + t0, pos + t0, gain, temp, sm_scale,
        0.0, static_cast<uint16_t*>(d_q) + qo, static_cast<uint16_t*>(d_k) + ko, static_cast<uint16_t*>(d_v) + ko,
        d_key_score + t0, d_gain + (size_t)b * Hq, d_temp + (size_t)b * Hq, ws, ws_bytes, stream, false);
    if (rc != TG_OK) return rc;
  }
  return hip_status(tg::launch_gated_attention_backward_varlen(
                        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                        static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(out), lse,
                        static_cast<const uint16_t*>(d_out), B, cu_seqlens, Hq, Hkv, d_h, key_score, pos, gain, temp,
                        sm_scale, rope_base, static_cast<uint16_t*>(d_q), static_cast<uint16_t*>(d_k),
                        static_cast<uint16_t*>(d_v), d_key_score, d_gain, d_temp, ws,
                        static_cast<hipStream_t>(stream)),
                    name);
}

int tg_gated_attention_backward_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse,
                                       const void* d_out, int B, const int32_t* cu_seqlens, int Hq, int Hkv, int d_h,
                                       const float* key_score, const int32_t* pos, const float* gain,
                                       const float* temp, float sm_scale, void* d_q, void* d_k, void* d_v,
                                       float* d_key_score, float* d_gain, float* d_temp, void* ws, size_t ws_bytes,
                                       void* stream) {
  return attention_backward_varlen_common("tg_gated_attention_backward_varlen", q, k, v, out, lse, d_out, B,
                                          cu_seqlens, Hq, Hkv, d_h, key_score, pos, gain, temp, sm_scale, 0.0, d_q,
                                          d_k, d_v, d_key_score, d_gain, d_temp, ws, ws_bytes, stream);
}

int tg_gated_attention_rope_backward_varlen(const void* q, const void* k, const void* v, const void* out,
                                            const float* lse, const void* d_out, int B, const int32_t* cu_seqlens,
                                            int Hq, int Hkv, int d_h, const float* key_score, const int32_t* pos,
                                            const float* gain, const float* temp, float sm_scale, double rope_base,
                                            void* d_q, void* d_k, void* d_v, float* d_key_score, float* d_gain,
                                            float* d_temp, void* ws, size_t ws_bytes, void* stream) {
  if (!(rope_base > 1.0) || !(rope_base < 1e300))
    return fail(TG_EINVAL, "tg_gated_attention_rope_backward_varlen: rope_base must be finite and > 1");
  return attention_backward_varlen_common("tg_gated_attention_rope_backward_varlen", q, k, v, out, lse, d_out, B,
                                          cu_seqlens, Hq, Hkv, d_h, key_score, pos, gain, temp, sm_scale, rope_base,
                                          d_q, d_k, d_v, d_key_score, d_gain, d_temp, ws, ws_bytes, stream);
}

}  // extern "C"
