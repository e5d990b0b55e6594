// Gate selection in one call (TokenGate paper, Section 4: sequence RMSNorm of
// the scores, second half of Eq. 3; the Top-K Selector, Eq. 4; compaction of
// the residual stream to the kept set, Appendix C.4): the results of
// tg_seq_rmsnorm, tg_topk_select and tg_compact in sequence, bit for bit.
//
// Rows of up to 32768 tokens take two launches instead of five:
//  * gate_select_kernel, one 1024-thread workgroup per batch row: the row is
//    loaded once, normalised (the shared single-workgroup reduction, so the
//    scores match tg_seq_rmsnorm exactly) and written, its prunable keys go
//    to LDS with the first digit's histogram counted on the way, the shared
//    LDS radix select finds the threshold, and the final pass in index order
//    writes the keep mask, kept_idx and the kept scores through block-wide
//    prefix counts (the non-prunable tokens before the span [r, p1) first,
//    then the kept prunable tokens ascending, then the non-prunable tokens
//    after the span).
//  * the residual row gather of tg_compact, given kept_idx.
// Longer rows run the three separate calls; in a varying-length batch, the
// rows longer than 32768 tokens take their multi-workgroup kernels (which
// skip the short rows) after the one-workgroup kernel (which skips the long
// ones).
#include "gate_select_row.h"
#include "select_device.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = sel::kRowThreads;
static_assert(sel::kRowChunk == kVarlenOneGroupRow, "the one-workgroup row limit");

__global__ __launch_bounds__(kThreads) void gate_select_kernel(const float* score_raw, int N, int r_all, int p1_all,
                                                               float eps, int K_all, VarlenRows vr, float* score,
                                                               uint8_t* __restrict__ keep,
                                                               int32_t* __restrict__ kept_idx,
                                                               float* __restrict__ score_kept) {
  __shared__ __attribute__((aligned(16))) unsigned char s_lds[selrow::kSelLdsBytes];
  selrow::gate_select_row<kThreads>(score_raw, N, r_all, p1_all, eps, K_all, vr, score, keep, kept_idx, score_kept,
                                    blockIdx.x, selrow::carve_sel_lds(s_lds));
}

}  // namespace

size_t gate_select_workspace(int B, int N) {
  if (N <= sel::kRowChunk) return 0;
  const size_t a = seq_rmsnorm_workspace(B, N), t = topk_select_workspace(B, N);
  return a > t ? a : t;  // the two calls use it one after the other
}

hipError_t launch_gate_select(const float* score_raw, int B, int N, int r, int p1, float eps, int K,
                              const void* resid, size_t row_bytes, float* score, uint8_t* keep, int32_t* kept_idx,
                              void* resid_out, float* score_kept, void* ws, hipStream_t s) {
  const int P = p1 - r;
  const int M = N - P + (K < P ? K : P);
  if (N > sel::kRowChunk) {
    hipError_t e = launch_seq_rmsnorm(score_raw, B, N, r, p1, eps, score, ws, s);
    if (e != hipSuccess) return e;
    e = launch_topk_select(score, B, N, r, p1, K, keep, ws, s);
    if (e != hipSuccess) return e;
    return launch_compact(resid, row_bytes, B, N, keep, score, M, kept_idx, resid_out, score_kept, s);
  }
  hipLaunchKernelGGL(gate_select_kernel, dim3(B), dim3(kThreads), 0, s, score_raw, N, r, p1, eps, K, VarlenRows{},
                     score, keep, kept_idx, score_kept);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_compact_gather(resid, row_bytes, B, N, M, kept_idx, resid_out, s);
}

hipError_t launch_gate_select_padded(const float* score_raw, int B, int N, int r, float eps, const int32_t* K,
                                     int pad, const void* resid, size_t row_bytes, float* score, uint8_t* keep,
                                     int32_t* kept_idx, void* resid_out, float* score_kept, int32_t* kept_count,
                                     hipStream_t s) {
  if (N > sel::kRowChunk) return hipErrorInvalidValue;
  VarlenRows vr{nullptr, nullptr, nullptr, K, nullptr, pad, kept_count};
  hipLaunchKernelGGL(gate_select_kernel, dim3(B), dim3(kThreads), 0, s, score_raw, N, r, N, eps, 0, vr, score, keep,
                     kept_idx, score_kept);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_compact_gather_padded(resid, row_bytes, B, N, kept_count, pad, kept_idx, resid_out, s);
}

hipError_t launch_gate_select_varlen(const float* score_raw, int B, int N, VarlenRows vr, int max_kept, float eps,
                                     const void* resid, size_t row_bytes, float* score, uint8_t* keep,
                                     int32_t* kept_idx, void* resid_out, float* score_kept, void* ws,
                                     hipStream_t s) {
  // rows of up to 32768 tokens: one workgroup each (the longer rows return at once)
  hipLaunchKernelGGL(gate_select_kernel, dim3(B), dim3(kThreads), 0, s, score_raw, N, 0, N, eps, 0, vr, score, keep,
                     kept_idx, score_kept);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (N > sel::kRowChunk) {
    // the longer rows: sliced normalisation, chunked selection, compaction
    // scan (each kernel skips the short rows), as the separate calls take
    // them for a uniform batch
    e = launch_seq_rmsnorm_long_rows(score_raw, B, N, vr, eps, score, ws, s);
    if (e != hipSuccess) return e;
    e = launch_topk_select_long_rows(score, B, N, vr, keep, ws, s);
    if (e != hipSuccess) return e;
    e = launch_compact_scan_long_rows(keep, score, B, N, vr, kept_idx, score_kept, s);
    if (e != hipSuccess) return e;
  }
  return launch_compact_gather_varlen(resid, row_bytes, B, N, vr.cu_kept, max_kept, kept_idx, resid_out, s);
}

}  // namespace tg
