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
#include "select_device.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = sel::kRowThreads;
constexpr int kVec = sel::kRowVec;
constexpr int kItems = 16;  // consecutive prunable tokens per thread in the final pass
static_assert(sel::kRowChunk == kVarlenOneGroupRow, "the one-workgroup row limit");

// score_raw and score may alias: every raw score is read before the
// reduction's barriers, and nothing reads score_raw after them.
// With vr.len set, batch row b has its own valid length, span and budget
// (clamped into range: 0 <= span_begin <= span_end <= len <= N, K >= 0) and
// writes its kept tokens at kept_idx + cu_kept[b], at most cu_kept[b + 1] -
// cu_kept[b] of them; tokens at or past len are padding (score 0, not kept).
__global__ __launch_bounds__(kThreads) void gate_select_kernel(const float* score_raw, int N, int r_all, int p1_all,
                                                               float eps, int K_all, VarlenRows vr, float* score,
                                                               uint8_t* __restrict__ keep,
                                                               int32_t* __restrict__ kept_idx,
                                                               float* __restrict__ score_kept) {
  __shared__ uint32_t s_keys[sel::kLdsKeyWords];
  __shared__ uint32_t s_hist[2048];
  __shared__ __attribute__((aligned(16))) uint32_t s_wave[16];
  __shared__ uint32_t s_sel[3];
  __shared__ double s_part[kThreads / 64];
  __shared__ double s_scale;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  int Nb = N, r = r_all, p1 = p1_all, K = K_all;
  if (vr.len != nullptr) {
    const RowSpec rs = varlen_row(vr, b, N);
    if (rs.len > kVarlenOneGroupRow) return;  // a longer row takes the sliced kernels
    Nb = rs.len;
    p1 = rs.p1;
    r = rs.r;
    K = rs.K;
  } else if (vr.K != nullptr) {
    // budget from the device, cut so that the kept set fits the pad rows
    K = min(max(vr.K[b], 0), vr.pad - (N - (p1 - r)));
  }
  const int P = p1 - r;
  const int Kp = K < P ? K : P;
  const int M = Nb - P + Kp;  // kept tokens of this row
  size_t out0 = (size_t)b * M;
  int lim = M;  // ranks this row may write
  if (vr.len != nullptr) {
    out0 = (size_t)max(vr.cu_kept[b], 0);
    lim = min(M, vr.cu_kept[b + 1] - vr.cu_kept[b]);
  } else if (vr.K != nullptr) {
    out0 = (size_t)b * vr.pad;
    if (tid == 0) vr.kept_count[b] = M;
  }
  const float* x = score_raw + (size_t)b * N;
  float* y = score + (size_t)b * N;
  uint8_t* kp = keep + (size_t)b * N;
  int32_t* ki = kept_idx + out0;
  float* sk = score_kept + out0;

  for (int i = tid; i < 2048; i += kThreads) s_hist[i] = 0;

  // sequence RMSNorm, exactly as tg_seq_rmsnorm's single-workgroup path
  const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
  f32x4 v[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) v[e] = sel::load_scores(x, (e * kThreads + tid) * 4, N, r, p1, vec);
  const double scale = sel::row_inv_rms(v, P, eps, s_part, &s_scale);  // (its barriers order the clear above)
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const int j = (e * kThreads + tid) * 4;
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)  // exactly 0 outside the span, also when the scale is not finite
      o[i] = (j + i >= r && j + i < p1) ? (float)((double)v[e][i] * scale) : 0.0f;
    if (vec && j + 4 <= N) {
      *reinterpret_cast<f32x4*>(y + j) = o;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i < N) y[j + i] = o[i];
    }
    // keys of the prunable scores (index j - r of the span) and the first digit
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (j + i >= r && j + i < p1) {
        const uint32_t key = sel::order_key(o[i]);
        s_keys[sel::key_slot(j + i - r)] = key;
        atomicAdd(&s_hist[key >> 21], 1u);
      }
    }
  }

  // padding of a short row in a batch wider than one workgroup's chunk
  for (int j = kThreads * kVec * 4 + tid; j < N; j += kThreads) y[j] = 0.0f;
  __syncthreads();  // every key and the first histogram are in LDS; y is written
  // the non-prunable tokens before the span are kept first, those after it
  // last (ranks r + K' ...), in order (their scores are 0)
  for (int j = tid; j < r; j += kThreads) {
    kp[j] = 1;
    if (j < lim) {
      ki[j] = j;
      sk[j] = 0.0f;
    }
  }
  for (int j = p1 + tid; j < Nb; j += kThreads) {
    kp[j] = 1;
    const int rank = r + Kp + (j - p1);
    if (rank < lim) {
      ki[rank] = j;
      sk[rank] = 0.0f;
    }
  }
  for (int j = Nb + tid; j < N; j += kThreads) kp[j] = 0;  // padding of a shorter row
  if (Kp <= 0 || Kp == P) {
    // trivial budgets: every prunable token or none
    const bool all = Kp > 0;
    for (int j = tid; j < P; j += kThreads) {
      kp[r + j] = all ? 1 : 0;
      if (all && r + j < lim) {
        ki[r + j] = r + j;
        sk[r + j] = y[r + j];
      }
    }
    return;
  }
  const sel::Threshold th = sel::radix_select_lds(s_keys, P, (uint32_t)Kp, s_hist, s_wave, s_sel);
  const uint32_t T = th.T, k_eq = th.k_eq;
  const bool all_ties = k_eq == th.n_eq;

  // Final pass in index order over kItems consecutive tokens per thread: keep
  // key > T, and key == T for the first k_eq such tokens; the kept tokens'
  // ranks come from a block-wide prefix count.
  static_assert(kItems == 16, "one 16-byte keep store per thread");
  const bool vec_store = ((reinterpret_cast<uintptr_t>(kp + r)) & 15u) == 0;
  uint32_t eq_base = 0;   // keys == T before the current chunk
  uint32_t out_base = r;  // kept tokens before the current chunk
  for (int c0 = 0; c0 < P; c0 += kThreads * kItems) {
    const int j0 = c0 + tid * kItems;
    uint32_t keys[kItems];
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const int j = j0 + e;
      keys[e] = j < P ? s_keys[sel::key_slot(j)] : 0u;
      n_eq += (j < P && keys[e] == T) ? 1u : 0u;
    }
    uint32_t eq_tot = 0, rank = 0;
    if (!all_ties) rank = eq_base + block_excl_scan_u32<kThreads / 64>(n_eq, s_wave, eq_tot);  // (block-uniform branch)
    uint32_t flags = 0;  // bit e: token j0 + e is kept
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const int j = j0 + e;
      bool kept = false;
      if (j < P) {
        if (keys[e] > T) {
          kept = true;
        } else if (keys[e] == T) {
          kept = all_ties || rank < k_eq;
          ++rank;
        }
      }
      flags |= kept ? (1u << e) : 0u;
    }
    uint32_t tot;
    uint32_t dst = out_base + block_excl_scan_u32<kThreads / 64>(__builtin_popcount(flags), s_wave, tot);
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < kItems; ++e) packed[e >> 2] |= ((flags >> e) & 1u) << (8 * (e & 3));
    // one pair of stores per kept token of this thread, ranks dst, dst + 1, ...
    // (a loop over the set bits: the wave issues as many store rounds as its
    // busiest lane has kept tokens, not one per item)
    for (uint32_t f = flags; f != 0u; f &= f - 1u) {
      const int e = __builtin_ctz(f);
      if ((int)dst < lim) {  // exactly M tokens are kept; never write past the row
        const uint32_t key = s_keys[sel::key_slot(j0 + e)];
        ki[dst] = r + j0 + e;
        // the key holds the score exactly, except that -0.0 and +0.0 share a
        // key and every NaN maps to key 0: only those re-read the score
        const float from_key = sel::key_score(key);
        sk[dst] = (key == 0u || from_key == 0.0f) ? y[r + j0 + e] : from_key;
      }
      ++dst;
    }
    if (vec_store && j0 + kItems <= P) {
      store16(kp + r + j0, u32x4{packed[0], packed[1], packed[2], packed[3]});
    } else {
#pragma unroll
      for (int e = 0; e < kItems; ++e)
        if (j0 + e < P) kp[r + j0 + e] = (uint8_t)(packed[e >> 2] >> (8 * (e & 3)));
    }
    eq_base += eq_tot;
    out_base += tot;
  }
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
