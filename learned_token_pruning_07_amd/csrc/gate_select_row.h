// One row of the gate selection (TokenGate paper, Section 4: sequence
// RMSNorm of the scores, second half of Eq. 3; the Top-K Selector, Eq. 4; the
// kept set in order, Appendix C.4) by one workgroup, shared by the fused
// selection kernel (gate_select.hip) and the fused gate (gate_score.hip) so
// that both give the same bits.
#pragma once

#include "select_device.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace selrow {

constexpr int kThreads = sel::kRowThreads;
constexpr int kVec = sel::kRowVec;
constexpr int kItems = 16;  // consecutive prunable tokens per thread in the final pass

// LDS of one row's selection (the fused gate carves it from its own buffer)
struct SelLds {
  uint32_t* keys;   // sel::kLdsKeyWords
  uint32_t* hist;   // 2048
  uint32_t* wave;   // 16, 16-byte aligned
  uint32_t* sel;    // 3
  double* part;     // kRowThreads / 64
  double* scale;    // 1
};
constexpr size_t kSelLdsBytes = (size_t)sel::kLdsKeyWords * 4 + 2048 * 4 + 16 * 4 + 16 + (kThreads / 64) * 8 + 16;
__device__ __forceinline__ SelLds carve_sel_lds(unsigned char* base) {
  SelLds l;
  l.keys = reinterpret_cast<uint32_t*>(base);
  l.hist = l.keys + sel::kLdsKeyWords;
  l.wave = l.hist + 2048;
  l.sel = l.wave + 16;
  l.part = reinterpret_cast<double*>(l.sel + 4);
  l.scale = l.part + kThreads / 64;
  return l;
}

// The selection of batch row b by one workgroup of THREADS threads (a
// divisor of 1024 standing in for the row layout's 1024, see
// sel::kRowParts): the results do not depend on THREADS.
// score_raw and score may alias: every raw score is read before the
// reduction's barriers, and nothing reads score_raw after them.
// With vr.len set, batch row b has its own valid length, span and budget
// (clamped into range: 0 <= span_begin <= span_end <= len <= N, K >= 0) and
// writes its kept tokens at kept_idx + cu_kept[b], at most cu_kept[b + 1] -
// cu_kept[b] of them; tokens at or past len are padding (score 0, not kept).
template <int THREADS>
__device__ __forceinline__ void gate_select_row(const float* score_raw, int N, int r_all, int p1_all, float eps,
                                                int K_all, const VarlenRows& vr, float* score,
                                                uint8_t* __restrict__ keep, int32_t* __restrict__ kept_idx,
                                                float* __restrict__ score_kept, int b, const SelLds& L) {
  constexpr int PARTS = sel::kRowParts<THREADS>;
  uint32_t* s_keys = L.keys;
  uint32_t* s_hist = L.hist;
  uint32_t* s_wave = L.wave;
  uint32_t* s_sel = L.sel;

  const int tid = threadIdx.x;
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

  for (int i = tid; i < 2048; i += THREADS) s_hist[i] = 0;

  // sequence RMSNorm, exactly as tg_seq_rmsnorm's single-workgroup path:
  // part s of this thread is row-layout thread tid + s THREADS.  Up to two
  // parts keep their scores in registers across the reduction; more parts
  // (small workgroups) run one part at a time and read their scores again
  // once the scale is known.
  const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
  constexpr bool kHold = PARTS <= 2;
  constexpr int kHeld = kHold ? PARTS : 1;
  f32x4 v[kVec * kHeld];
  auto load_part = [&](int s, f32x4* vs) __attribute__((always_inline)) {
    sel::load_score_groups<kVec>(vs, x, [&](int e) { return (e * kThreads + tid + s * THREADS) * 4; }, N, r, p1,
                                 vec);
  };
  // normalised scores of part s out to y; its prunable keys to LDS with the first digit's histogram
  auto emit_part = [&](int s, const f32x4* vs, double scale) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const int j = (e * kThreads + tid + s * THREADS) * 4;
      const f32x4 vv = vs[e];
      // Three wave-uniform cases for the wave's 64 groups of this e (scores
      // jw .. jw + 255): none in the prunable span (zeros out, no keys); all
      // in it with r % 4 == 0, so that a group's 4 key slots are consecutive
      // (straight-line form); otherwise the masked form below, whose
      // per-score branches cost exec mask saves and restores.
      const int jw = (e * kThreads + (tid & ~63) + s * THREADS) * 4;
      if (jw >= p1 || jw + 256 <= r) {
        if (jw < N) {
          if (vec && j + 4 <= N) {
            *reinterpret_cast<f32x4*>(y + j) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (j + i < N) y[j + i] = 0.0f;
          }
        }
        continue;
      }
      if ((r & 3) == 0 && jw >= r && jw + 256 <= p1) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (float)((double)vv[i] * scale);
        if (vec) {
          *reinterpret_cast<f32x4*>(y + j) = o;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) y[j + i] = o[i];
        }
        const int slot = sel::key_slot(j - r);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t key = sel::order_key(o[i]);
          s_keys[slot + i] = key;
          atomicAdd(&s_hist[key >> 21], 1u);
        }
        continue;
      }
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)  // exactly 0 outside the span, also when the scale is not finite
        o[i] = (j + i >= r && j + i < p1) ? (float)((double)vv[i] * scale) : 0.0f;
      if (vec && j + 4 <= N) {
        *reinterpret_cast<f32x4*>(y + j) = o;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (j + i < N) y[j + i] = o[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (j + i >= r && j + i < p1) {
          const uint32_t key = sel::order_key(o[i]);
          s_keys[sel::key_slot(j + i - r)] = key;
          atomicAdd(&s_hist[key >> 21], 1u);
        }
      }
    }
  };
  double scale;
  if constexpr (kHold) {
    sel::load_score_groups<PARTS * kVec>(
        v, x, [&](int q) { return ((q % kVec) * kThreads + tid + (q / kVec) * THREADS) * 4; }, N, r, p1, vec);
    scale = sel::row_inv_rms<THREADS>(v, P, eps, L.part, L.scale);  // (its barriers order the clear above)
#pragma unroll
    for (int s = 0; s < PARTS; ++s) emit_part(s, v + s * kVec, scale);
  } else {
#pragma unroll 1
    for (int s = 0; s < PARTS; ++s) {
      load_part(s, v);
      sel::rms_part<THREADS>(sel::part_sum_squares(v), s, L.part);
    }
    scale = sel::rms_finish(P, eps, L.part, L.scale);
#pragma unroll 1
    for (int s = 0; s < PARTS; ++s) {
      load_part(s, v);
      emit_part(s, v, scale);
    }
  }
  // padding of a short row in a batch wider than one workgroup's chunk
  for (int j = kThreads * kVec * 4 + tid; j < N; j += THREADS) y[j] = 0.0f;
  __syncthreads();  // every key and the first histogram are in LDS; y is written
  // the non-prunable tokens before the span are kept first, those after it
  // last (ranks r + K' ...), in order (their scores are 0)
  for (int j = tid; j < r; j += THREADS) {
    kp[j] = 1;
    if (j < lim) {
      ki[j] = j;
      sk[j] = 0.0f;
    }
  }
  for (int j = p1 + tid; j < Nb; j += THREADS) {
    kp[j] = 1;
    const int rank = r + Kp + (j - p1);
    if (rank < lim) {
      ki[rank] = j;
      sk[rank] = 0.0f;
    }
  }
  for (int j = Nb + tid; j < N; j += THREADS) kp[j] = 0;  // padding of a shorter row
  if (Kp <= 0 || Kp == P) {
    // trivial budgets: every prunable token or none
    const bool all = Kp > 0;
    for (int j = tid; j < P; j += THREADS) {
      kp[r + j] = all ? 1 : 0;
      if (all && r + j < lim) {
        ki[r + j] = r + j;
        sk[r + j] = y[r + j];
      }
    }
    return;
  }
  const sel::Threshold th = sel::radix_select_lds<THREADS>(s_keys, P, (uint32_t)Kp, s_hist, s_wave, s_sel);
  const uint32_t T = th.T, k_eq = th.k_eq;
  const bool all_ties = k_eq == th.n_eq;

  // Final pass in index order over kItems consecutive tokens per thread: keep
  // key > T, and key == T for the first k_eq such tokens; the kept tokens'
  // ranks come from a block-wide prefix count.
  static_assert(kItems == 16, "one 16-byte keep store per thread");
  const bool vec_store = ((reinterpret_cast<uintptr_t>(kp + r)) & 15u) == 0;
  uint32_t eq_base = 0;   // keys == T before the current chunk
  uint32_t out_base = r;  // kept tokens before the current chunk
  for (int c0 = 0; c0 < P; c0 += THREADS * kItems) {
    const int j0 = c0 + tid * kItems;
    // This thread's keys, read unconditionally (items past P read key P - 1
    // and are masked off), compared to T as bit masks: conditional reads made
    // the compiler wait for each read before the next, and per-item branches
    // cost exec-mask saves and restores.
    const int nv = min(max(P - j0, 0), kItems);
    const uint32_t vmask = (1u << nv) - 1u;
    uint32_t gtm = 0, eqm = 0;  // bit e: key of token j0 + e is > T, == T
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const uint32_t key = s_keys[sel::key_slot(min(j0 + e, P - 1))];
      gtm |= (key > T ? 1u : 0u) << e;
      eqm |= (key == T ? 1u : 0u) << e;
    }
    gtm &= vmask;
    eqm &= vmask;
    uint32_t eq_tot = 0;
    uint32_t flags = gtm | eqm;  // bit e: token j0 + e is kept
    if (!all_ties) {             // (block-uniform) only the first k_eq keys equal to T, in index order
      uint32_t rank = eq_base + block_excl_scan_u32<THREADS / 64>(__builtin_popcount(eqm), s_wave, eq_tot);
      uint32_t keep_eq = 0;
#pragma unroll
      for (int e = 0; e < kItems; ++e) {
        const uint32_t b = (eqm >> e) & 1u;
        keep_eq |= (b & (rank < k_eq ? 1u : 0u)) << e;
        rank += b;
      }
      flags = gtm | keep_eq;
    }
    uint32_t tot;
    uint32_t dst = out_base + block_excl_scan_u32<THREADS / 64>(__builtin_popcount(flags), s_wave, tot);
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < kItems; ++e) packed[e >> 2] |= ((flags >> e) & 1u) << (8 * (e & 3));
    // one pair of stores per kept token of this thread, ranks dst, dst + 1, ...
    // (a loop over the set bits: the wave issues as many store rounds as its
    // busiest lane has kept tokens, not one per item).  The key holds the
    // score exactly, except that -0.0 and +0.0 share a key and every NaN maps
    // to key 0: those kept tokens are marked and re-read afterwards, outside
    // this loop (a global load inside it made every round wait for the
    // round's stores).
    const uint32_t dst0 = dst;
    uint32_t reread = 0;  // bit e: kept token j0 + e needs its exact score
    for (uint32_t f = flags; f != 0u; f &= f - 1u) {
      const int e = __builtin_ctz(f);
      if ((int)dst < lim) {  // exactly M tokens are kept; never write past the row
        const uint32_t key = s_keys[sel::key_slot(j0 + e)];
        ki[dst] = r + j0 + e;
        const float from_key = sel::key_score(key);
        sk[dst] = from_key;
        reread |= (key == 0u || from_key == 0.0f) ? (1u << e) : 0u;
      }
      ++dst;
    }
    if (__ballot(reread != 0u) != 0) {  // (rare; wave-uniform)
      uint32_t d = dst0;
      for (uint32_t f = flags; f != 0u; f &= f - 1u) {
        const int e = __builtin_ctz(f);
        if ((reread >> e) & 1u) sk[d] = y[r + j0 + e];  // (d < lim: only such tokens were marked)
        ++d;
      }
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

}  // namespace selrow
}  // namespace tg
