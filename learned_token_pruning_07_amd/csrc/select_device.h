// Device code shared by the sequence RMSNorm, the top-K selector and the
// fused gate selection (TokenGate paper, Section 4: second half of Eq. 3 and
// Eq. 4), so that every path runs the same arithmetic and the fused call
// reproduces the separate calls bit for bit.
#pragma once

#include "tg_device.h"

namespace tg {
namespace sel {

// One workgroup normalises a row of up to kRowChunk scores: each of the
// kRowThreads threads holds kRowVec groups of four consecutive scores, group
// e of thread t starting at score (e * kRowThreads + t) * 4.
constexpr int kRowThreads = 1024;
constexpr int kRowVec = 8;
constexpr int kRowChunk = kRowThreads * kRowVec * 4;  // 32768 scores

// Up to kLdsKeys prunable keys live in LDS, one padding word after every 16
// keys: the coalesced passes and the 16-consecutive-key final pass both read
// without bank conflicts.
constexpr int kLdsKeys = 32768;
constexpr int kLdsKeyWords = kLdsKeys + kLdsKeys / 16;
__device__ __forceinline__ int key_slot(int j) { return j + (j >> 4); }

// NV groups of four scores, group e from x[jf(e) .. jf(e) + 3] (j a multiple
// of 4; 0 outside [r, p1) and past N).  Every load is issued before any is
// used: a row that is 16-byte aligned (`aligned`, from the caller) with
// N % 4 == 0 takes one 16-byte load per group (a group past the row reads
// the row's first group, then masked), any other row takes four clamped
// 4-byte loads per group.  Loading one group at a time, with a branch per
// group between the two forms and the mask right after, made the compiler
// wait for each group's load before issuing the next.
template <int NV, typename JF>
__device__ __forceinline__ void load_score_groups(f32x4* v, const float* x, JF jf, int N, int r, int p1,
                                                  bool aligned) {
  if (aligned && (N & 3) == 0) {  // (wave-uniform)
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int j = jf(e);
      v[e] = *reinterpret_cast<const f32x4*>(x + (j + 4 <= N ? j : 0));
    }
  } else {
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int j = jf(e);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[e][i] = x[min(j + i, N - 1)];
    }
  }
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int j = jf(e);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[e][i] = (j + i >= r && j + i < p1 && j + i < N) ? v[e][i] : 0.0f;
  }
}

// A workgroup of THREADS threads (a divisor of kRowThreads) stands in for
// the kRowThreads threads of the row layout: thread t plays the parts of
// threads t + s THREADS, s < kRowThreads / THREADS, and holds their groups
// in v[s kRowVec + e].  Every result below is the same bit for bit whatever
// THREADS is.
template <int THREADS>
constexpr int kRowParts = kRowThreads / THREADS;

// Fixed-order fp32 sum of squares of one row-layout thread's kRowVec groups.
__device__ __forceinline__ float part_sum_squares(const f32x4* v) {
  float part = 0.0f;
#pragma unroll
  for (int e = 0; e < kRowVec; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(v[e][i], v[e][i], part);
  return part;
}

// The row reduction in two halves: rms_part adds part s's fp32 sum of
// squares (row-layout threads tid + s THREADS) to the fp64 wave partials in
// s_part (kRowThreads / 64 doubles); rms_finish combines them in a fixed
// order into 1 / sqrt(mean of squares + eps) over P prunable scores (0 when
// P == 0).  rms_finish contains barriers.
template <int THREADS>
__device__ __forceinline__ void rms_part(float part, int s, double* s_part) {
  static_assert(kRowThreads % THREADS == 0 && THREADS % 64 == 0, "row parts");
  // the lanes of this wave are row-layout threads of one row-layout wave
  const double acc = wave_sum_f64((double)part);
  if ((threadIdx.x & 63) == 0) s_part[(threadIdx.x >> 6) + s * (THREADS / 64)] = acc;
}
__device__ __forceinline__ double rms_finish(int P, float eps, double* s_part, double* s_scale) {
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kRowThreads / 64; ++w) t += s_part[w];
    *s_scale = P > 0 ? 1.0 / sqrt(t / (double)P + (double)eps) : 0.0;
  }
  __syncthreads();
  return *s_scale;
}

// Block-wide 1 / sqrt(mean of squares + eps) of a row from the fp32 sums of
// squares of this thread's parts: wave and block partials are combined in
// fp64 in a fixed order.  Contains barriers.
template <int THREADS = kRowThreads>
__device__ __forceinline__ double row_inv_rms_parts(const float (&part)[kRowParts<THREADS>], int P, float eps,
                                                    double* s_part, double* s_scale) {
#pragma unroll
  for (int s = 0; s < kRowParts<THREADS>; ++s) rms_part<THREADS>(part[s], s, s_part);
  return rms_finish(P, eps, s_part, s_scale);
}

// The same, from the row-layout groups this thread holds in v (zeros outside
// the prunable span): v[s kRowVec + e] is group e of part s.
template <int THREADS = kRowThreads>
__device__ __forceinline__ double row_inv_rms(const f32x4 (&v)[kRowVec * kRowParts<THREADS>], int P, float eps,
                                              double* s_part, double* s_scale) {
  float part[kRowParts<THREADS>];
#pragma unroll
  for (int s = 0; s < kRowParts<THREADS>; ++s) part[s] = part_sum_squares(v + s * kRowVec);
  return row_inv_rms_parts<THREADS>(part, P, eps, s_part, s_scale);
}

// Order-preserving key: larger score -> larger key; -0.0 folds onto +0.0;
// every NaN maps to key 0, below -inf (whose key is 0x007FFFFF).
// (Branch-free: a positive score sets the top bit, a negative one flips
// every bit; -0.0 would land at 0x7FFFFFFF, just below +0.0's 0x80000000.)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  k = k == 0x7FFFFFFFu ? 0x80000000u : k;  // -0.0 -> +0.0
  return f != f ? 0u : k;                  // NaN
}

// The score of a key (the inverse of order_key for every non-NaN score other
// than -0.0, which comes back as +0.0).
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Result of the radix select over one row's prunable keys.
struct Threshold {
  uint32_t T;     // exact key of the K'-th largest
  uint32_t k_eq;  // how many keys equal to T are kept
  uint32_t n_eq;  // how many keys equal T
};

// Block-wide radix select over P keys in LDS (key_slot order) for the K'-th
// largest, 0 < K' < P, three digits [31:21], [20:10], [9:0].  On entry
// s_hist holds the histogram of digit [31:21] of all P keys (2048 bins).
// s_wave holds 16 words, s_sel 3.  Contains barriers.  Integer counting
// only: the threshold does not depend on THREADS.
// Thread t owns keys t + q THREADS.  The second pass reads all of them and
// marks in a bit mask (bit q) those whose first digit is the selected one;
// the third pass re-reads only the marked keys, the only ones that can
// carry the selected 22-bit prefix (a few percent of the keys for spread-out
// scores), instead of all P again.
template <int THREADS = kRowThreads>
__device__ __forceinline__ Threshold radix_select_lds(const uint32_t* s_keys, int P, uint32_t Kp, uint32_t* s_hist,
                                                      uint32_t* s_wave, uint32_t* s_sel) {
  const int tid = threadIdx.x;
  constexpr int kBatch = 8;
  constexpr int kBatches = (kLdsKeys + kBatch * THREADS - 1) / (kBatch * THREADS);
  constexpr int kMaskWords = (kBatches * kBatch + 31) / 32;
  uint32_t marked[kMaskWords];
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) marked[w] = 0u;
  uint32_t prefix = 0, pmask = 0, krem = Kp;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    if (pass > 0) {
      for (int i = tid; i < nb; i += THREADS) s_hist[i] = 0;
      __syncthreads();
    }
    if (pass == 1) {
      // batches of kBatch keys per thread: every LDS read of a batch is issued
      // before any is tested
#pragma unroll
      for (int bt = 0; bt < kBatches; ++bt) {
        const int j0 = tid + bt * kBatch * THREADS;
        if (bt * kBatch * THREADS >= P) break;  // (block-uniform)
        uint32_t key[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j = j0 + u * THREADS;
          key[u] = j < P ? s_keys[key_slot(j)] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const bool hit = j0 + u * THREADS < P && (key[u] & pmask) == prefix;
          if (hit) atomicAdd(&s_hist[(key[u] >> shift) & (uint32_t)(nb - 1)], 1u);
          const int q = bt * kBatch + u;
          marked[q >> 5] |= (hit ? 1u : 0u) << (q & 31);
        }
      }
    } else if (pass == 2) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w)
        for (uint32_t f = marked[w]; f != 0u; f &= f - 1u) {
          const uint32_t key = s_keys[key_slot(tid + (w * 32 + __builtin_ctz(f)) * THREADS)];
          if ((key & pmask) == prefix) atomicAdd(&s_hist[key & (uint32_t)(nb - 1)], 1u);
        }
    }
    __syncthreads();
    // Bins in descending digit order; thread t owns descending bins
    // [t*per, t*per + per).  Find the bin where the running count from the
    // top first reaches krem.
    const int per = nb / THREADS;  // bins per thread
    uint32_t local = 0;
    for (int e = 0; e < per; ++e) local += s_hist[nb - 1 - (tid * per + e)];
    uint32_t tot;
    uint32_t cum = block_excl_scan_u32<THREADS / 64>(local, s_wave, tot);
    for (int e = 0; e < per; ++e) {
      const int digit = nb - 1 - (tid * per + e);
      const uint32_t c = s_hist[digit];
      if (cum < krem && cum + c >= krem) {
        s_sel[0] = (uint32_t)digit;
        s_sel[1] = krem - cum;
        s_sel[2] = c;  // keys sharing the selected prefix (after the last pass: keys equal to T)
      }
      cum += c;
    }
    __syncthreads();
    prefix |= s_sel[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem = s_sel[1];
    __syncthreads();
  }
  return Threshold{prefix, krem, s_sel[2]};
}

}  // namespace sel
}  // namespace tg
