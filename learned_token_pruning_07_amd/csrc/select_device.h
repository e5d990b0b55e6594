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

// Four scores from x[j..j+3] (0 past N and below r).
__device__ __forceinline__ f32x4 load_scores(const float* x, int j, int N, int r, int p1, bool vec) {
  f32x4 v;
  if (vec && j + 4 <= N) {
    v = *reinterpret_cast<const f32x4*>(x + j);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = j + i < N ? x[j + i] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (j + i >= r && j + i < p1) ? v[i] : 0.0f;
  return v;
}

// Block-wide 1 / sqrt(mean of squares + eps) of a row whose scores this
// thread holds in v (zeros outside the prunable span), P prunable scores.
// Each thread's sum of squares (32 terms) is fp32; thread and wave partials
// are combined in fp64 in a fixed order.  0 when P == 0.  Contains barriers.
__device__ __forceinline__ double row_inv_rms(const f32x4 (&v)[kRowVec], int P, float eps, double* s_part,
                                              double* s_scale) {
  const int tid = threadIdx.x;
  float part = 0.0f;
#pragma unroll
  for (int e = 0; e < kRowVec; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(v[e][i], v[e][i], part);
  double acc = wave_sum_f64((double)part);
  if ((tid & 63) == 0) s_part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kRowThreads / 64; ++w) t += s_part[w];
    *s_scale = P > 0 ? 1.0 / sqrt(t / (double)P + (double)eps) : 0.0;
  }
  __syncthreads();
  return *s_scale;
}

// Order-preserving key: larger score -> larger key; -0.0 folds onto +0.0;
// every NaN maps to key 0, below -inf (whose key is 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                      // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
// s_wave holds 16 words, s_sel 3.  Contains barriers.
__device__ __forceinline__ Threshold radix_select_lds(const uint32_t* s_keys, int P, uint32_t Kp, uint32_t* s_hist,
                                                      uint32_t* s_wave, uint32_t* s_sel) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0, krem = Kp;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    if (pass > 0) {
      for (int i = tid; i < nb; i += kRowThreads) s_hist[i] = 0;
      __syncthreads();
      // batches of kBatch keys per thread: every LDS read of a batch is issued
      // before any is tested
      constexpr int kBatch = 8;
      for (int j0 = tid; j0 < P; j0 += kBatch * kRowThreads) {
        uint32_t key[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j = j0 + u * kRowThreads;
          key[u] = j < P ? s_keys[key_slot(j)] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (j0 + u * kRowThreads < P && (key[u] & pmask) == prefix)
            atomicAdd(&s_hist[(key[u] >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    // Bins in descending digit order; thread t owns descending bins
    // [t*per, t*per + per).  Find the bin where the running count from the
    // top first reaches krem.
    const int per = nb / kRowThreads;  // 2 or 1
    uint32_t local = 0;
    for (int e = 0; e < per; ++e) local += s_hist[nb - 1 - (tid * per + e)];
    uint32_t tot;
    uint32_t cum = block_excl_scan_u32<kRowThreads / 64>(local, s_wave, tot);
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
