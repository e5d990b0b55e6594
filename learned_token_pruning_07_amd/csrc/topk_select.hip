// Top-K selector (TokenGate paper, Section 4, "Top-K Selector", Eq. 4): keep
// the K' = min(K, N - r) highest-scoring prunable tokens plus every
// non-prunable token.
//
// Radix select on an order-preserving 32-bit key, one workgroup per batch row:
//  1. key(score): larger score -> larger key; -0.0 folds onto +0.0; every NaN
//     maps to key 0, below -inf (whose key is 0x007FFFFF).
//  2. Three LDS-histogram passes over digits [31:21], [20:10], [9:0] find the
//     exact key T of the K'-th largest prunable score and how many of the
//     keys equal to T must be kept (k_eq).
//  3. A final pass in index order keeps key > T, and key == T for the first
//     k_eq such tokens by index (block-wide prefix count), which is the
//     lower-index tie-break.
// Spans of up to 32768 prunable tokens run in one workgroup with the keys in
// LDS (136 KiB with one padding word after every 16 keys, so that both the
// coalesced passes and the final pass's 16 consecutive keys per thread read
// without bank conflicts).  Longer spans take five short launches over
// 4096-key chunks, the histograms in the workspace: clear, one histogram
// launch per digit (LDS counts added to the global histogram with atomics;
// every workgroup re-derives the previous digits from the previous
// histogram), and the final pass.
// Integer counting only: the mask is exact and deterministic.
#include "select_device.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

using sel::key_slot;
using sel::order_key;
constexpr int kThreads = sel::kRowThreads;
constexpr int kLdsKeys = sel::kLdsKeys;
constexpr int kItems = 16;  // consecutive keys per thread in the final pass

// Spans of up to kLdsKeys prunable tokens (and the trivial budgets of any span).
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float* __restrict__ score, int N, int r,
                                                               int p1, int K, uint8_t* __restrict__ keep) {
  __shared__ uint32_t s_keys[sel::kLdsKeyWords];
  __shared__ uint32_t s_hist[2048];
  __shared__ __attribute__((aligned(16))) uint32_t s_wave[16];
  __shared__ uint32_t s_sel[3];

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const float* sc = score + (size_t)b * N + r;
  uint8_t* kp = keep + (size_t)b * N;
  const int P = p1 - r;
  const int Kp = K < P ? K : P;

  for (int j = tid; j < r; j += kThreads) kp[j] = 1;
  for (int j = p1 + tid; j < N; j += kThreads) kp[j] = 1;  // non-prunable tokens after the span
  if (Kp <= 0 || Kp == P) {
    const uint8_t v = Kp > 0 ? 1 : 0;
    for (int j = tid; j < P; j += kThreads) kp[r + j] = v;
    return;
  }

  for (int i = tid; i < 2048; i += kThreads) s_hist[i] = 0;
  __syncthreads();
  {
    // all loads of a thread are issued before any is used (latency-bound);
    // the first digit's histogram is counted on the way in
    constexpr int kLoad = kLdsKeys / kThreads;
    float f[kLoad];
#pragma unroll
    for (int e = 0; e < kLoad; ++e) {
      const int j = e * kThreads + tid;
      f[e] = j < P ? sc[j] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < kLoad; ++e) {
      const int j = e * kThreads + tid;
      if (j < P) {
        const uint32_t key = order_key(f[e]);
        s_keys[key_slot(j)] = key;
        atomicAdd(&s_hist[key >> 21], 1u);
      }
    }
  }
  const sel::Threshold th = sel::radix_select_lds(s_keys, P, (uint32_t)Kp, s_hist, s_wave, s_sel);
  const uint32_t T = th.T, k_eq = th.k_eq;

  static_assert(kItems == 16, "one 16-byte store per thread");
  const bool vec_store = ((reinterpret_cast<uintptr_t>(kp + r)) & 15u) == 0;
  if (k_eq == th.n_eq) {
    // Every key equal to T is kept (always so for distinct scores): keep is
    // key >= T, with no index-order ranking.
    for (int j0 = tid * kItems; j0 < P; j0 += kThreads * kItems) {
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < kItems; ++e) {
        const int j = j0 + e;
        packed[e >> 2] |= (j < P && s_keys[key_slot(j)] >= T ? 1u : 0u) << (8 * (e & 3));
      }
      if (vec_store && j0 + kItems <= P) {
        store16(kp + r + j0, u32x4{packed[0], packed[1], packed[2], packed[3]});
      } else {
#pragma unroll
        for (int e = 0; e < kItems; ++e)
          if (j0 + e < P) kp[r + j0 + e] = (uint8_t)(packed[e >> 2] >> (8 * (e & 3)));
      }
    }
    return;
  }

  // Final pass in index order.  Each thread decides kItems consecutive
  // tokens and writes them as one 16-byte store when the row allows it.
  uint32_t base = 0;  // number of keys == T before the current chunk
  for (int c0 = 0; c0 < P; c0 += kThreads * kItems) {
    uint32_t keys[kItems];
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const int j = c0 + tid * kItems + e;
      keys[e] = j < P ? s_keys[key_slot(j)] : 0u;
      n_eq += (j < P && keys[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t rank = base + block_excl_scan_u32<kThreads / 64>(n_eq, s_wave, tot);
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const int j = c0 + tid * kItems + e;
      uint32_t v = 0;
      if (j < P) {
        if (keys[e] > T) {
          v = 1;
        } else if (keys[e] == T) {
          v = rank < k_eq ? 1u : 0u;
          ++rank;
        }
      }
      packed[e >> 2] |= v << (8 * (e & 3));
    }
    const int j0 = c0 + tid * kItems;
    if (vec_store && j0 + kItems <= P) {
      store16(kp + r + j0, u32x4{packed[0], packed[1], packed[2], packed[3]});
    } else {
#pragma unroll
      for (int e = 0; e < kItems; ++e)
        if (j0 + e < P) kp[r + j0 + e] = (uint8_t)(packed[e >> 2] >> (8 * (e & 3)));
    }
    base += tot;
  }
}

// ---- prunable spans longer than the LDS key cache ----
constexpr int kMThreads = 256;
constexpr int kMItems = 16;                   // consecutive keys per thread
constexpr int kMChunk = kMThreads * kMItems;  // keys per workgroup
// workspace per batch row (32-bit words): digit histograms of 2048, 2048 and
// 1024 bins, then the state handed from one launch to the next
constexpr int kH0 = 0, kH1 = 2048, kH2 = 4096, kState = 5120, kWsWords = 5124;

// keys of this thread's kMItems consecutive prunable tokens from c0 + tid * kMItems
__device__ __forceinline__ void chunk_keys(const float* sc, int P, int j0, uint32_t (&key)[kMItems]) {
  if (((reinterpret_cast<uintptr_t>(sc + j0)) & 15u) == 0 && j0 + kMItems <= P) {
#pragma unroll
    for (int q = 0; q < kMItems / 4; ++q) {
      const u32x4 w = load16(sc + j0 + q * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[q * 4 + e] = order_key(__uint_as_float(w[e]));
    }
  } else {
    float x[kMItems];  // clamped, unconditional loads, all issued before any is used
#pragma unroll
    for (int e = 0; e < kMItems; ++e) x[e] = sc[min(j0 + e, P - 1)];
#pragma unroll
    for (int e = 0; e < kMItems; ++e) key[e] = j0 + e < P ? order_key(x[e]) : 0u;
  }
}

// Block-wide: the digit of `hist` (nb bins, LDS) at which the count from the
// largest digit down first reaches krem.  Returns it in sel[0], the count
// still to take inside it in sel[1], and its bin count in sel[2].
__device__ void select_digit(const uint32_t* hist, int nb, uint32_t krem, uint32_t* s_wave, uint32_t* sel) {
  const int tid = threadIdx.x;
  const int per = nb / kMThreads;
  uint32_t local = 0;
  for (int e = 0; e < per; ++e) local += hist[nb - 1 - (tid * per + e)];
  uint32_t tot;
  uint32_t cum = block_excl_scan_u32<kMThreads / 64>(local, s_wave, tot);
  for (int e = 0; e < per; ++e) {
    const int digit = nb - 1 - (tid * per + e);
    const uint32_t c = hist[digit];
    if (cum < krem && cum + c >= krem) {
      sel[0] = (uint32_t)digit;
      sel[1] = krem - cum;
      sel[2] = c;
    }
    cum += c;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kMThreads) void topk_ws_clear_kernel(uint32_t* __restrict__ ws) {
  uint32_t* w = ws + (size_t)blockIdx.x * kWsWords;
  for (int i = threadIdx.x; i < kWsWords; i += kMThreads) w[i] = 0;
}

// Row b's span and budget: the uniform ones, or with vr.len set its own
// (a row of up to kVarlenOneGroupRow tokens is not this path's: skip = true).
__device__ __forceinline__ bool long_row(const VarlenRows& vr, int b, int N, int& r, int& p1, int& Kp, int& len) {
  len = N;
  if (vr.len == nullptr) return true;
  const RowSpec rs = varlen_row(vr, b, N);
  r = rs.r;
  p1 = rs.p1;
  Kp = min(rs.K, p1 - r);
  len = rs.len;
  return rs.len > kVarlenOneGroupRow;
}

// Histogram of digit PASS over the keys that match the digits already chosen
// (which every workgroup re-derives from the previous histogram; workgroup 0
// also records them for the next launch).
template <int PASS>
__global__ __launch_bounds__(kMThreads) void topk_hist_kernel(const float* __restrict__ score, int N, int r, int p1,
                                                              int Kp, VarlenRows vr,
                                                              uint32_t* __restrict__ ws) {
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_prev[2048];
  __shared__ __attribute__((aligned(16))) uint32_t s_wave[kMThreads / 64];
  __shared__ uint32_t s_sel[3];
  const int tid = threadIdx.x, b = blockIdx.y, c0 = blockIdx.x * kMChunk;
  int len;
  if (!long_row(vr, b, N, r, p1, Kp, len)) return;
  const int P = p1 - r;
  // chunks past the span, and the trivial budgets (settled by the final pass)
  if (c0 >= P || Kp <= 0 || Kp == P) return;
  const float* sc = score + (size_t)b * N + r;
  uint32_t* w = ws + (size_t)b * kWsWords;
  uint32_t key[kMItems];
  chunk_keys(sc, P, c0 + tid * kMItems, key);  // requested first

  constexpr int shift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr int nb = PASS == 2 ? 1024 : 2048;
  uint32_t prefix = 0, pmask = 0;
  if (PASS > 0) {
    const int pnb = 2048;  // bins of the previous digit
    const uint32_t* prev = w + (PASS == 1 ? kH0 : kH1);
    for (int i = tid; i < pnb; i += kMThreads) s_prev[i] = prev[i];
    const uint32_t krem_prev = PASS == 1 ? (uint32_t)Kp : w[kState + 1];
    const uint32_t prefix_prev = PASS == 1 ? 0u : w[kState + 0];
    __syncthreads();
    select_digit(s_prev, pnb, krem_prev, s_wave, s_sel);
    const int pshift = PASS == 1 ? 21 : 10;
    prefix = prefix_prev | (s_sel[0] << pshift);
    pmask = PASS == 1 ? 0xFFE00000u : 0xFFFFFC00u;
    if (blockIdx.x == 0 && tid == 0) {
      w[kState + 2 * (PASS - 1)] = prefix;         // digits chosen so far
      w[kState + 2 * (PASS - 1) + 1] = s_sel[1];   // how many keys to take among those matching them
    }
  }
  for (int i = tid; i < nb; i += kMThreads) s_hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    const int j = c0 + tid * kMItems + e;
    if (j < P && (key[e] & pmask) == prefix) atomicAdd(&s_hist[(key[e] >> shift) & (uint32_t)(nb - 1)], 1u);
  }
  __syncthreads();
  uint32_t* h = w + (PASS == 0 ? kH0 : (PASS == 1 ? kH1 : kH2));
  for (int i = tid; i < nb; i += kMThreads)
    if (s_hist[i] != 0) atomicAdd(&h[i], s_hist[i]);
}

// keep: key > T, or key == T among the first k_eq such tokens by index
// (tokens outside the span: 1 up to the row's length, 0 past it)
__global__ __launch_bounds__(kMThreads) void topk_final_kernel(const float* __restrict__ score, int N, int r, int p1,
                                                               int Kp, VarlenRows vr,
                                                               const uint32_t* __restrict__ ws,
                                                               uint8_t* __restrict__ keep) {
  __shared__ uint32_t s_prev[1024];
  __shared__ __attribute__((aligned(16))) uint32_t s_wave[kMThreads / 64];
  __shared__ uint32_t s_sel[3];
  const int tid = threadIdx.x, b = blockIdx.y, c0 = blockIdx.x * kMChunk;
  int len;
  if (!long_row(vr, b, N, r, p1, Kp, len)) return;
  const float* sc = score + (size_t)b * N + r;
  const uint32_t* w = ws + (size_t)b * kWsWords;
  uint8_t* kp = keep + (size_t)b * N;
  const int P = p1 - r;
  const int j0 = c0 + tid * kMItems;
  if (blockIdx.x == 0) {
    for (int j = tid; j < r; j += kMThreads) kp[j] = 1;
    for (int j = p1 + tid; j < len; j += kMThreads) kp[j] = 1;
    for (int j = len + tid; j < N; j += kMThreads) kp[j] = 0;
  }
  if (c0 >= P) return;
  if (Kp <= 0 || Kp == P) {
    // trivial budgets: every prunable token of the chunk or none
    const uint8_t v = Kp > 0 ? 1 : 0;
    for (int e = 0; e < kMItems; ++e)
      if (j0 + e < P) kp[r + j0 + e] = v;
    return;
  }
  uint32_t key[kMItems];
  chunk_keys(sc, P, j0, key);

  for (int i = tid; i < 1024; i += kMThreads) s_prev[i] = w[kH2 + i];
  const uint32_t prefix = w[kState + 2], krem = w[kState + 3];
  __syncthreads();
  select_digit(s_prev, 1024, krem, s_wave, s_sel);
  const uint32_t T = prefix | s_sel[0];
  const uint32_t k_eq = s_sel[1], n_eq = s_sel[2];

  uint32_t rank = 0;  // keys == T before this thread's first token
  if (k_eq != n_eq) {
    // ties straddle the budget: rank the keys equal to T by index -- those in
    // earlier chunks are counted here from the scores (rare path)
    uint32_t before = 0;
    for (int j = tid; j < c0; j += kMThreads) before += order_key(sc[j]) == T ? 1u : 0u;
    uint32_t tot;
    before = block_excl_scan_u32<kMThreads / 64>(before, s_wave, tot);
    const uint32_t base = tot;
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < kMItems; ++e) mine += (j0 + e < P && key[e] == T) ? 1u : 0u;
    rank = base + block_excl_scan_u32<kMThreads / 64>(mine, s_wave, tot);
  }
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    uint32_t v = 0;
    if (j0 + e < P) {
      if (key[e] > T) {
        v = 1;
      } else if (key[e] == T) {
        v = (k_eq == n_eq || rank < k_eq) ? 1u : 0u;
        ++rank;
      }
    }
    packed[e >> 2] |= v << (8 * (e & 3));
  }
  if ((((reinterpret_cast<uintptr_t>(kp + r + j0)) & 15u) == 0) && j0 + kMItems <= P) {
    store16(kp + r + j0, u32x4{packed[0], packed[1], packed[2], packed[3]});
  } else {
#pragma unroll
    for (int e = 0; e < kMItems; ++e)
      if (j0 + e < P) kp[r + j0 + e] = (uint8_t)(packed[e >> 2] >> (8 * (e & 3)));
  }
}

}  // namespace

size_t topk_select_workspace(int B, int N) {
  return N > kLdsKeys ? (size_t)B * kWsWords * sizeof(uint32_t) : 0;
}

hipError_t launch_topk_select(const float* score, int B, int N, int r, int p1, int K, uint8_t* keep, void* ws,
                              hipStream_t s) {
  const int P = p1 - r;
  const int Kp = K < P ? K : P;
  if (P <= kLdsKeys || Kp <= 0 || Kp == P) {  // (the single workgroup also settles the trivial budgets)
    hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(kThreads), 0, s, score, N, r, p1, K, keep);
    return hipGetLastError();
  }
  uint32_t* w = static_cast<uint32_t*>(ws);
  const dim3 grid((P + kMChunk - 1) / kMChunk, B);
  hipLaunchKernelGGL(topk_ws_clear_kernel, dim3(B), dim3(kMThreads), 0, s, w);
  const VarlenRows none{};
  hipLaunchKernelGGL(topk_hist_kernel<0>, grid, dim3(kMThreads), 0, s, score, N, r, p1, Kp, none, w);
  hipLaunchKernelGGL(topk_hist_kernel<1>, grid, dim3(kMThreads), 0, s, score, N, r, p1, Kp, none, w);
  hipLaunchKernelGGL(topk_hist_kernel<2>, grid, dim3(kMThreads), 0, s, score, N, r, p1, Kp, none, w);
  hipLaunchKernelGGL(topk_final_kernel, grid, dim3(kMThreads), 0, s, score, N, r, p1, Kp, none, w, keep);
  return hipGetLastError();
}

hipError_t launch_topk_select_long_rows(const float* score, int B, int N, VarlenRows vr, uint8_t* keep, void* ws,
                                        hipStream_t s) {
  if (N <= kVarlenOneGroupRow) return hipSuccess;
  uint32_t* w = static_cast<uint32_t*>(ws);
  const dim3 grid((N + kMChunk - 1) / kMChunk, B);  // every span fits N
  hipLaunchKernelGGL(topk_ws_clear_kernel, dim3(B), dim3(kMThreads), 0, s, w);
  hipLaunchKernelGGL(topk_hist_kernel<0>, grid, dim3(kMThreads), 0, s, score, N, 0, 0, 0, vr, w);
  hipLaunchKernelGGL(topk_hist_kernel<1>, grid, dim3(kMThreads), 0, s, score, N, 0, 0, 0, vr, w);
  hipLaunchKernelGGL(topk_hist_kernel<2>, grid, dim3(kMThreads), 0, s, score, N, 0, 0, 0, vr, w);
  hipLaunchKernelGGL(topk_final_kernel, grid, dim3(kMThreads), 0, s, score, N, 0, 0, 0, vr, w, keep);
  return hipGetLastError();
}

}  // namespace tg
