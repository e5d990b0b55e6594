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
// The keys stay in LDS when the prunable span fits (<= 32768 keys, 136 KiB
// with one padding word after every 16 keys, so that both the coalesced
// passes and the final pass's 16 consecutive keys per thread read without
// bank conflicts); longer spans re-read the scores from global memory
// (L2-resident) per pass.
// Integer counting only: the mask is exact and deterministic.
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 1024;
constexpr int kLdsKeys = 32768;
__device__ __forceinline__ int key_slot(int j) { return j + (j >> 4); }  // padded LDS position of key j
constexpr int kItems = 16;  // consecutive keys per thread in the final pass
constexpr int kBatch = 16;  // loads in flight per thread when the keys are re-read from global memory

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                      // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float* __restrict__ score, int N, int r,
                                                               int K, uint8_t* __restrict__ keep) {
  __shared__ uint32_t s_keys[kLdsKeys + kLdsKeys / 16];
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_wave[16];
  __shared__ uint32_t s_sel[3];

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const float* sc = score + (size_t)b * N + r;
  uint8_t* kp = keep + (size_t)b * N;
  const int P = N - r;
  const int Kp = K < P ? K : P;

  for (int j = tid; j < r; j += kThreads) kp[j] = 1;
  if (Kp <= 0 || Kp == P) {
    const uint8_t v = Kp > 0 ? 1 : 0;
    for (int j = tid; j < P; j += kThreads) kp[r + j] = v;
    return;
  }

  const bool cached = P <= kLdsKeys;
  for (int i = tid; i < 2048; i += kThreads) s_hist[i] = 0;
  __syncthreads();
  if (cached) {
    // all loads of a thread are issued before any is used (latency-bound);
    // the first pass's histogram (digit [31:21]) is counted on the way in
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

  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)Kp;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    if (pass > 0 || !cached) {  // (the cached first pass was counted during the load)
      if (pass > 0)
        for (int i = tid; i < nb; i += kThreads) s_hist[i] = 0;
      __syncthreads();
    }
    if (cached && pass == 0) {
      // counted during the load
    } else if (cached) {
      for (int j = tid; j < P; j += kThreads) {
        const uint32_t key = s_keys[key_slot(j)];
        if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    } else {
      for (int c0 = 0; c0 < P; c0 += kThreads * kBatch) {
        float f[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
          const int j = c0 + e * kThreads + tid;
          f[e] = j < P ? sc[j] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
          const int j = c0 + e * kThreads + tid;
          const uint32_t key = order_key(f[e]);
          if (j < P && (key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        }
      }
    }
    __syncthreads();
    // Bins in descending digit order; thread t owns descending bins
    // [t*per, t*per + per).  Find the bin where the running count from the top
    // first reaches krem.
    const int per = nb / kThreads;  // 2 or 1
    uint32_t local = 0;
    for (int e = 0; e < per; ++e) local += s_hist[nb - 1 - (tid * per + e)];
    uint32_t tot;
    uint32_t cum = block_excl_scan_u32(local, s_wave, tot);
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
  const uint32_t T = prefix;  // exact key of the K'-th largest score
  const uint32_t k_eq = krem;  // how many keys equal to T are kept
  const uint32_t n_eq_all = s_sel[2];  // how many keys equal T

  if (k_eq == n_eq_all) {
    // Every key equal to T is kept (always so for distinct scores): keep is
    // key >= T, with no index-order ranking.
    static_assert(kItems == 16, "one 16-byte store per thread");
    const bool vec = ((reinterpret_cast<uintptr_t>(kp + r)) & 15u) == 0;
    for (int j0 = tid * kItems; j0 < P; j0 += kThreads * kItems) {
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < kItems; ++e) {
        const int j = j0 + e;
        const uint32_t key = j < P ? (cached ? s_keys[key_slot(j)] : order_key(sc[j])) : 0u;
        packed[e >> 2] |= (j < P && key >= T ? 1u : 0u) << (8 * (e & 3));
      }
      if (vec && j0 + kItems <= P) {
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
  static_assert(kItems == 16, "one 16-byte store per thread");
  const bool vec_store = ((reinterpret_cast<uintptr_t>(kp + r)) & 15u) == 0;
  uint32_t base = 0;  // number of keys == T before the current chunk
  for (int c0 = 0; c0 < P; c0 += kThreads * kItems) {
    uint32_t keys[kItems];
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const int j = c0 + tid * kItems + e;
      keys[e] = j < P ? (cached ? s_keys[key_slot(j)] : order_key(sc[j])) : 0u;
      n_eq += (j < P && keys[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t rank = base + block_excl_scan_u32(n_eq, s_wave, tot);
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

}  // namespace

hipError_t launch_topk_select(const float* score, int B, int N, int r, int K, uint8_t* keep, hipStream_t s) {
  hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(kThreads), 0, s, score, N, r, K, keep);
  return hipGetLastError();
}

}  // namespace tg
