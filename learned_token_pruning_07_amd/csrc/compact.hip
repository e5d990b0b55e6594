// Compaction of the residual stream to the kept set (TokenGate paper,
// Section 4, "Top-K Selector": the residual stream of pruned tokens stops at
// layer L and the kept set continues; Appendix C.4: kept tokens keep their
// original positions).
//
// Two kernels on the same stream:
//  * compact_scan: one workgroup per batch row runs a block-wide exclusive
//    prefix count over the keep mask and writes, in ascending original order,
//    kept_idx[m] = j and score_out[m] = score[j] (a few hundred KiB at most).
//  * compact_gather: a streaming 16-byte row copy resid_out[m] = resid[kept_idx[m]],
//    the HBM-bound part (2 * M * row_bytes).
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanItems = 32;  // consecutive tokens per thread per chunk
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

// Every load of a chunk (keep flags and scores of kScanItems consecutive
// tokens per thread) is issued before the block-wide scan, so a chunk costs
// one memory round trip.
__global__ __launch_bounds__(kScanThreads) void compact_scan_kernel(const uint8_t* __restrict__ keep,
                                                                    const float* __restrict__ score, int N,
                                                                    int M, int32_t* __restrict__ kept_idx,
                                                                    float* __restrict__ score_out) {
  __shared__ uint32_t s_wave[16];
  const int b = blockIdx.x;
  const uint8_t* kp = keep + (size_t)b * N;
  const float* sc = score + (size_t)b * N;
  int32_t* ki = kept_idx + (size_t)b * M;
  float* so = score_out + (size_t)b * M;
  const int tid = threadIdx.x;
  const bool vec = ((reinterpret_cast<uintptr_t>(kp) | reinterpret_cast<uintptr_t>(sc)) & 15u) == 0;
  uint32_t base = 0;
  for (int c0 = 0; c0 < N; c0 += kScanThreads * kScanItems) {
    const int j0 = c0 + tid * kScanItems;
    uint8_t flags[kScanItems];
    float sv[kScanItems];
    if (vec && j0 + kScanItems <= N) {
#pragma unroll
      for (int q = 0; q < kScanItems / 16; ++q) {
        const u32x4 w = load16(kp + j0 + q * 16);
#pragma unroll
        for (int e = 0; e < 16; ++e) flags[q * 16 + e] = ((w[e >> 2] >> ((e & 3) * 8)) & 0xFFu) != 0;
      }
#pragma unroll
      for (int q = 0; q < kScanItems / 4; ++q) {
        const u32x4 w = load16(sc + j0 + q * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[q * 4 + e] = __uint_as_float(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kScanItems; ++e) {
        const int j = j0 + e;
        flags[e] = (j < N && kp[j] != 0) ? 1 : 0;
        sv[e] = j < N ? sc[j] : 0.0f;
      }
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < kScanItems; ++e) cnt += flags[e];
    uint32_t tot;
    uint32_t dst = base + block_excl_scan_u32(cnt, s_wave, tot);
#pragma unroll
    for (int e = 0; e < kScanItems; ++e) {
      if (flags[e]) {
        if ((int)dst < M) {
          ki[dst] = j0 + e;
          so[dst] = sv[e];
        }
        ++dst;
      }
    }
    base += tot;
  }
}

// One thread copies kGatherUnroll 16-byte chunks spaced kGatherThreads apart;
// chunk c of batch row b covers kept row c / cpr, part c % cpr.
__global__ __launch_bounds__(kGatherThreads) void compact_gather_kernel(const uint8_t* __restrict__ resid,
                                                                        size_t row_bytes, int N, int M,
                                                                        const int32_t* __restrict__ kept_idx,
                                                                        uint8_t* __restrict__ out) {
  const int b = blockIdx.y;
  const size_t cpr = row_bytes / 16;
  const size_t total = (size_t)M * cpr;
  const int32_t* ki = kept_idx + (size_t)b * M;
  const uint8_t* src = resid + (size_t)b * N * row_bytes;
  uint8_t* dst = out + (size_t)b * M * row_bytes;
  const size_t c0 = (size_t)blockIdx.x * kGatherThreads * kGatherUnroll + threadIdx.x;
  u32x4 v[kGatherUnroll];
  size_t off_out[kGatherUnroll];
  bool ok[kGatherUnroll];
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) {
    const size_t c = c0 + (size_t)u * kGatherThreads;
    ok[u] = c < total;
    if (ok[u]) {
      const size_t m = c / cpr, part = c - m * cpr;
      const int32_t j = ki[m];
      // a keep mask with fewer ones than M leaves kept_idx entries unwritten;
      // never follow an index outside [0, N)
      ok[u] = (uint32_t)j < (uint32_t)N;
      if (ok[u]) v[u] = load16_stream(src + (size_t)j * row_bytes + part * 16);
      off_out[u] = m * row_bytes + part * 16;
    }
  }
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) {
    if (ok[u]) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst + off_out[u]));
  }
}

}  // namespace

hipError_t launch_compact(const void* resid, size_t row_bytes, int B, int N, const uint8_t* keep,
                          const float* score, int M, int32_t* kept_idx, void* resid_out, float* score_out,
                          hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_scan_kernel, dim3(B), dim3(kScanThreads), 0, s, keep, score, N, M, kept_idx,
                     score_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)M * (row_bytes / 16);
  const size_t per_block = (size_t)kGatherThreads * kGatherUnroll;
  const unsigned grid = (unsigned)((total + per_block - 1) / per_block);
  hipLaunchKernelGGL(compact_gather_kernel, dim3(grid, B), dim3(kGatherThreads), 0, s,
                     reinterpret_cast<const uint8_t*>(resid), row_bytes, N, M, kept_idx,
                     reinterpret_cast<uint8_t*>(resid_out));
  return hipGetLastError();
}

}  // namespace tg
