// Compaction of the residual stream to the kept set (TokenGate paper,
// Section 4, "Top-K Selector": the residual stream of pruned tokens stops at
// layer L and the kept set continues; Appendix C.4: kept tokens keep their
// original positions).
//
// Two kernels on the same stream:
//  * compact_scan: workgroup c of a batch row takes tokens [c S, c S + S),
//    S = kScanChunk.  It counts the set bytes of the mask before its chunk
//    itself (at most N bytes, L2-resident: no cross-workgroup traffic and no
//    workspace), runs a block-wide exclusive prefix count over its chunk and
//    writes, in ascending original order, kept_idx[m] = j and
//    score_out[m] = score[j].
//  * compact_gather: a streaming 16-byte row copy resid_out[m] = resid[kept_idx[m]],
//    the HBM-bound part (2 * M * row_bytes).
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;                             // consecutive tokens per thread
constexpr int kScanChunk = kScanThreads * kScanItems;     // tokens per workgroup
constexpr int kCountUnroll = 8;                           // 16-byte mask loads in flight per thread
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

// number of non-zero bytes of a 32-bit word
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
  const uint32_t hi = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w;
  return __builtin_popcount(hi & 0x80808080u);
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* s_wave) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) s_wave[wid] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) t += s_wave[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kScanThreads) void compact_scan_kernel(const uint8_t* __restrict__ keep,
                                                                    const float* __restrict__ score, int N,
                                                                    int M, int32_t* __restrict__ kept_idx,
                                                                    float* __restrict__ score_out) {
  __shared__ __attribute__((aligned(16))) uint32_t s_wave[kScanThreads / 64];
  const int b = blockIdx.y;
  const uint8_t* kp = keep + (size_t)b * N;
  const float* sc = score + (size_t)b * N;
  int32_t* ki = kept_idx + (size_t)b * M;
  float* so = score_out + (size_t)b * M;
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * kScanChunk;

  // this chunk: kScanItems consecutive tokens per thread (requested first, so
  // their latency overlaps the count below)
  const int j0 = c0 + tid * kScanItems;
  uint32_t flags = 0;  // bit e: token j0 + e is kept
  float sv[kScanItems];
#pragma unroll
  for (int e = 0; e < kScanItems; ++e) {
    const int j = j0 + e;
    flags |= (j < N && kp[j] != 0) ? (1u << e) : 0u;
    sv[e] = j < N ? sc[j] : 0.0f;
  }

  // ones before this chunk; every load of a batch is issued before any is used
  uint32_t cnt = 0;
  if ((reinterpret_cast<uintptr_t>(kp) & 15u) == 0) {
    const int n16 = c0 / 16;  // c0 is a multiple of 16
    for (int q0 = 0; q0 < n16; q0 += kScanThreads * kCountUnroll) {
      u32x4 w[kCountUnroll];
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u) {
        const int q = q0 + u * kScanThreads + tid;
        w[u] = q < n16 ? load16(kp + (size_t)q * 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u)
        cnt += nonzero_bytes(w[u][0]) + nonzero_bytes(w[u][1]) + nonzero_bytes(w[u][2]) + nonzero_bytes(w[u][3]);
    }
  } else {
    for (int j = tid; j < c0; j += kScanThreads) cnt += kp[j] != 0 ? 1u : 0u;
  }
  const uint32_t base = block_sum_u32(cnt, s_wave);

  uint32_t tot;
  uint32_t dst = base + block_excl_scan_u32<kScanThreads / 64>(__builtin_popcount(flags), s_wave, tot);
#pragma unroll
  for (int e = 0; e < kScanItems; ++e) {
    if (flags & (1u << e)) {
      if ((int)dst < M) {
        ki[dst] = j0 + e;
        so[dst] = sv[e];
      }
      ++dst;
    }
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

// Packed rows of varying count: batch row b owns output rows
// [cu_kept[b], cu_kept[b + 1]); chunk c of row b covers its kept row c / cpr.
__global__ __launch_bounds__(kGatherThreads) void compact_gather_varlen_kernel(
    const uint8_t* __restrict__ resid, size_t row_bytes, int N, const int32_t* __restrict__ cu_kept,
    const int32_t* __restrict__ kept_idx, uint8_t* __restrict__ out) {
  const int b = blockIdx.y;
  const size_t cpr = row_bytes / 16;
  const int o0 = cu_kept[b];
  const int Mb = cu_kept[b + 1] - o0;
  const size_t total = Mb > 0 ? (size_t)Mb * cpr : 0;
  const int32_t* ki = kept_idx + o0;
  const uint8_t* src = resid + (size_t)b * N * row_bytes;
  uint8_t* dst = out + (size_t)o0 * row_bytes;
  const size_t c0 = (size_t)blockIdx.x * kGatherThreads * kGatherUnroll + threadIdx.x;
  u32x4 v[kGatherUnroll];
  size_t off_out[kGatherUnroll];
  bool ok[kGatherUnroll];
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) {
    const size_t c = c0 + (size_t)u * kGatherThreads;
    ok[u] = o0 >= 0 && c < total;
    if (ok[u]) {
      const size_t m = c / cpr, part = c - m * cpr;
      const int32_t j = ki[m];
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

hipError_t launch_compact_gather(const void* resid, size_t row_bytes, int B, int N, int M,
                                 const int32_t* kept_idx, void* resid_out, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const size_t total = (size_t)M * (row_bytes / 16);
  const size_t per_block = (size_t)kGatherThreads * kGatherUnroll;
  const unsigned grid = (unsigned)((total + per_block - 1) / per_block);
  hipLaunchKernelGGL(compact_gather_kernel, dim3(grid, B), dim3(kGatherThreads), 0, s,
                     reinterpret_cast<const uint8_t*>(resid), row_bytes, N, M, kept_idx,
                     reinterpret_cast<uint8_t*>(resid_out));
  return hipGetLastError();
}

hipError_t launch_compact_gather_varlen(const void* resid, size_t row_bytes, int B, int N, const int32_t* cu_kept,
                                        int max_kept, const int32_t* kept_idx, void* resid_out, hipStream_t s) {
  if (max_kept <= 0) return hipSuccess;
  const size_t total = (size_t)max_kept * (row_bytes / 16);
  const size_t per_block = (size_t)kGatherThreads * kGatherUnroll;
  const unsigned grid = (unsigned)((total + per_block - 1) / per_block);
  hipLaunchKernelGGL(compact_gather_varlen_kernel, dim3(grid, B), dim3(kGatherThreads), 0, s,
                     reinterpret_cast<const uint8_t*>(resid), row_bytes, N, cu_kept, kept_idx,
                     reinterpret_cast<uint8_t*>(resid_out));
  return hipGetLastError();
}

hipError_t launch_compact(const void* resid, size_t row_bytes, int B, int N, const uint8_t* keep,
                          const float* score, int M, int32_t* kept_idx, void* resid_out, float* score_out,
                          hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_scan_kernel, dim3((N + kScanChunk - 1) / kScanChunk, B), dim3(kScanThreads), 0, s,
                     keep, score, N, M, kept_idx, score_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_compact_gather(resid, row_bytes, B, N, M, kept_idx, resid_out, s);
}

}  // namespace tg
