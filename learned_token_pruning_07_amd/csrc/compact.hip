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
//    the HBM-bound part (2 * M * row_bytes), a wave per kGatherRowsPerWave
//    kept rows (row_gather.h).
#include "row_gather.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;                             // consecutive tokens per thread
constexpr int kScanChunk = kScanThreads * kScanItems;     // tokens per workgroup
constexpr int kCountUnroll = 8;                           // 16-byte mask loads in flight per thread
constexpr int kGatherThreads = 256;
constexpr int kGatherRowsPerBlock = (kGatherThreads / 64) * kGatherRowsPerWave;

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

// With vr.len set: rows of a varying-length batch longer than
// kVarlenOneGroupRow tokens only, row b writing at most cu_kept[b + 1] -
// cu_kept[b] entries from cu_kept[b] on.
__global__ __launch_bounds__(kScanThreads) void compact_scan_kernel(const uint8_t* __restrict__ keep,
                                                                    const float* __restrict__ score, int N,
                                                                    int M, VarlenRows vr,
                                                                    int32_t* __restrict__ kept_idx,
                                                                    float* __restrict__ score_out) {
  __shared__ __attribute__((aligned(16))) uint32_t s_wave[kScanThreads / 64];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * kScanChunk;
  size_t out0 = (size_t)b * M;
  if (vr.len != nullptr) {
    const RowSpec rs = varlen_row(vr, b, N);
    if (rs.len <= kVarlenOneGroupRow || c0 >= rs.len) return;  // (no kept token past the length)
    out0 = (size_t)max(vr.cu_kept[b], 0);
    M = vr.cu_kept[b + 1] - vr.cu_kept[b];
  }
  const uint8_t* kp = keep + (size_t)b * N;
  const float* sc = score + (size_t)b * N;
  int32_t* ki = kept_idx + out0;
  float* so = score_out + out0;

  // this chunk: kScanItems consecutive tokens per thread (requested first, so
  // their latency overlaps the count below)
  const int j0 = c0 + tid * kScanItems;
  uint32_t flags = 0;  // bit e: token j0 + e is kept
  float sv[kScanItems];
#pragma unroll
  for (int e = 0; e < kScanItems; ++e) {  // (clamped, unconditional loads: masked ones would each be waited for)
    const int j = j0 + e, jc = min(j, N - 1);
    const uint8_t kv = kp[jc];
    const float x = sc[jc];
    flags |= (j < N && kv != 0) ? (1u << e) : 0u;
    sv[e] = j < N ? x : 0.0f;
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
        w[u] = load16(kp + (size_t)min(q, n16 - 1) * 16);  // (q0 < n16, so n16 >= 1)
      }
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u)
        if (q0 + u * kScanThreads + tid >= n16) w[u] = u32x4{0, 0, 0, 0};
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

// Batch row b: kept rows m0 .. m0 + kGatherRowsPerWave - 1 per wave.
__global__ __launch_bounds__(kGatherThreads) void compact_gather_kernel(const uint8_t* __restrict__ resid,
                                                                        size_t row_bytes, int N, int M,
                                                                        const int32_t* __restrict__ kept_idx,
                                                                        uint8_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = (blockIdx.x * (kGatherThreads / 64) + wave) * kGatherRowsPerWave;
  if (m0 >= M) return;
  // (a keep mask with fewer ones than M leaves kept_idx entries unwritten;
  // the gather never follows an index outside [0, N))
  gather_rows_wave(resid + (size_t)b * N * row_bytes, out + (size_t)b * M * row_bytes, row_bytes, N, M,
                   kept_idx + (size_t)b * M, m0, lane);
}

// Packed rows of varying count: batch row b owns output rows
// [cu_kept[b], cu_kept[b + 1]).  With count set instead (pad rows per batch
// row), batch row b owns output rows [b pad, b pad + count[b]).
__global__ __launch_bounds__(kGatherThreads) void compact_gather_varlen_kernel(
    const uint8_t* __restrict__ resid, size_t row_bytes, int N, const int32_t* __restrict__ cu_kept,
    const int32_t* __restrict__ count, int pad, const int32_t* __restrict__ kept_idx, uint8_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int o0 = count != nullptr ? b * pad : cu_kept[b];
  const int Mb = count != nullptr ? min(max(count[b], 0), pad) : cu_kept[b + 1] - o0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = (blockIdx.x * (kGatherThreads / 64) + wave) * kGatherRowsPerWave;
  if (o0 < 0 || m0 >= Mb) return;
  gather_rows_wave(resid + (size_t)b * N * row_bytes, out + (size_t)o0 * row_bytes, row_bytes, N, Mb,
                   kept_idx + o0, m0, lane);
}

}  // namespace

hipError_t launch_compact_gather(const void* resid, size_t row_bytes, int B, int N, int M,
                                 const int32_t* kept_idx, void* resid_out, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(((size_t)M + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock);
  hipLaunchKernelGGL(compact_gather_kernel, dim3(grid, B), dim3(kGatherThreads), 0, s,
                     reinterpret_cast<const uint8_t*>(resid), row_bytes, N, M, kept_idx,
                     reinterpret_cast<uint8_t*>(resid_out));
  return hipGetLastError();
}

hipError_t launch_compact_gather_varlen(const void* resid, size_t row_bytes, int B, int N, const int32_t* cu_kept,
                                        int max_kept, const int32_t* kept_idx, void* resid_out, hipStream_t s) {
  if (max_kept <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(((size_t)max_kept + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock);
  hipLaunchKernelGGL(compact_gather_varlen_kernel, dim3(grid, B), dim3(kGatherThreads), 0, s,
                     reinterpret_cast<const uint8_t*>(resid), row_bytes, N, cu_kept, nullptr, 0, kept_idx,
                     reinterpret_cast<uint8_t*>(resid_out));
  return hipGetLastError();
}

hipError_t launch_compact_gather_padded(const void* resid, size_t row_bytes, int B, int N, const int32_t* count,
                                        int pad, const int32_t* kept_idx, void* resid_out, hipStream_t s) {
  if (pad <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(((size_t)pad + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock);
  hipLaunchKernelGGL(compact_gather_varlen_kernel, dim3(grid, B), dim3(kGatherThreads), 0, s,
                     reinterpret_cast<const uint8_t*>(resid), row_bytes, N, nullptr, count, pad, kept_idx,
                     reinterpret_cast<uint8_t*>(resid_out));
  return hipGetLastError();
}

hipError_t launch_compact(const void* resid, size_t row_bytes, int B, int N, const uint8_t* keep,
                          const float* score, int M, int32_t* kept_idx, void* resid_out, float* score_out,
                          hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_scan_kernel, dim3((N + kScanChunk - 1) / kScanChunk, B), dim3(kScanThreads), 0, s,
                     keep, score, N, M, VarlenRows{}, kept_idx, score_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_compact_gather(resid, row_bytes, B, N, M, kept_idx, resid_out, s);
}

hipError_t launch_compact_scan_long_rows(const uint8_t* keep, const float* score, int B, int N, VarlenRows vr,
                                         int32_t* kept_idx, float* score_out, hipStream_t s) {
  if (N <= kVarlenOneGroupRow) return hipSuccess;
  hipLaunchKernelGGL(compact_scan_kernel, dim3((N + kScanChunk - 1) / kScanChunk, B), dim3(kScanThreads), 0, s,
                     keep, score, N, 0, vr, kept_idx, score_out);
  return hipGetLastError();
}

}  // namespace tg
