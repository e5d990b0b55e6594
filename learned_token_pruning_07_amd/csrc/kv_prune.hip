// Post-prefill pruning of the KV cache of the layers at and below the gate
// (TokenGate paper, Section 5, "Implementation and timing", with Appendix B:
// once prefill is done, the KV cache of every layer l <= L may keep only the
// selected tokens, so that decoding holds the same kept entries at every
// layer).  A row gather for each layer and each of K and V:
//     out[l][b, m] = cache[l][b, kept_idx[b, m]]
// with rows of Hkv * d_h two-byte values.  One launch covers every layer and
// both caches (grid z = 2 * layers, y = batch row).  A wave moves
// kRowsPerWave kept rows: it reads their indices, then each lane issues its
// 16-byte chunks of all of them (up to kMaxCpl per row and pass; rows longer
// than 64 * kMaxCpl chunks take several passes) before any store, with
// streaming loads and stores.  One wave per row keeps each 16-byte access
// coalesced along the row; four rows per wave give 8 loads in flight per lane
// at the stage's 2 KiB rows.
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 4;
constexpr int kMaxCpl = 4;  // 16-byte chunks per lane, row and pass

__global__ __launch_bounds__(kThreads) void kv_prune_kernel(const uint8_t* __restrict__ k_cache,
                                                            const uint8_t* __restrict__ v_cache, size_t row_bytes,
                                                            int B, int N, int M, const int32_t* __restrict__ kept_idx,
                                                            uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out) {
  const int z = blockIdx.z;
  const int l = z >> 1;
  const bool is_v = (z & 1) != 0;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cpr = (int)(row_bytes / 16);
  const int32_t* ki = kept_idx + (size_t)b * M;
  const uint8_t* src = (is_v ? v_cache : k_cache) + ((size_t)l * B + b) * (size_t)N * row_bytes;
  uint8_t* dst = (is_v ? v_out : k_out) + ((size_t)l * B + b) * (size_t)M * row_bytes;
  const int m0 = (blockIdx.x * (kThreads / 64) + wave) * kRowsPerWave;
  int jrow[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) jrow[i] = m0 + i < M ? ki[m0 + i] : -1;
  for (int c0 = 0; c0 < cpr; c0 += 64 * kMaxCpl) {
    u32x4 v[kRowsPerWave][kMaxCpl];
    // every load is issued unconditionally (a row or chunk that is not moved
    // reads the cache's first chunk instead, and its store is skipped): a
    // masked load per chunk made the compiler wait for each before the next
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const bool ok = (uint32_t)jrow[i] < (uint32_t)N;  // an index outside [0, N) leaves its row unwritten
      const size_t row_off = ok ? (size_t)jrow[i] * row_bytes : 0;
#pragma unroll
      for (int c = 0; c < kMaxCpl; ++c) {
        const int ch = c0 + c * 64 + lane;
        v[i][c] = load16_stream(src + row_off + (size_t)(ch < cpr ? ch : 0) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const bool ok = (uint32_t)jrow[i] < (uint32_t)N;
#pragma unroll
      for (int c = 0; c < kMaxCpl; ++c) {
        const int ch = c0 + c * 64 + lane;
        if (ok && ch < cpr)
          __builtin_nontemporal_store(v[i][c],
                                      reinterpret_cast<u32x4*>(dst + (size_t)(m0 + i) * row_bytes + (size_t)ch * 16));
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_cache_prune(const void* k_cache, const void* v_cache, int n_layers, int B, int N, int Hkv,
                                 int dh, const int32_t* kept_idx, int M, void* k_out, void* v_out, hipStream_t s) {
  if (M <= 0 || n_layers <= 0) return hipSuccess;
  const size_t row_bytes = (size_t)Hkv * dh * 2;
  const size_t per_block = (size_t)(kThreads / 64) * kRowsPerWave;  // kept rows per workgroup
  const size_t grid = ((size_t)M + per_block - 1) / per_block;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_prune_kernel, dim3((unsigned)grid, B, 2 * n_layers), dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache), row_bytes, B, N, M,
                     kept_idx, static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out));
  return hipGetLastError();
}

}  // namespace tg
