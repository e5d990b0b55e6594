// Post-prefill pruning of the KV cache of the layers at and below the gate
// (TokenGate paper, Section 5, "Implementation and timing", with Appendix B:
// once prefill is done, the KV cache of every layer l <= L may keep only the
// selected tokens, so that decoding holds the same kept entries at every
// layer).  A row gather for each layer and each of K and V:
//     out[l][b, m] = cache[l][b, kept_idx[b, m]]
// with rows of Hkv * d_h two-byte values.  One launch covers every layer and
// both caches (grid z = 2 * layers, y = batch row); each wave moves
// kGatherRowsPerWave kept rows (row_gather.h).
#include "row_gather.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_prune_kernel(const uint8_t* __restrict__ k_cache,
                                                            const uint8_t* __restrict__ v_cache, size_t row_bytes,
                                                            int B, int N, int M, const int32_t* __restrict__ kept_idx,
                                                            uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out) {
  const int z = blockIdx.z;
  const int l = z >> 1;
  const bool is_v = (z & 1) != 0;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* src = (is_v ? v_cache : k_cache) + ((size_t)l * B + b) * (size_t)N * row_bytes;
  uint8_t* dst = (is_v ? v_out : k_out) + ((size_t)l * B + b) * (size_t)M * row_bytes;
  const int m0 = (blockIdx.x * (kThreads / 64) + wave) * kGatherRowsPerWave;
  gather_rows_wave(src, dst, row_bytes, N, M, kept_idx + (size_t)b * M, m0, lane);
}

}  // namespace

hipError_t launch_kv_cache_prune(const void* k_cache, const void* v_cache, int n_layers, int B, int N, int Hkv,
                                 int dh, const int32_t* kept_idx, int M, void* k_out, void* v_out, hipStream_t s) {
  if (M <= 0 || n_layers <= 0) return hipSuccess;
  const size_t row_bytes = (size_t)Hkv * dh * 2;
  const size_t per_block = (size_t)(kThreads / 64) * kGatherRowsPerWave;  // kept rows per workgroup
  const size_t grid = ((size_t)M + per_block - 1) / per_block;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_prune_kernel, dim3((unsigned)grid, B, 2 * n_layers), dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache), row_bytes, B, N, M,
                     kept_idx, static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out));
  return hipGetLastError();
}

}  // namespace tg
