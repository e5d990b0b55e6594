// Row gather shared by the compaction of the residual stream (the kept rows,
// TokenGate paper, Section 4, "Top-K Selector") and the KV-cache pruning of
// the layers at and below the gate (Section 5, "Implementation and timing"):
//     dst[m] = src[ki[m]],  m in [0, M)
// A wave moves kGatherRowsPerWave whole rows: it reads their indices, then
// each lane issues its 16-byte chunks of all of them (up to kGatherMaxCpl
// per row and pass; rows longer than 64 kGatherMaxCpl chunks take several
// passes) before any store, with streaming loads and stores.  One wave per
// row keeps each 16-byte access coalesced along the row; four rows per wave
// give 16 loads in flight per lane at 4 KiB rows.  Every load is issued
// unconditionally (a row or chunk that is not moved reads the source's first
// chunk instead, and its store is skipped): a masked load per chunk made the
// compiler wait for each before the next.  An index outside [0, N) leaves its
// row unwritten.  row_bytes is a multiple of 16.
#pragma once

#include "tg_device.h"

namespace tg {

constexpr int kGatherRowsPerWave = 4;
constexpr int kGatherMaxCpl = 4;  // 16-byte chunks per lane, row and pass

// Rows m0 .. m0 + kGatherRowsPerWave - 1 (those below M) by one wave.
__device__ __forceinline__ void gather_rows_wave(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                 size_t row_bytes, int N, int M, const int32_t* __restrict__ ki,
                                                 int m0, int lane) {
  const int cpr = (int)(row_bytes / 16);
  int jrow[kGatherRowsPerWave];
#pragma unroll
  for (int i = 0; i < kGatherRowsPerWave; ++i) jrow[i] = ki[min(m0 + i, M - 1)];
#pragma unroll
  for (int i = 0; i < kGatherRowsPerWave; ++i) jrow[i] = m0 + i < M ? jrow[i] : -1;
  for (int c0 = 0; c0 < cpr; c0 += 64 * kGatherMaxCpl) {
    u32x4 v[kGatherRowsPerWave][kGatherMaxCpl];
#pragma unroll
    for (int i = 0; i < kGatherRowsPerWave; ++i) {
      const bool ok = (uint32_t)jrow[i] < (uint32_t)N;
      const size_t row_off = ok ? (size_t)jrow[i] * row_bytes : 0;
#pragma unroll
      for (int c = 0; c < kGatherMaxCpl; ++c) {
        const int ch = c0 + c * 64 + lane;
        v[i][c] = load16_stream(src + row_off + (size_t)(ch < cpr ? ch : 0) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < kGatherRowsPerWave; ++i) {
      const bool ok = (uint32_t)jrow[i] < (uint32_t)N;
#pragma unroll
      for (int c = 0; c < kGatherMaxCpl; ++c) {
        const int ch = c0 + c * 64 + lane;
        if (ok && ch < cpr)
          __builtin_nontemporal_store(v[i][c],
                                      reinterpret_cast<u32x4*>(dst + (size_t)(m0 + i) * row_bytes + (size_t)ch * 16));
      }
    }
  }
}

}  // namespace tg
