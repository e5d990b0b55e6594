// Device-side helpers shared by the TokenGate HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 values -> two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 values -> two fp16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Wave64 reductions (fixed butterfly order: deterministic).
__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Max / sum of x with the partner lane (lane ^ 32), identical in both lanes
// (v_permlane32_swap exchanges the two 32-lane halves of a wave).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves: a
// Hillis-Steele scan inside each 16-lane row (shifts 1, 2, 4, 8; lanes
// shifted in from outside the row read 0), then the last lane of row 0 is
// added to row 1 and of row 2 to row 3 (row_bcast:15), and the last lane of
// row 1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 1, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 2, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 4, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 8, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast15, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast31, 0xC, 0xF, false);
  return x;
}

// Running maximum over the 64 lanes of a wave, on the same DPP lane moves
// (lanes shifted in from outside a row read 0, the identity): lane 63 ends
// with the wave's maximum.
__device__ __forceinline__ uint32_t wave_incl_max_u32(uint32_t x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 1, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 2, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 4, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 8, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast15, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast31, 0xC, 0xF, false));
  return x;
}

// Exclusive prefix sum over a whole block of NW waves (blockDim.x == 64 NW,
// NW a multiple of 4, at most 16).  `s_wave` holds NW words of LDS, 16-byte
// aligned.  Returns the exclusive prefix of `v`; `total` receives the block
// total.  Contains barriers: every thread of the block must call it.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  static_assert(NW % 4 == 0 && NW <= 16, "wave count");
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == 63) s_wave[wid] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < NW / 4; ++q) {
    const u32x4 t = reinterpret_cast<const u32x4*>(s_wave)[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      before += (4 * q + i < wid) ? t[i] : 0u;
      tot += t[i];
    }
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// Workgroup id remapped so that consecutive logical ids land on the same XCD.
// The hardware hands workgroups to the 8 XCDs round-robin; this bijection
// gives XCD x the contiguous logical range [x*q + min(x, rem), ...).
__device__ __forceinline__ int xcd_logical_id(int id, int total) {
  const int q = total >> 3, rem = total & 7;
  const int x = id & 7;
  return x * q + (x < rem ? x : rem) + (id >> 3);
}

// The last s < n with first[s] <= x, for non-decreasing first[] with
// first[0] = 0 <= x (the sequence of a block or workgroup in a varlen table;
// empty sequences, whose first equals the next one's, are never returned
// for x < first[n]).
__device__ __forceinline__ int seq_of(const int* first, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace tg
