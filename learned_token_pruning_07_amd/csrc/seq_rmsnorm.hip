// Sequence RMSNorm of the raw scores (TokenGate paper, Section 4, "Scoring
// Network", second half of Eq. 3): the scores of the prunable tokens are
// divided by their root mean square over the prunable span; the scores of the
// non-prunable tokens are fixed to 0.
//
// Rows of up to 32768 scores: one workgroup per batch row.  The kernel is
// latency-bound: each thread issues all of its 16-byte loads for the row
// before using any and keeps them in registers for the scaling pass.
// Longer rows: two launches over slices of kSlice scores -- fp64 partial sums
// of squares per slice into the workspace, then every slice's workgroup sums
// the row's partials in index order and scales its own slice (so the
// in-place call is safe: no slice is written before every sum is taken).
// Each thread's sum of squares (32 terms) is fp32; thread, wave, slice and
// chunk partials are combined in fp64 in a fixed order (deterministic).
#include "select_device.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = sel::kRowThreads;
constexpr int kVec = sel::kRowVec;           // 16-byte loads per thread
constexpr int kChunk = sel::kRowChunk;      // 32768 scores: the single-workgroup limit
static_assert(kChunk == kVarlenOneGroupRow, "the one-workgroup row limit");

// Rows of up to kChunk scores.  `in` and `out` may alias (in-place
// normalisation): every score is read before the barriers of the reduction.
__global__ __launch_bounds__(kThreads) void seq_rmsnorm_kernel(const float* in, int N, int r, int p1, float eps,
                                                               float* out) {
  __shared__ double s_part[kThreads / 64];
  __shared__ double s_scale;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const float* x = in + (size_t)b * N;
  float* y = out + (size_t)b * N;
  const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;

  f32x4 v[kVec];
  sel::load_score_groups<kVec>(v, x, [&](int e) { return (e * kThreads + tid) * 4; }, N, r, p1, vec);
  const double scale = sel::row_inv_rms(v, p1 - r, eps, s_part, &s_scale);
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const int j = (e * kThreads + tid) * 4;
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)  // exactly 0 outside the span, also when the scale is not finite
      o[i] = (j + i >= r && j + i < p1) ? (float)((double)v[e][i] * scale) : 0.0f;
    if (vec && j + 4 <= N) {
      *reinterpret_cast<f32x4*>(y + j) = o;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i < N) y[j + i] = o[i];
    }
  }
}

// ---- rows longer than one chunk ----
constexpr int kSliceThreads = 256;
constexpr int kSlice = kSliceThreads * kVec * 4;  // 8192 scores per workgroup

__device__ __forceinline__ double block_sum_f64(double v, double* s_part) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kSliceThreads / 64; ++w) t += s_part[w];
  return t;
}

// partial[b, c] = sum of squares of the prunable scores in slice c of row b.
// With vr.len set, row b takes its own span, and a row of up to
// kVarlenOneGroupRow tokens is left to the one-workgroup kernel.
__global__ __launch_bounds__(kSliceThreads) void seq_sumsq_kernel(const float* in, int N, int r, int p1,
                                                                  VarlenRows vr, double* __restrict__ partial) {
  __shared__ double s_part[kSliceThreads / 64];
  const int b = blockIdx.y, c0 = blockIdx.x * kSlice, tid = threadIdx.x;
  if (vr.len != nullptr) {
    const RowSpec rs = varlen_row(vr, b, N);
    if (rs.len <= kVarlenOneGroupRow) return;
    r = rs.r;
    p1 = rs.p1;
  }
  const float* x = in + (size_t)b * N;
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  f32x4 v[kVec];
  sel::load_score_groups<kVec>(v, x, [&](int e) { return c0 + (e * kSliceThreads + tid) * 4; }, N, r, p1, vec);
  float part = 0.0f;
#pragma unroll
  for (int e = 0; e < kVec; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(v[e][i], v[e][i], part);
  const double t = block_sum_f64((double)part, s_part);
  if (tid == 0) partial[(size_t)b * gridDim.x + blockIdx.x] = t;
}

// Every workgroup of row b sums the row's partials in index order (the same
// value in each), then scales its own slice.  A slice past a shorter row's
// last prunable token adds an exact 0 to that sum, so a row normalises to
// the same bits in a wider batch.
__global__ __launch_bounds__(kSliceThreads) void seq_scale_kernel(const float* in, int N, int r, int p1, float eps,
                                                                  VarlenRows vr, const double* __restrict__ partial,
                                                                  int nblk, float* out) {
  __shared__ double s_part[kSliceThreads / 64];
  const int b = blockIdx.y, c0 = blockIdx.x * kSlice, tid = threadIdx.x;
  if (vr.len != nullptr) {
    const RowSpec rs = varlen_row(vr, b, N);
    if (rs.len <= kVarlenOneGroupRow) return;
    r = rs.r;
    p1 = rs.p1;
  }
  const float* x = in + (size_t)b * N;
  float* y = out + (size_t)b * N;
  const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
  f32x4 v[kVec];
  sel::load_score_groups<kVec>(v, x, [&](int e) { return c0 + (e * kSliceThreads + tid) * 4; }, N, r, p1, vec);
  double acc = 0.0;
  for (int c = tid; c < nblk; c += kSliceThreads) acc += partial[(size_t)b * nblk + c];
  const double t = block_sum_f64(acc, s_part);
  const int P = p1 - r;
  const double scale = P > 0 ? 1.0 / sqrt(t / (double)P + (double)eps) : 0.0;
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const int j = c0 + (e * kSliceThreads + tid) * 4;
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)  // exactly 0 outside the span, also when the scale is not finite
      o[i] = (j + i >= r && j + i < p1) ? (float)((double)v[e][i] * scale) : 0.0f;
    if (vec && j + 4 <= N) {
      *reinterpret_cast<f32x4*>(y + j) = o;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i < N) y[j + i] = o[i];
    }
  }
}

}  // namespace

size_t seq_rmsnorm_workspace(int B, int N) {
  return N > kChunk ? (size_t)B * ((N + kSlice - 1) / kSlice) * sizeof(double) : 0;
}

hipError_t launch_seq_rmsnorm(const float* in, int B, int N, int r, int p1, float eps, float* out, void* ws,
                              hipStream_t s) {
  if (N <= kChunk) {
    hipLaunchKernelGGL(seq_rmsnorm_kernel, dim3(B), dim3(kThreads), 0, s, in, N, r, p1, eps, out);
    return hipGetLastError();
  }
  const int nblk = (N + kSlice - 1) / kSlice;
  double* partial = static_cast<double*>(ws);
  hipLaunchKernelGGL(seq_sumsq_kernel, dim3(nblk, B), dim3(kSliceThreads), 0, s, in, N, r, p1, VarlenRows{},
                     partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seq_scale_kernel, dim3(nblk, B), dim3(kSliceThreads), 0, s, in, N, r, p1, eps, VarlenRows{},
                     partial, nblk, out);
  return hipGetLastError();
}

hipError_t launch_seq_rmsnorm_long_rows(const float* in, int B, int N, VarlenRows vr, float eps, float* out,
                                        void* ws, hipStream_t s) {
  if (N <= kVarlenOneGroupRow) return hipSuccess;
  const int nblk = (N + kSlice - 1) / kSlice;
  double* partial = static_cast<double*>(ws);
  hipLaunchKernelGGL(seq_sumsq_kernel, dim3(nblk, B), dim3(kSliceThreads), 0, s, in, N, 0, 0, vr, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seq_scale_kernel, dim3(nblk, B), dim3(kSliceThreads), 0, s, in, N, 0, 0, eps, vr, partial, nblk,
                     out);
  return hipGetLastError();
}

}  // namespace tg
