// Sequence RMSNorm of the raw scores (TokenGate paper, Section 4, "Scoring
// Network", second half of Eq. 3): the scores of the prunable tokens are
// divided by their root mean square over the prunable span; the scores of the
// non-prunable tokens are fixed to 0.
//
// One workgroup per batch row.  The data is at most N * 4 bytes (512 KiB at
// N = 128k), so the kernel is latency-bound: each thread issues all of its
// 16-byte loads for a chunk of kThreads * kVec * 4 scores before using any,
// and keeps them in registers for the scaling pass when the row fits one
// chunk.  Each thread's sum of squares over a chunk (32 terms) is fp32;
// chunk, thread and wave partials are combined in fp64 in a fixed order
// (deterministic).
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 1024;
constexpr int kVec = 8;                       // 16-byte loads per thread per chunk
constexpr int kChunk = kThreads * kVec * 4;  // 32768 scores

__device__ __forceinline__ f32x4 load_scores(const float* x, int j, int N, int r, bool vec) {
  f32x4 v;
  if (vec && j + 4 <= N) {
    v = *reinterpret_cast<const f32x4*>(x + j);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = j + i < N ? x[j + i] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = j + i >= r ? v[i] : 0.0f;
  return v;
}

// `in` and `out` may alias (in-place normalisation).
__global__ __launch_bounds__(kThreads) void seq_rmsnorm_kernel(const float* in, int N, int r, float eps,
                                                               float* out) {
  __shared__ double s_part[kThreads / 64];
  __shared__ double s_scale;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const float* x = in + (size_t)b * N;
  float* y = out + (size_t)b * N;
  const int P = N - r;
  const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;

  f32x4 v[kVec];
  double acc = 0.0;
  for (int c0 = 0; c0 < N; c0 += kChunk) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) v[e] = load_scores(x, c0 + (e * kThreads + tid) * 4, N, r, vec);
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < kVec; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(v[e][i], v[e][i], part);
    acc += (double)part;
  }
  acc = wave_sum_f64(acc);
  if ((tid & 63) == 0) s_part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) t += s_part[w];
    s_scale = P > 0 ? 1.0 / sqrt(t / (double)P + (double)eps) : 0.0;
  }
  __syncthreads();
  const double scale = s_scale;
  for (int c0 = 0; c0 < N; c0 += kChunk) {
    if (N > kChunk) {  // otherwise the single chunk is still in registers (read before the barrier)
#pragma unroll
      for (int e = 0; e < kVec; ++e) v[e] = load_scores(x, c0 + (e * kThreads + tid) * 4, N, r, vec);
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const int j = c0 + (e * kThreads + tid) * 4;
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (float)((double)v[e][i] * scale);
      if (vec && j + 4 <= N) {
        *reinterpret_cast<f32x4*>(y + j) = o;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (j + i < N) y[j + i] = o[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_seq_rmsnorm(const float* in, int B, int N, int r, float eps, float* out, hipStream_t s) {
  hipLaunchKernelGGL(seq_rmsnorm_kernel, dim3(B), dim3(kThreads), 0, s, in, N, r, eps, out);
  return hipGetLastError();
}

}  // namespace tg
