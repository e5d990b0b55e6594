// Sequence RMSNorm of the raw scores (TokenGate paper, Section 4, "Scoring
// Network", second half of Eq. 3): the scores of the prunable tokens are
// divided by their root mean square over the prunable span; the scores of the
// non-prunable tokens are fixed to 0.
//
// One workgroup per batch row.  The sum of squares is accumulated in fp64 per
// thread and reduced in a fixed butterfly/wave order, so the result is
// deterministic.  The data is at most N * 4 bytes (512 KiB at N = 128k): this
// kernel is latency-bound, not bandwidth-bound.
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void seq_rmsnorm_kernel(const float* __restrict__ in, int N, int r,
                                                               float eps, float* __restrict__ out) {
  __shared__ double s_part[kThreads / 64];
  __shared__ double s_scale;
  const int b = blockIdx.x;
  const float* x = in + (size_t)b * N;
  float* y = out + (size_t)b * N;
  const int P = N - r;

  double acc = 0.0;
  for (int j = r + threadIdx.x; j < N; j += kThreads) {
    const double v = (double)x[j];
    acc = fma(v, v, acc);
  }
  acc = wave_sum_f64(acc);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) t += s_part[w];
    s_scale = P > 0 ? 1.0 / sqrt(t / (double)P + (double)eps) : 0.0;
  }
  __syncthreads();
  const double scale = s_scale;
  for (int j = threadIdx.x; j < N; j += kThreads) {
    y[j] = j < r ? 0.0f : (float)((double)x[j] * scale);
  }
}

}  // namespace

hipError_t launch_seq_rmsnorm(const float* in, int B, int N, int r, float eps, float* out, hipStream_t s) {
  hipLaunchKernelGGL(seq_rmsnorm_kernel, dim3(B), dim3(kThreads), 0, s, in, N, r, eps, out);
  return hipGetLastError();
}

}  // namespace tg
