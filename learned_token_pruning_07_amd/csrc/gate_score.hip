// Row RMSNorm + scoring MLP (TokenGate paper, Section 4, "Scoring Network",
// Eq. 1 and the first half of Eq. 3; Appendix C.4): for every prunable token j
//     a~_j = a_j * w / sqrt(mean(a_j^2) + eps),   b~_j = w2 . silu(W1 a~_j + b1) + b2
// and b~_j = 0 for the non-prunable tokens j < r.
//
// bf16 path (the HBM-bound one): one workgroup of 4 waves owns a tile of
// kRows tokens and ALL h hidden units, so the h -> 1 reduction closes inside
// the workgroup (no cross-workgroup traffic, fixed summation order).
//  * The residual tile streams HBM -> registers (non-temporal: read once) ->
//    LDS in 64-column chunks, double-buffered.  On the way the row's sum of
//    squares is accumulated and the RMSNorm weight is applied; the 1/rms
//    factor is folded into the epilogue: W1 (w (.) a) * inv_rms.
//  * Wave w computes all kRows tokens x its h/4 hidden units with
//    v_mfma_f32_16x16x32_bf16 (fp32 accumulate).  Its W1 slice streams from
//    L2 (W1 is 1 MiB at d=2048, h=256, shared by every workgroup) straight
//    into MFMA B-fragments, one chunk ahead.
//  * Epilogue: u = acc * inv_rms + b1, silu, times w2, summed over the wave's
//    hidden units (16-lane butterfly), then over the 4 waves in LDS in fixed
//    order.
// fp32 path (small parity workloads): plain fp32 FMA with the normalised rows
// staged in LDS.
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKC = 64;             // residual columns per chunk
constexpr int kLda = kKC + 8;       // padded LDS row (bf16): conflict-free fragment reads
constexpr int kTpr = kKC / 8;       // threads per row per chunk (16 bytes each)

__device__ __forceinline__ float silu(float u) { return u / (1.0f + __expf(-u)); }

template <int H, int ROWS>
__global__ __launch_bounds__(kThreads) void gate_score_bf16_kernel(
    const uint16_t* __restrict__ resid, int N, int d, int r, const uint16_t* __restrict__ norm_w, float eps_row,
    const uint16_t* __restrict__ W1, const float* __restrict__ b1, const uint16_t* __restrict__ w2,
    const float* __restrict__ b2, float* __restrict__ out) {
  constexpr int RT = ROWS / 16;               // 16-row MFMA tiles (each wave covers every row)
  constexpr int CT = H / (kWaves * 16);       // 16-column MFMA tiles per wave
  constexpr int AL = ROWS * kTpr / kThreads;  // 16-byte residual loads per thread per chunk
  static_assert(AL >= 1 && CT >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][ROWS * kLda];
  __shared__ float s_inv[ROWS];
  __shared__ float s_part[kWaves][ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.y;
  const int row0 = r + blockIdx.x * ROWS;
  const uint16_t* Rb = resid + (size_t)b * N * d;
  float* ob = out + (size_t)b * N;

  for (int j = blockIdx.x * kThreads + tid; j < r; j += gridDim.x * kThreads) ob[j] = 0.0f;
  if (row0 >= N) return;  // whole workgroup: no barrier is skipped by part of it

  // residual staging slots: slot e covers row (tid + 256 e) / kTpr, columns kp*8..kp*8+7
  const int kp = tid % kTpr;
  int a_row[AL];
  bool a_ok[AL];
#pragma unroll
  for (int e = 0; e < AL; ++e) {
    a_row[e] = (tid + kThreads * e) / kTpr;
    a_ok[e] = row0 + a_row[e] < N;
  }
  float ss[AL];
#pragma unroll
  for (int e = 0; e < AL; ++e) ss[e] = 0.0f;

  // W1 rows this lane feeds into its B fragments
  const int ncol0 = wid * (H / kWaves) + (lane & 15);
  const int kq = (lane >> 4) * 8;  // k offset of this lane inside a 32-wide k-step

  const int nch = (d + kKC - 1) / kKC;
  u32x4 ra[AL], rw;
  u32x4 bcur[2][CT], bnext[2][CT];

  auto load_a = [&](int c) {
    const int k = c * kKC + kp * 8;
    const bool kin = k < d;
    rw = kin ? load16(norm_w + k) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < AL; ++e)
      ra[e] = (kin && a_ok[e]) ? load16_stream(Rb + (size_t)(row0 + a_row[e]) * d + k) : u32x4{0, 0, 0, 0};
  };
  auto store_a = [&](int buf) {
    float w[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = bf16_lo(rw[i]);
      w[2 * i + 1] = bf16_hi(rw[i]);
    }
#pragma unroll
    for (int e = 0; e < AL; ++e) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = bf16_lo(ra[e][i]), hi = bf16_hi(ra[e][i]);
        ss[e] = fmaf(lo, lo, ss[e]);
        ss[e] = fmaf(hi, hi, ss[e]);
        o[i] = pack_bf16x2(lo * w[2 * i], hi * w[2 * i + 1]);
      }
      store16(&sA[buf][a_row[e] * kLda + kp * 8], o);
    }
  };
  auto load_b = [&](int c, u32x4 (&dst)[2][CT]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int k = c * kKC + ks * 32 + kq;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        dst[ks][ct] = k < d ? load16(W1 + (size_t)(ncol0 + ct * 16) * d + k) : u32x4{0, 0, 0, 0};
    }
  };

  f32x4 acc[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  load_b(0, bcur);
  store_a(0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more) {
      load_a(c + 1);
      load_b(c + 1, bnext);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        af[rt] = *reinterpret_cast<const bf16x8*>(&sA[buf][(rt * 16 + (lane & 15)) * kLda + ks * 32 + kq]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt], as_bf16x8(bcur[ks][ct]), acc[rt][ct], 0,
                                                                0, 0);
    }
    if (more) {
      store_a(buf ^ 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bcur[ks][ct] = bnext[ks][ct];
    }
    __syncthreads();
  }

  // 1/rms per row: the kTpr threads of a row are consecutive lanes
#pragma unroll
  for (int e = 0; e < AL; ++e) {
    float t = ss[e];
#pragma unroll
    for (int o = 1; o < kTpr; o <<= 1) t += __shfl_xor(t, o, 64);
    if (kp == 0) s_inv[a_row[e]] = 1.0f / sqrtf(t / (float)d + eps_row);
  }
  __syncthreads();

  // epilogue: C fragment lane l holds column (l & 15), rows 4*(l >> 4) + i
  float bias1[CT], wout[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int n = ncol0 + ct * 16;
    bias1[ct] = b1[n];
    wout[ct] = bf16_to_f32(w2[n]);
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * 16 + (lane >> 4) * 4 + i;
      const float inv = s_inv[row];
      float part = 0.0f;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) part = fmaf(wout[ct], silu(fmaf(acc[rt][ct][i], inv, bias1[ct])), part);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) part += __shfl_xor(part, o, 64);
      if ((lane & 15) == 0) s_part[wid][row] = part;
    }
  }
  __syncthreads();
  if (tid < ROWS && row0 + tid < N) {
    float v = s_part[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += s_part[w][tid];
    ob[row0 + tid] = v + b2[0];
  }
}

// ---------------------------------------------------------------- fp32 ----
constexpr int kF32Rows = 4;
constexpr int kF32MaxD = 4096;
constexpr int kF32MaxH = 1024;

__global__ __launch_bounds__(kThreads) void gate_score_f32_kernel(const float* __restrict__ resid, int N, int d,
                                                                  int r, const float* __restrict__ norm_w,
                                                                  float eps_row, const float* __restrict__ W1,
                                                                  const float* __restrict__ b1, int h,
                                                                  const float* __restrict__ w2,
                                                                  const float* __restrict__ b2,
                                                                  float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float s_x[kF32Rows][kF32MaxD];
  __shared__ float s_act[kF32Rows][kF32MaxH];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.y;
  const int row0 = r + blockIdx.x * kF32Rows;
  float* ob = out + (size_t)b * N;
  for (int j = blockIdx.x * kThreads + tid; j < r; j += gridDim.x * kThreads) ob[j] = 0.0f;
  if (row0 >= N) return;

  // wave w normalises row row0 + w
  {
    const int row = row0 + wid;
    const bool ok = row < N;
    const float* a = resid + ((size_t)b * N + (ok ? row : 0)) * d;
    float ssq = 0.0f;
    for (int k = lane; k < d; k += 64) {
      const float x = ok ? a[k] : 0.0f;
      ssq = fmaf(x, x, ssq);
    }
    ssq = wave_sum_f32(ssq);
    const float inv = 1.0f / sqrtf(ssq / (float)d + eps_row);
    for (int k = lane; k < d; k += 64) s_x[wid][k] = ok ? a[k] * inv * norm_w[k] : 0.0f;
  }
  __syncthreads();
  for (int idx = tid; idx < kF32Rows * h; idx += kThreads) {
    const int rr = idx / h, n = idx - rr * h;
    const float* wr = W1 + (size_t)n * d;
    float u = 0.0f;
    for (int k = 0; k < d; k += 4) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + k);
      u = fmaf(s_x[rr][k], wv.x, u);
      u = fmaf(s_x[rr][k + 1], wv.y, u);
      u = fmaf(s_x[rr][k + 2], wv.z, u);
      u = fmaf(s_x[rr][k + 3], wv.w, u);
    }
    u += b1[n];
    s_act[rr][n] = w2[n] * (u / (1.0f + expf(-u)));
  }
  __syncthreads();
  if (tid < kF32Rows && row0 + tid < N) {
    float v = 0.0f;
    for (int n = 0; n < h; ++n) v += s_act[tid][n];
    ob[row0 + tid] = v + b2[0];
  }
}

template <int H>
hipError_t launch_bf16_h(const uint16_t* resid, int B, int N, int d, int r, const uint16_t* norm_w, float eps,
                         const uint16_t* W1, const float* b1, const uint16_t* w2, const float* b2, float* out,
                         hipStream_t s) {
  constexpr int ROWS = 64;
  const int P = N - r;
  const int nblk = P > 0 ? (P + ROWS - 1) / ROWS : 1;
  hipLaunchKernelGGL((gate_score_bf16_kernel<H, ROWS>), dim3(nblk, B), dim3(kThreads), 0, s, resid, N, d, r,
                     norm_w, eps, W1, b1, w2, b2, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_score_bf16(const uint16_t* resid, int B, int N, int d, int r, const uint16_t* norm_w,
                                  float eps_row, const uint16_t* W1, const float* b1, int h, const uint16_t* w2,
                                  const float* b2, float* out, hipStream_t s) {
  switch (h) {
    case 64:
      return launch_bf16_h<64>(resid, B, N, d, r, norm_w, eps_row, W1, b1, w2, b2, out, s);
    case 128:
      return launch_bf16_h<128>(resid, B, N, d, r, norm_w, eps_row, W1, b1, w2, b2, out, s);
    case 256:
      return launch_bf16_h<256>(resid, B, N, d, r, norm_w, eps_row, W1, b1, w2, b2, out, s);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gate_score_f32(const float* resid, int B, int N, int d, int r, const float* norm_w,
                                 float eps_row, const float* W1, const float* b1, int h, const float* w2,
                                 const float* b2, float* out, hipStream_t s) {
  if (d > kF32MaxD || h > kF32MaxH) return hipErrorInvalidValue;
  const int P = N - r;
  const int nblk = P > 0 ? (P + kF32Rows - 1) / kF32Rows : 1;
  hipLaunchKernelGGL(gate_score_f32_kernel, dim3(nblk, B), dim3(kThreads), 0, s, resid, N, d, r, norm_w, eps_row,
                     W1, b1, h, w2, b2, out);
  return hipGetLastError();
}

}  // namespace tg
