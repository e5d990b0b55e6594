// Row RMSNorm + scoring MLP (TokenGate paper, Section 4, "Scoring Network",
// Eq. 1 and the first half of Eq. 3; Appendix C.4): for every prunable token j
//     a~_j = a_j * w / sqrt(mean(a_j^2) + eps),   b~_j = w2 . silu(W1 a~_j + b1) + b2
// and b~_j = 0 for the non-prunable tokens: those before the prunable span
// [r, p1) (the question x_R) and, when the document is followed by more
// non-prunable text, those after it (the span's end p1 is N for a prompt
// [x_R, x_D]).
//
// bf16 path (the HBM-bound one):
//  * A prepass folds the RMSNorm weight into the first layer once per call,
//    W1w = bf16(W1 * diag(w)) (exact when w = 1), so that W1 a~_j =
//    (W1w a_j) / rms(a_j) and the residual enters the MFMA untouched.  It
//    writes W1w in fragment order: the 64 lanes' B fragments of one
//    (chunk, k-step, wave, column tile) are 1 KiB contiguous, so every
//    fragment load reads whole cache lines.
//  * One workgroup of 4 waves owns a tile of ROWS tokens and ALL h hidden
//    units, so the h -> 1 reduction closes inside the workgroup (no
//    cross-workgroup traffic, fixed summation order).
//  * The residual tile streams HBM -> registers -> LDS in 64-column chunks:
//    loads run kDepth chunks ahead in a register ring (enough bytes in flight
//    per CU to cover HBM latency), LDS is double-buffered.  A chunk row is
//    128 bytes whose 16-byte units are XOR-swizzled by the row's low three
//    bits: the fragment reads (16 rows x 4 units per k-step) are then free of
//    bank conflicts on gfx950, where padded 144-byte rows conflicted 2-way.
//    Wave w computes every row of the tile x its h/4 hidden units with
//    v_mfma_f32_16x16x32_bf16 (fp32 accumulate), its W1w slice streaming from
//    L2 straight into B fragments one chunk ahead.  All global loads are raw
//    buffer loads with a scalar chunk offset: the loop issues no address
//    arithmetic and no per-element VALU work.
//  * Each row's sum of squares comes from the matrix cores too: wave w also
//    multiplies its own row tile's A fragment with itself, whose diagonal is
//    sum_k a_jk^2 (fp32 accumulation of exact bf16 products).
//  * Epilogue: u = acc / rms + b1, silu, times w2, summed over the wave's
//    hidden units (16-lane butterfly), then over the 4 waves in LDS in fixed
//    order.
// fp32 path (small parity workloads): plain fp32 FMA with the normalised rows
// staged in LDS.
#include <mutex>

#include "gate_select_row.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

// The selection part of the fused gate (tg_gate): the row's last workgroup
// to finish its scores runs it, found by counting finished workgroups in
// count[b] (left at zero for the next call).
struct FusedSelect {
  float eps_seq;
  int K;
  float* score;
  uint8_t* keep;
  int32_t* kept_idx;
  float* score_kept;
  uint32_t* count;
};

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKC = 64;             // residual columns per chunk
constexpr int kLda = kKC;           // LDS row (bf16): 128 bytes, 16-byte units XOR-swizzled by row & 7
constexpr int kTpr = kKC / 8;       // threads per row per chunk (16 bytes each)
constexpr int kBufferConfig = 0x00020000;  // raw buffer resource word 3 (gfx9 family, 32-bit data)
constexpr int kDepth = 4;           // residual chunks in flight per workgroup
constexpr int kWDepth = 3;          // W1w fragment chunks resident per wave (two in flight)
constexpr int kUnroll = 12;         // chunk loop unroll: a multiple of 2, kDepth and kWDepth
constexpr int kTallTileMinBlocks = 240;  // 128-token tiles once they give about every CU of the chip a workgroup

__device__ __forceinline__ float silu(float u) { return u / (1.0f + __expf(-u)); }

// Fragment-order W1w: 16-byte unit u = (((c * 2 + ks) * kWaves + w) * CT + ct) * 64 + l holds
// bf16(W1[n][k + i] * norm_w[k + i]), i < 8, with n = w * (h / kWaves) + ct * 16 + (l & 15) and
// k = c * kKC + ks * 32 + (l >> 4) * 8: the B fragment lane l of wave w feeds to its
// MFMAs for column tile ct in k-step ks of chunk c.
__global__ __launch_bounds__(kThreads) void fold_norm_weight_kernel(const uint16_t* __restrict__ W1,
                                                                    const uint16_t* __restrict__ w, int d, int h,
                                                                    uint16_t* __restrict__ W1f) {
  const int u = blockIdx.x * kThreads + threadIdx.x;
  const int CT = h / (kWaves * 16);
  if (u >= h * d / 8) return;
  const int l = u & 63;
  int q = u >> 6;
  const int ct = q % CT;
  q /= CT;
  const int wv = q % kWaves;
  q /= kWaves;  // q = c * 2 + ks
  const int n = wv * (h / kWaves) + ct * 16 + (l & 15);
  const int k = q * 32 + (l >> 4) * 8;
  const u32x4 a = load16(W1 + (size_t)n * d + k), s = load16(w + k);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(bf16_lo(a[j]) * bf16_lo(s[j]), bf16_hi(a[j]) * bf16_hi(s[j]));
  store16(W1f + (size_t)u * 8, o);
}

// s_waitcnt vmcnt(0): every store (and load) this wave issued has completed
// at its L2 (a workgroup barrier alone does not wait for them)
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int H, int ROWS, int WAVES, int NCH_FIXED, bool FUSED = false>
__global__ __launch_bounds__(64 * WAVES) void gate_score_bf16_kernel(const uint16_t* __restrict__ resid, int N,
                                                                   int d, int r_in, int p1_in,
                                                                   const int32_t* __restrict__ span_begin,
                                                                   const int32_t* __restrict__ span_end, float eps_row,
                                                                   const uint16_t* __restrict__ W1w,
                                                                   const float* __restrict__ b1,
                                                                   const uint16_t* __restrict__ w2,
                                                                   const float* __restrict__ b2,
                                                                   float* __restrict__ out, const FusedSelect fs) {
  constexpr int THREADS = 64 * WAVES;
  constexpr int RT = ROWS / 16;               // 16-row MFMA tiles (each wave covers every row)
  constexpr int CT = H / (WAVES * 16);        // 16-column MFMA tiles per wave
  constexpr int AL = ROWS * kTpr / THREADS;   // 16-byte residual loads per thread per chunk
  constexpr int GR = RT / WAVES;              // row tiles whose sum of squares this wave computes
  static_assert(AL >= 1 && CT >= 1 && GR >= 1 && AL * THREADS == ROWS * kTpr && GR * WAVES == RT, "tile shape");

  // LDS: the residual chunks, 1/rms and the per-wave partials of the h -> 1
  // sum (the fused gate's selection reuses the same bytes afterwards)
  constexpr size_t kScoreLds = (size_t)2 * ROWS * kLda * 2 + ROWS * 4 + (size_t)WAVES * ROWS * 4;
  constexpr size_t kLdsBytes = FUSED && selrow::kSelLdsBytes > kScoreLds ? selrow::kSelLdsBytes : kScoreLds;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  auto& sA = *reinterpret_cast<uint16_t(*)[2][ROWS * kLda]>(smem);
  auto& s_inv = *reinterpret_cast<float(*)[ROWS]>(smem + (size_t)2 * ROWS * kLda * 2);
  auto& s_part = *reinterpret_cast<float(*)[WAVES][ROWS]>(smem + (size_t)2 * ROWS * kLda * 2 + ROWS * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  int r = r_in, p1 = p1_in;  // per-row spans of a varying-length batch, clamped into [0, N]
  if (span_begin != nullptr) {  // (a span longer than the grid's p1_in - r_in rows is cut to it)
    p1 = min(max(span_end[b], 0), N);
    r = min(max(span_begin[b], 0), p1);
    p1 = min(p1, r + (p1_in - r_in));
  }
  const int row0 = r + blockIdx.x * ROWS;
  float* ob = out + (size_t)b * N;

  for (int j = blockIdx.x * THREADS + tid; j < r; j += gridDim.x * THREADS) ob[j] = 0.0f;
  for (int j = p1 + blockIdx.x * THREADS + tid; j < N; j += gridDim.x * THREADS) ob[j] = 0.0f;
  // whole workgroup: no barrier is skipped by part of it (the fused gate's
  // workgroups all reach its count, an empty tile with a zero-size range)
  if (!FUSED && row0 >= p1) return;

  // residual tile: rows past the span read as 0 through the buffer range check
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(resid + ((size_t)b * N + row0) * d), (short)0,
      (int)((size_t)max(p1 - row0, 0) * d * 2), kBufferConfig);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(W1w), (short)0, (int)((size_t)H * d * 2), kBufferConfig);
  // slot e of this thread: row (tid + 256 e) / kTpr, columns kp*8 .. kp*8+7 of each chunk
  const int kp = tid % kTpr;
  int a_off[AL], a_lds[AL];
#pragma unroll
  for (int e = 0; e < AL; ++e) {
    const int row = (tid + THREADS * e) / kTpr;
    a_off[e] = (row * d + kp * 8) * 2;
    a_lds[e] = row * kLda + ((kp ^ (row & 7)) * 8);
  }
  // this lane's B fragments in the fragment-ordered W1w (see fold_norm_weight_kernel)
  const int ncol0 = wid * (H / WAVES) + (lane & 15);
  constexpr int kStepBytes = WAVES * CT * 64 * 16;  // one (chunk, k-step) of W1w: H / 16 KiB
  int w_off[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) w_off[ct] = ((wid * CT + ct) * 64 + lane) * 16;

  const int nch = NCH_FIXED > 0 ? NCH_FIXED : d / kKC;
  u32x4 ra[kDepth][AL];        // residual ring: chunk c lives in slot c % kDepth
  u32x4 wb[kWDepth][2][CT];    // W1w fragment ring: chunk c lives in slot c % kWDepth
  // Workgroups start their pass over d at different chunks (logical chunk c
  // is chunk (c + rot) mod nch of the row), so the workgroups of an XCD, which
  // all stream the same W1w fragments, do not ask for the same L2 lines at the
  // same time.  Only the fp32 summation order of a tile's rows depends on it.
  const int rot = (int)(blockIdx.x % (unsigned)nch);
  auto phys = [&](int c) { int p = c + rot; p = p >= nch ? p - nch : p; return p; };
  auto load_a = [&](int c, u32x4 (&dst)[AL]) {
    const int pc = phys(c);
#pragma unroll
    for (int e = 0; e < AL; ++e)
      dst[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off[e], pc * kKC * 2, 0));
  };
  auto store_a = [&](int buf, const u32x4 (&src)[AL]) {
#pragma unroll
    for (int e = 0; e < AL; ++e) store16(&sA[buf][a_lds[e]], src[e]);
  };
  auto load_b = [&](int c, u32x4 (&dst)[2][CT]) {
    const int pc = phys(c);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        dst[ks][ct] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_off[ct], (pc * 2 + ks) * kStepBytes, 0));
  };

  f32x4 acc[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 gram[GR];
#pragma unroll
  for (int i = 0; i < GR; ++i) gram[i] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < kWDepth - 1; ++j)
    if (j < nch) load_b(j, wb[j]);
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (j < nch) load_a(j, ra[j]);
  store_a(0, ra[0]);
  __syncthreads();

  // chunk c: MFMAs on LDS buffer c & 1 with W1w slot c % kWDepth, while the
  // W1w fragments of chunk c + kWDepth - 1 and then residual chunk c + kDepth
  // load into the slots that chunks c - 1 and c vacated, and chunk c + 1 moves
  // ring -> LDS.  Vector loads retire in order, so each wait for a chunk's
  // W1w fragments also waits for the residual chunks issued before them:
  // issuing the fragments first keeps the residual kDepth - 1 chunks ahead.
  constexpr int kOuterUnroll = NCH_FIXED > 0 ? (NCH_FIXED + kUnroll - 1) / kUnroll : 1;
#pragma unroll kOuterUnroll
  for (int c0 = 0; c0 < nch; c0 += kUnroll) {
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int c = c0 + j;
      if (c < nch) {  // uniform
        const int buf = j & 1;  // == c & 1 (kUnroll is even)
        const bool more = c + 1 < nch;
        const u32x4 (&bcur)[2][CT] = wb[j % kWDepth];
        if (c + kWDepth - 1 < nch) load_b(c + kWDepth - 1, wb[(j + kWDepth - 1) % kWDepth]);
        if (c + kDepth < nch) load_a(c + kDepth, ra[j % kDepth]);
        bf16x8 af[2][RT], gf[2][GR];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            af[ks][rt] = *reinterpret_cast<const bf16x8*>(
                &sA[buf][(rt * 16 + (lane & 15)) * kLda + (((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 8)]);
#pragma unroll
          for (int i = 0; i < GR; ++i)
            gf[ks][i] = *reinterpret_cast<const bf16x8*>(
                &sA[buf][((wid + WAVES * i) * 16 + (lane & 15)) * kLda + (((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 8)]);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][rt], as_bf16x8(bcur[ks][ct]), acc[rt][ct],
                                                                    0, 0, 0);
          // Gram tile of this wave's rows: its diagonal is the rows' sum of squares
#pragma unroll
          for (int i = 0; i < GR; ++i) gram[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gf[ks][i], gf[ks][i], gram[i], 0, 0, 0);
        }
        if (more) store_a(buf ^ 1, ra[(j + 1) % kDepth]);
        // Fixed issue order per chunk: the global loads, then every fragment
        // reads, then the products (each waits only for its own fragments),
        // then the LDS stores.  Left to itself the compiler read one fragment
        // just before the two products that use it and waited for it there.
        __builtin_amdgcn_sched_group_barrier(0x020, 2 * CT + AL, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RT + GR), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * (RT * CT + GR), 0);
        __builtin_amdgcn_sched_group_barrier(0x200, AL, 0);
        __syncthreads();
      }
    }
  }

  // 1/rms per row: diagonal element (m, m) of a 16x16 C tile sits in lane
  // m + 16 * (m / 4), register m % 4
#pragma unroll
  for (int i = 0; i < GR; ++i) {
    const int m = lane & 15;
    if ((lane >> 4) == (m >> 2)) {
      const float ssq = gram[i][m & 3];
      s_inv[(wid + WAVES * i) * 16 + m] = 1.0f / sqrtf(ssq / (float)d + eps_row);
    }
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
  if (tid < ROWS && row0 + tid < p1) {
    float v = s_part[0][tid];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v += s_part[w][tid];
    ob[row0 + tid] = v + b2[0];
  }
  if constexpr (FUSED) {
    // the row's last workgroup to finish runs the selection on all of its
    // scores.  Every wave waits until its score stores have reached its L2;
    // after the barrier, thread 0's release (one write-back of this XCD's L2
    // per workgroup) makes them visible device-wide before the workgroup is
    // counted.  Only the last workgroup acquires (invalidating its caches)
    // before it reads the others' scores: an acquire in every workgroup would
    // evict the W1 tiles that the running workgroups stream from L2.
    wait_own_stores();
    __syncthreads();  // (also: every read of s_part is done; LDS is free)
    uint32_t* s_flag = reinterpret_cast<uint32_t*>(smem);
    if (tid == 0) {
      const uint32_t done = __hip_atomic_fetch_add(fs.count + b, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      *s_flag = done == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    const bool last = *s_flag != 0;
    __syncthreads();  // every thread has the flag before the selection reuses LDS
    if (!last) return;  // (workgroup-uniform)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    selrow::gate_select_row<THREADS>(out, N, r_in, p1_in, fs.eps_seq, fs.K, VarlenRows{}, fs.score, fs.keep,
                                     fs.kept_idx, fs.score_kept, b, selrow::carve_sel_lds(smem));
    if (tid == 0) fs.count[b] = 0u;  // zero again for the next call
  }
}

// ---------------------------------------------------------------- fp32 ----
constexpr int kF32Rows = 4;
constexpr int kF32MaxD = 4096;
constexpr int kF32MaxH = 1024;

__global__ __launch_bounds__(kThreads) void gate_score_f32_kernel(const float* __restrict__ resid, int N, int d,
                                                                  int r_in, int p1_in,
                                                                  const int32_t* __restrict__ span_begin,
                                                                  const int32_t* __restrict__ span_end,
                                                                  const float* __restrict__ norm_w,
                                                                  float eps_row, const float* __restrict__ W1,
                                                                  const float* __restrict__ b1, int h,
                                                                  const float* __restrict__ w2,
                                                                  const float* __restrict__ b2,
                                                                  float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float s_x[kF32Rows][kF32MaxD];
  __shared__ float s_act[kF32Rows][kF32MaxH];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.y;
  int r = r_in, p1 = p1_in;
  if (span_begin != nullptr) {  // (a span longer than the grid's p1_in - r_in rows is cut to it)
    p1 = min(max(span_end[b], 0), N);
    r = min(max(span_begin[b], 0), p1);
    p1 = min(p1, r + (p1_in - r_in));
  }
  const int row0 = r + blockIdx.x * kF32Rows;
  float* ob = out + (size_t)b * N;
  for (int j = blockIdx.x * kThreads + tid; j < r; j += gridDim.x * kThreads) ob[j] = 0.0f;
  for (int j = p1 + blockIdx.x * kThreads + tid; j < N; j += gridDim.x * kThreads) ob[j] = 0.0f;
  if (row0 >= p1) return;

  // wave w normalises row row0 + w
  {
    const int row = row0 + wid;
    const bool ok = row < p1;
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
  if (tid < kF32Rows && row0 + tid < p1) {
    float v = 0.0f;
    for (int n = 0; n < h; ++n) v += s_act[tid][n];
    ob[row0 + tid] = v + b2[0];
  }
}

template <int H, int ROWS, int WAVES>
hipError_t launch_rows(const uint16_t* resid, int B, int N, int d, int r, int p1, const int32_t* sb,
                       const int32_t* se, float eps, const uint16_t* W1w,
                       const float* b1, const uint16_t* w2, const float* b2, float* out, const FusedSelect* fs,
                       hipStream_t s) {
  const int P = p1 - r;
  const int nblk = P > 0 ? (P + ROWS - 1) / ROWS : 1;
  // d = 2048 (the model width) gets a fully unrolled chunk loop: the compiler
  // then counts outstanding loads exactly instead of waiting for all of them
  // at the loop's back edge, which would void the prefetch ring
  if (fs != nullptr) {
    if (d == 2048)
      hipLaunchKernelGGL((gate_score_bf16_kernel<H, ROWS, WAVES, 32, true>), dim3(nblk, B), dim3(64 * WAVES), 0, s,
                         resid, N, d, r, p1, sb, se, eps, W1w, b1, w2, b2, out, *fs);
    else
      hipLaunchKernelGGL((gate_score_bf16_kernel<H, ROWS, WAVES, 0, true>), dim3(nblk, B), dim3(64 * WAVES), 0, s,
                         resid, N, d, r, p1, sb, se, eps, W1w, b1, w2, b2, out, *fs);
  } else if (d == 2048) {
    hipLaunchKernelGGL((gate_score_bf16_kernel<H, ROWS, WAVES, 32>), dim3(nblk, B), dim3(64 * WAVES), 0, s, resid,
                       N, d, r, p1, sb, se, eps, W1w, b1, w2, b2, out, FusedSelect{});
  } else {
    hipLaunchKernelGGL((gate_score_bf16_kernel<H, ROWS, WAVES, 0>), dim3(nblk, B), dim3(64 * WAVES), 0, s, resid, N,
                       d, r, p1, sb, se, eps, W1w, b1, w2, b2, out, FusedSelect{});
  }
  return hipGetLastError();
}

template <int H>
hipError_t launch_bf16_h(const uint16_t* resid, int B, int N, int d, int r, int p1, const int32_t* sb,
                         const int32_t* se, float eps, const uint16_t* W1w,
                         const float* b1, const uint16_t* w2, const float* b2, float* out, const FusedSelect* fs,
                         hipStream_t s) {
  // Every workgroup streams all of W1w through L1, so W1 bytes per token fall
  // with the tile height: 128-token tiles of 8 waves (each wave with the
  // registers of the 64-token layout's waves) once they still give about
  // every CU a workgroup, else 64-token tiles of 4 waves.
  const int P = p1 - r;
  if constexpr (H >= 128) {
    if ((long long)B * ((P + 127) / 128) >= kTallTileMinBlocks)
      return launch_rows<H, 128, 8>(resid, B, N, d, r, p1, sb, se, eps, W1w, b1, w2, b2, out, fs, s);
  }
  return launch_rows<H, 64, 4>(resid, B, N, d, r, p1, sb, se, eps, W1w, b1, w2, b2, out, fs, s);
}

hipError_t launch_folded_h(const uint16_t* resid, int B, int N, int d, int r, int p1, const int32_t* sb,
                           const int32_t* se, float eps_row, const uint16_t* W1w, const float* b1, int h,
                           const uint16_t* w2, const float* b2, float* out, const FusedSelect* fs, hipStream_t s) {
  switch (h) {
    case 64:
      return launch_bf16_h<64>(resid, B, N, d, r, p1, sb, se, eps_row, W1w, b1, w2, b2, out, fs, s);
    case 128:
      return launch_bf16_h<128>(resid, B, N, d, r, p1, sb, se, eps_row, W1w, b1, w2, b2, out, fs, s);
    case 256:
      return launch_bf16_h<256>(resid, B, N, d, r, p1, sb, se, eps_row, W1w, b1, w2, b2, out, fs, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gate_score_workspace(int h, int d) { return (size_t)h * d * 2; }

// A fixed scratch array for callers that cannot allocate (tg_gate_score_noalloc):
// it holds the folded W1 in place of a caller's workspace.  Each device that
// runs the library has its own copy, kept until the process ends.  In host
// code the name is only a stand-in for the symbol: kernels and copies use the
// device address looked up below.
static __device__ __align__(256) unsigned char scratch[kGateScoreScratchBytes];

hipError_t gate_score_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_gate_fold(const uint16_t* W1, const uint16_t* norm_w, int h, int d, void* W1f, hipStream_t s) {
  hipLaunchKernelGGL(fold_norm_weight_kernel, dim3((h * d / 8 + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     W1, norm_w, d, h, static_cast<uint16_t*>(W1f));
  return hipGetLastError();
}

hipError_t launch_gate_score_bf16(const uint16_t* resid, int B, int N, int d, int r, int p1, const int32_t* sb,
                                  const int32_t* se, const uint16_t* norm_w,
                                  float eps_row, const uint16_t* W1, const float* b1, int h, const uint16_t* w2,
                                  const float* b2, float* out, void* ws, hipStream_t s) {
  hipError_t e = launch_gate_fold(W1, norm_w, h, d, ws, s);
  if (e != hipSuccess) return e;
  return launch_gate_score_folded(resid, B, N, d, r, p1, sb, se, eps_row, static_cast<const uint16_t*>(ws), b1, h,
                                  w2, b2, out, s);
}

hipError_t launch_gate_score_folded(const uint16_t* resid, int B, int N, int d, int r, int p1, const int32_t* sb,
                                    const int32_t* se, float eps_row, const uint16_t* W1w, const float* b1, int h,
                                    const uint16_t* w2, const float* b2, float* out, hipStream_t s) {
  return launch_folded_h(resid, B, N, d, r, p1, sb, se, eps_row, W1w, b1, h, w2, b2, out, nullptr, s);
}

hipError_t launch_gate_fused(const uint16_t* resid, int B, int N, int d, int r, const uint16_t* W1w, float eps_row,
                             const float* b1, int h, const uint16_t* w2, const float* b2, float eps_seq, int K,
                             float* score_raw, float* score, uint8_t* keep, int32_t* kept_idx, uint16_t* resid_out,
                             float* score_kept, uint32_t* count, hipStream_t s) {
  if (N > sel::kRowChunk) return hipErrorInvalidValue;
  const FusedSelect fs{eps_seq, K, score, keep, kept_idx, score_kept, count};
  hipError_t e = launch_folded_h(resid, B, N, d, r, N, nullptr, nullptr, eps_row, W1w, b1, h, w2, b2, score_raw,
                                 &fs, s);
  if (e != hipSuccess) return e;
  const int P = N - r;
  const int M = N - P + (K < P ? K : P);
  return launch_compact_gather(resid, (size_t)d * 2, B, N, M, kept_idx, resid_out, s);
}

hipError_t launch_gate_score_f32(const float* resid, int B, int N, int d, int r, int p1, const int32_t* sb,
                                 const int32_t* se, const float* norm_w,
                                 float eps_row, const float* W1, const float* b1, int h, const float* w2,
                                 const float* b2, float* out, hipStream_t s) {
  if (d > kF32MaxD || h > kF32MaxH) return hipErrorInvalidValue;
  const int P = p1 - r;
  const int nblk = P > 0 ? (P + kF32Rows - 1) / kF32Rows : 1;
  hipLaunchKernelGGL(gate_score_f32_kernel, dim3(nblk, B), dim3(kThreads), 0, s, resid, N, d, r, p1, sb, se, norm_w, eps_row,
                     W1, b1, h, w2, b2, out);
  return hipGetLastError();
}

}  // namespace tg
