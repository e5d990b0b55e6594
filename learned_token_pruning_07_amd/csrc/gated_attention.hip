// Token-gated causal GQA attention over the kept set (TokenGate paper,
// Section 4: token-gated attention Eq. 5, head-wise gain Eq. 6, temperature
// Eq. 7, combined into the key-bias form Eq. 8; Appendix C.4).
//
//   z_ij = (q_i . k_j) * sm_scale / (temp_h * ratio_i) + gain_h * b_j,  j <= i
//   ratio_i = 1 if pos_i == i else ln(max(pos_i+1, 2)) / ln(max(i+1, 2))
//
// Flash-style forward on gfx950: Q.K^T on bf16 MFMA 32x32x16, P.V on fp16 MFMA
// 32x32x16, fp32 accumulation, fp32 softmax.
//  * Workgroup = 2 groups x 4 waves.  Within a group the 4 waves are the G
//    query heads of one KV head x (4/G) sets of 32 query rows, so every K/V
//    tile staged in LDS serves G heads.  The two groups split the block's key
//    range (group g takes tiles g, g+2, ...) and merge their online-softmax
//    states in LDS at the end: the longest causal row runs as two
//    independent chains, one per wave slot of each SIMD.
//  * Scores are computed transposed, S^T = K Q^T: a lane owns one query and
//    16 keys of a 32-key tile, so the row max/sum is an in-lane reduction
//    plus one exchange with the partner lane (l ^ 32).  The softmax numerator
//    P^T is then already in B-fragment layout for O^T += V^T P^T; the key
//    order inside each 16-key step is permuted identically on both operands.
//  * The logit is formed in the log2 domain with one FMA per element:
//    z = s * (sm_scale*log2e/tau_i) + (gain_h*log2e) * b_j, the key term
//    pre-multiplied per head when the tile is staged.
//  * The P.V product runs in fp16 (v_mfma_f32_32x32x16_f16): the softmax
//    numerator P lies in [0, 1], where fp16 keeps 11 significant bits against
//    bf16's 8, so rounding P costs 8x less.  V is converted once per call by
//    a prepass into V^T (key-contiguous) fp16 scaled by 2^-8: bf16 values
//    convert exactly up to |v| = 65504 * 2^8 (larger values saturate), values
//    below 2^-6 land in fp16's subnormal range with an absolute error under
//    2^-16.  The 2^8 is folded into the final 1/l.
//  * K tiles are stored row-major (bf16) and V^T tiles key-contiguous (fp16)
//    in LDS, padded rows, double-buffered through registers (each group
//    stages its own tiles: 4 tiles of 36 KiB resident per workgroup).
//  * Grid: heaviest causal query blocks first, remapped so that every
//    workgroup of one KV head lands on the same XCD (shared L2 for its K/V).
#include <math.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;  // keys per tile

constexpr int kVScaleLog2 = 8;  // V^T holds fp16(V * 2^-8)
constexpr int kBufferConfig = 0x00020000;  // raw buffer resource word 3 (gfx9 family, 32-bit data)
// The running max is only moved (and the accumulator rescaled) when a tile's
// max exceeds it by more than this many log2 units; P stays <= 2^8, well
// inside fp16.
constexpr float kRescaleSlack = 8.0f;

// max(a, b, c) as one v_max3_f32.  (The compiler's fmaxf adds a quieting
// v_max_f32 x,x,x per operand in IEEE mode; the logits here are never NaN.)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// V [B, M, Hkv, DH] bf16 -> V^T [B, Hkv, DH, Mp] fp16 (scaled, zero-padded to Mp).
template <int DH>
__global__ __launch_bounds__(kThreads) void v_to_f16t_kernel(const uint16_t* __restrict__ v, int M, int Mp, int Hkv,
                                                             uint16_t* __restrict__ vt) {
  __shared__ uint16_t sT[DH][kBK + 2];
  const int m0 = blockIdx.x * kBK, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const float scale = 1.0f / (float)(1 << kVScaleLog2);
  for (int c = tid; c < kBK * DH / 8; c += kThreads) {
    const int key = c / (DH / 8), part = c % (DH / 8);
    const int m = m0 + key;
    const u32x4 w = m < M ? load16(v + (((size_t)b * M + m) * Hkv + g) * DH + part * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // round toward zero: exact for every in-range value, saturates beyond
      const uint32_t h2 =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(w[i]) * scale, bf16_hi(w[i]) * scale));
      sT[part * 8 + 2 * i][key] = (uint16_t)(h2 & 0xFFFFu);
      sT[part * 8 + 2 * i + 1][key] = (uint16_t)(h2 >> 16);
    }
  }
  __syncthreads();
  for (int c = tid; c < DH * (kBK / 8); c += kThreads) {
    const int d = c / (kBK / 8), kc = c % (kBK / 8);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (uint32_t)sT[d][kc * 8 + 2 * i] | ((uint32_t)sT[d][kc * 8 + 2 * i + 1] << 16);
    store16(vt + (((size_t)b * Hkv + g) * DH + d) * Mp + m0 + kc * 8, o);
  }
}

constexpr int kGroups = 2;                         // wave groups splitting a key range
constexpr int kAttnThreads = kThreads * kGroups;   // 8 waves, 2 per SIMD

template <int DH, int G>
__global__ __launch_bounds__(kAttnThreads, 2) void gated_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt, int M, int Mp,
    int Hq, int Hkv, const float* __restrict__ key_score, const int32_t* __restrict__ pos,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nqb, int total_wg) {
  constexpr int RG = 4 / G;        // 32-row groups per head
  constexpr int BQ = 32 * RG;      // query rows per workgroup
  constexpr int KS = DH / 16;      // k-steps of S^T = K Q^T
  constexpr int DT = DH / 32;      // 32-row tiles of O^T
  constexpr int LDK = DH + 8;      // sK row stride (bf16)
  constexpr int LDV = kBK + 4;     // sVt row stride (fp16): 34 dwords, conflict-free 8-byte reads
  constexpr int KCH = kBK * DH / 8;          // 16-byte chunks of a K tile
  constexpr int KL = KCH / kThreads;         // per thread
  constexpr int VCH = DH * (kBK / 8);        // 16-byte chunks of a V^T tile
  constexpr int VL = VCH / kThreads;
  static_assert(KL >= 1 && VL >= 1, "tile shape");

  constexpr int NV = DT * 16 + 2;            // floats per lane handed over in the merge
  static_assert(4 * 64 * NV * 4 <= (int)sizeof(uint16_t) * 2 * kGroups * kBK * LDK, "merge buffer");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kGroups][kBK * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][kGroups][DH * LDV];
  __shared__ __attribute__((aligned(16))) float sBias[2][kGroups][G][kBK];

  const int lane = threadIdx.x & 63;
  const int wall = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: branches stay scalar
  const int grp = wall >> 2;       // key-range group of this wave
  const int wid = wall & 3;        // wave index inside the group
  const int tid = threadIdx.x & (kThreads - 1);  // thread index inside the group
  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  const int bg = logical / nqb;
  const int qb = nqb - 1 - (logical - bg * nqb);
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int q0 = qb * BQ;
  const int kv_end = min(M, q0 + BQ);
  const int nkb = (kv_end + kBK - 1) / kBK;

  const int hloc = wid / RG;
  const int hq = g * G + hloc;
  const int rbase = q0 + (wid % RG) * 32;
  const int ql = lane & 31, gq = lane >> 5;
  const int qi = rbase + ql;  // this lane's query (kept rank)
  const bool q_ok = qi < M;
  const bool wave_rows = rbase < M;

  // per-query logit scale in the log2 domain
  float cq = 0.0f;
  if (q_ok) {
    const int p = pos[(size_t)b * M + qi];
    float ratio = 1.0f;
    if (p != qi) ratio = logf((float)max(p + 1, 2)) / logf((float)max(qi + 1, 2));
    cq = sm_scale * kLog2e / (temp[hq] * ratio);
  }

  bf16x8 qf[KS];
  {
    const uint16_t* qp = q + (((size_t)b * M + (q_ok ? qi : 0)) * Hq + hq) * DH + gq * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(q_ok ? load16(qp + ks * 16) : u32x4{0, 0, 0, 0});
  }

  // ---- tile staging ----
  // Raw buffer loads: each thread's offset is fixed for the whole loop.  K and
  // the key scores get a resource per tile (base advanced to the tile, size
  // shrunk to what is left; scalar work only), so the hardware range check
  // returns 0 for keys >= M -- the check covers the per-lane offset only, not
  // a scalar offset.  V^T is padded to Mp keys and zero-filled, so its tiles
  // are always in range and share one resource with a scalar tile offset.
  const uint16_t* k_base = k + ((size_t)b * M * Hkv + g) * DH;
  const long long k_bytes = (((long long)M - 1) * Hkv + 1) * DH * 2;  // up to the end of head g's last row
  const float* b_base = key_score + (size_t)b * M;
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vt + ((size_t)b * Hkv + g) * DH * Mp), (short)0, (int)((size_t)DH * Mp * 2),
      kBufferConfig);
  int k_off[KL], v_off[VL];
#pragma unroll
  for (int e = 0; e < KL; ++e) {
    const int c = tid + kThreads * e;
    k_off[e] = ((c / (DH / 8)) * Hkv * DH + (c % (DH / 8)) * 8) * 2;
  }
#pragma unroll
  for (int e = 0; e < VL; ++e) {
    const int c = tid + kThreads * e;
    v_off[e] = ((c / (kBK / 8)) * Mp + (c % (kBK / 8)) * 8) * 2;
  }
  const int b_off = (tid % kBK) * 4;
  u32x4 rk[KL], rv[VL];
  float rb = 0.0f;
  auto load_tile = [&](int kb) {
    const int key0 = kb * kBK;
    const long long k_skip = (long long)key0 * Hkv * DH * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(k_base + (size_t)key0 * Hkv * DH), (short)0, (int)(k_bytes - k_skip), kBufferConfig);
#pragma unroll
    for (int e = 0; e < KL; ++e)
      rk[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_off[e], 0, 0));
#pragma unroll
    for (int e = 0; e < VL; ++e)
      rv[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, v_off[e], key0 * 2, 0));
    if (tid < G * kBK) {
      const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(b_base + key0), (short)0, (M - key0) * 4, kBufferConfig);
      rb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(b_rsrc, b_off, 0, 0));
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      const int c = tid + kThreads * e;
      const int key = c / (DH / 8), part = c % (DH / 8);
      store16(&sK[buf][grp][key * LDK + part * 8], rk[e]);
    }
#pragma unroll
    for (int e = 0; e < VL; ++e) {
      const int c = tid + kThreads * e;
      const int d = c / (kBK / 8), kc = c % (kBK / 8);
      u32x2* dst = reinterpret_cast<u32x2*>(&sVt[buf][grp][d * LDV + kc * 8]);
      dst[0] = u32x2{rv[e][0], rv[e][1]};
      dst[1] = u32x2{rv[e][2], rv[e][3]};
    }
    if (tid < G * kBK) {
      const int hh = tid / kBK;
      sBias[buf][grp][hh][tid % kBK] = rb * (gain[g * G + hh] * kLog2e);
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // One 64-key tile for this wave's 32 queries.  `diag` (wave-uniform): the
  // tile reaches past the wave's first query (diagonal or ragged tail), so
  // keys after the query are masked; every other tile skips that block.
  auto tile = [&](int buf, int key0, bool diag) {
    // S^T = K Q^T for the two 32-key halves, the two accumulation chains
    // interleaved so consecutive MFMAs are independent
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.0f;
      s1[i] = 0.0f;
    }
    const uint16_t* kr0 = &sK[buf][grp][ql * LDK + gq * 8];
    const uint16_t* kr1 = kr0 + 32 * LDK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kr0 + ks * 16);
      const bf16x8 kc = *reinterpret_cast<const bf16x8*>(kr1 + ks * 16);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc, qf[ks], s1, 0, 0, 0);
    }
    // logits (log2 domain); lane holds keys 32T + 8(i/4) + 4gq + (i%4)
    auto logits = [&](f32x16& st, int T) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 bb = *reinterpret_cast<const f32x4*>(&sBias[buf][grp][hloc][T * 32 + i4 * 8 + gq * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i4 * 4 + i] = fmaf(st[i4 * 4 + i], cq, bb[i]);
      }
    };
    logits(s0, 0);
    logits(s1, 1);
    if (diag) {
      // key offset inside the tile (minus this lane's 4*gq) beyond thr => masked
      const int thr = qi - key0 - gq * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = (i >> 2) * 8 + (i & 3);
        s0[i] = off > thr ? -INFINITY : s0[i];
        s1[i] = off + 32 > thr ? -INFINITY : s1[i];
      }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mloc = max3f(mloc, s0[i], s1[i]);
    mloc = pair_max(mloc);
    if (__ballot(mloc > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    }
    // (a lane with no visible key yet keeps m_run = -inf; its logits are all
    // -inf too, and a finite reference keeps exp2 at 0 instead of NaN)
    const float mref = m_run == -INFINITY ? 0.0f : m_run;
    // numerators (rounded to fp16 for the P.V product) and their fp32 row sum
    uint32_t pk[2][8];
    float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s0[i] - mref), p1 = __builtin_amdgcn_exp2f(s0[i + 1] - mref);
      const float p2 = __builtin_amdgcn_exp2f(s1[i] - mref), p3 = __builtin_amdgcn_exp2f(s1[i + 1] - mref);
      l0 += p0 + p1;
      l1 += p2 + p3;
      pk[0][i / 2] = pack_f16x2(p0, p1);
      pk[1][i / 2] = pack_f16x2(p2, p3);
    }
    l_run += l0 + l1;
    // O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int T = st >> 1, h8 = (st & 1) * 4;
      const u32x4 pw = {pk[T][h8], pk[T][h8 + 1], pk[T][h8 + 2], pk[T][h8 + 3]};
      const f16x8 pf = as_f16x8(pw);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint16_t* vr = &sVt[buf][grp][(t * 32 + ql) * LDV + st * 16 + gq * 4];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
        const u32x4 vw = {lo[0], lo[1], hi[0], hi[1]};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vw), pf, o[t], 0, 0, 0);
      }
    }
  };

  // group grp owns tiles grp, grp + 2, ...; both groups meet at every barrier
  const int nit = (nkb + kGroups - 1) / kGroups;
  if (grp < nkb) {
    load_tile(grp);
    store_tile(0);
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int buf = it & 1;
    const int kb = it * kGroups + grp;
    const bool more = kb + kGroups < nkb;
    if (more) load_tile(kb + kGroups);
    const int key0 = kb * kBK;
    if (kb < nkb && wave_rows && key0 <= rbase + 31) tile(buf, key0, key0 + kBK - 1 > rbase);  // wave-uniform
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // merge the two groups' online-softmax states (the tile buffers are free now)
  float* sm = reinterpret_cast<float*>(&sK[0][0][0]);
  const int slot = wid * 64 + lane;
  if (grp == 1) {
    sm[slot] = m_run;
    sm[256 + slot] = l_run;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) sm[(2 + t * 16 + i) * 256 + slot] = o[t][i];
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const float m1 = sm[slot], l1 = sm[256 + slot];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    m_run = m;
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] = o[t][i] * a0 + sm[(2 + t * 16 + i) * 256 + slot] * a1;
  }

  if (!wave_rows) return;
  const float l_tot = pair_sum(l_run);
  if (!q_ok) return;
  const float inv = (float)(1 << kVScaleLog2) / l_tot;
  uint16_t* op = out + (((size_t)b * M + qi) * Hq + hq) * DH;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = t * 32 + i4 * 8 + gq * 4;
      u32x2 w;
      w[0] = pack_bf16x2(o[t][i4 * 4 + 0] * inv, o[t][i4 * 4 + 1] * inv);
      w[1] = pack_bf16x2(o[t][i4 * 4 + 2] * inv, o[t][i4 * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + d0) = w;
    }
  }
  if (lse != nullptr && gq == 0) lse[((size_t)b * Hq + hq) * M + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int DH, int G>
hipError_t launch_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq, int Hkv,
                    const float* ks, const int32_t* pos, const float* gain, const float* temp, float sm_scale,
                    uint16_t* out, float* lse, uint16_t* vt, hipStream_t s) {
  constexpr int BQ = 32 * (4 / G);
  const int Mp = (M + kBK - 1) / kBK * kBK;
  hipLaunchKernelGGL((v_to_f16t_kernel<DH>), dim3(Mp / kBK, Hkv, B), dim3(kThreads), 0, s, v, M, Mp, Hkv, vt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (M + BQ - 1) / BQ;
  const long long total = (long long)nqb * Hkv * B;
  if (total <= 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gated_attn_kernel<DH, G>), dim3((unsigned)total), dim3(kAttnThreads), 0, s, q, k, vt, M, Mp, Hq,
                     Hkv, ks, pos, gain, temp, sm_scale, out, lse, nqb, (int)total);
  return hipGetLastError();
}

}  // namespace

size_t gated_attention_workspace(int B, int M, int Hkv, int dh) {
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  return (size_t)B * Hkv * dh * Mp * 2;
}

hipError_t launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq,
                                  int Hkv, int dh, const float* key_score, const int32_t* pos, const float* gain,
                                  const float* temp, float sm_scale, uint16_t* out, float* lse, void* ws,
                                  hipStream_t s) {
  const int G = Hq / Hkv;
  uint16_t* vt = static_cast<uint16_t*>(ws);
#define TG_ATTN_CASE(DHV, GV)                                                                                \
  if (dh == DHV && G == GV)                                                                                  \
    return launch_t<DHV, GV>(q, k, v, B, M, Hq, Hkv, key_score, pos, gain, temp, sm_scale, out, lse, vt, s);
  TG_ATTN_CASE(128, 2)
  TG_ATTN_CASE(128, 1)
  TG_ATTN_CASE(128, 4)
  TG_ATTN_CASE(64, 2)
  TG_ATTN_CASE(64, 1)
  TG_ATTN_CASE(64, 4)
#undef TG_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace tg
