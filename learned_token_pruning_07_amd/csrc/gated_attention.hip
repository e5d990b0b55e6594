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
//    pre-multiplied per head by the prepass.
//  * The P.V product runs in fp16 (v_mfma_f32_32x32x16_f16): the softmax
//    numerator P lies in [0, 1], where fp16 keeps 11 significant bits against
//    bf16's 8, so rounding P costs 8x less.  V is converted once per call by
//    a prepass into V^T (key-contiguous) fp16 scaled by 2^-8: bf16 values
//    convert exactly up to |v| = 65504 * 2^8 (larger values saturate), values
//    below 2^-6 land in fp16's subnormal range with an absolute error under
//    2^-16.  The 2^8 is folded into the final 1/l.  Inside every 16-key group
//    of V^T the middle two quads of keys are swapped, so that the 8 keys one
//    lane contributes to a 16-key P.V step (4 at 4*gq, 4 at 8 + 4*gq) form
//    one 16-byte chunk.
//  * Tiles travel from global memory straight into LDS (buffer loads with the
//    LDS-destination bit: each lane's 16 bytes land at the wave's LDS base +
//    16 * lane), double-buffered per group, so staging costs no registers and
//    no LDS store instructions.  K rows (bf16) and V^T rows (fp16, 64 keys)
//    are unpadded with their 16-byte chunks XOR-swizzled by (row & 7), which
//    keeps the fragment reads free of bank conflicts; the lane-to-chunk map of
//    each load applies the same swizzle.  The prepass also writes the
//    key-score term of every query head, gain_h * log2(e) * b_j, so that tile
//    too is a plain copy.
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

// Key stored in slot s of a V^T tile row: the middle two quads of each
// 16-key group are swapped.
__device__ __forceinline__ int vt_slot_key(int s) {
  const int q = (s >> 2) & 3;
  const int kq = q == 1 ? 2 : (q == 2 ? 1 : q);
  return (s & ~15) | (kq << 2) | (s & 3);
}

// Prepass, per 64-key block of KV head g:
//   V [B, M, Hkv, DH] bf16 -> V^T [B, Hkv, DH, Mp] fp16 (scaled by 2^-8, keys
//   in slot order, zero beyond M);
//   key-score term kb [B, Hq, Mp] fp32 = gain_h * log2(e) * key_score for the
//   G query heads of g (zero beyond M).
template <int DH>
__global__ __launch_bounds__(kThreads) void attn_prepass_kernel(const uint16_t* __restrict__ v,
                                                                const float* __restrict__ key_score,
                                                                const float* __restrict__ gain, int M, int Mp,
                                                                int Hkv, int G, uint16_t* __restrict__ vt,
                                                                float* __restrict__ kbias) {
  __shared__ uint16_t sT[DH][kBK + 2];
  const int m0 = blockIdx.x * kBK, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const float scale = 1.0f / (float)(1 << kVScaleLog2);
  constexpr int NL = kBK * DH / 8 / kThreads;  // 16-byte loads per thread, all issued before any use
  u32x4 w[NL];
#pragma unroll
  for (int e = 0; e < NL; ++e) {
    const int c = tid + e * kThreads;
    const int key = c / (DH / 8), part = c % (DH / 8);
    const int m = m0 + key;
    w[e] = m < M ? load16(v + (((size_t)b * M + m) * Hkv + g) * DH + part * 8) : u32x4{0, 0, 0, 0};
  }
  const int Hq = Hkv * G;
  for (int c = tid; c < G * kBK; c += kThreads) {
    const int hq = g * G + c / kBK, m = m0 + c % kBK;
    kbias[((size_t)b * Hq + hq) * Mp + m] = m < M ? key_score[(size_t)b * M + m] * (gain[hq] * kLog2e) : 0.0f;
  }
#pragma unroll
  for (int e = 0; e < NL; ++e) {
    const int c = tid + e * kThreads;
    const int key = c / (DH / 8), part = c % (DH / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // round toward zero: exact for every in-range value, saturates beyond
      const uint32_t h2 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(w[e][i]) * scale, bf16_hi(w[e][i]) * scale));
      sT[part * 8 + 2 * i][key] = (uint16_t)(h2 & 0xFFFFu);
      sT[part * 8 + 2 * i + 1][key] = (uint16_t)(h2 >> 16);
    }
  }
  __syncthreads();
  for (int c = tid; c < DH * (kBK / 8); c += kThreads) {
    const int d = c / (kBK / 8), kc = c % (kBK / 8);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)sT[d][vt_slot_key(kc * 8 + 2 * i)] | ((uint32_t)sT[d][vt_slot_key(kc * 8 + 2 * i + 1)] << 16);
    store16(vt + (((size_t)b * Hkv + g) * DH + d) * Mp + m0 + kc * 8, o);
  }
}

constexpr int kGroups = 2;                         // wave groups splitting a key range
constexpr int kAttnThreads = kThreads * kGroups;   // 8 waves, 2 per SIMD

// Raw buffer loads of 16 or 4 bytes per lane into LDS: lane l's data lands at
// lds + 16 l (or 4 l); lds is wave-uniform.  Completion is tracked by vmcnt.
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset,
                                                     int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset,
                                           0, 0);
}
__device__ __forceinline__ void buffer_load4_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 4, voffset, soffset, 0,
                                           0);
}
// s_waitcnt vmcnt(0): wait for every load of this wave, LDS-destination ones included
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DH, int G>
__global__ __launch_bounds__(kAttnThreads, 2) void gated_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const float* __restrict__ kbias, int M, int Mp, int Hq, int Hkv, const int32_t* __restrict__ pos,
    const float* __restrict__ temp, float sm_scale, uint16_t* __restrict__ out, float* __restrict__ lse, int nqb,
    int total_wg) {
  constexpr int RG = 4 / G;        // 32-row groups per head
  constexpr int BQ = 32 * RG;      // query rows per workgroup
  constexpr int KS = DH / 16;      // k-steps of S^T = K Q^T
  constexpr int DT = DH / 32;      // 32-row tiles of O^T
  constexpr int KROW = DH * 2;      // bytes of a K row in LDS (unpadded, swizzled)
  constexpr int KCH = DH / 8;       // its 16-byte chunks
  constexpr int VROW = kBK * 2;     // bytes of a V^T row (64 keys, fp16)
  constexpr int TILE = kBK * DH * 2;           // bytes of a K tile = bytes of a V^T tile
  constexpr int NI = TILE / 1024 / 4;          // 1 KiB loads per wave per tile, for each of K and V^T
  constexpr int BIAS = G * kBK * 4;            // bytes of a key-score tile (G heads)
  constexpr int V_BASE = 2 * kGroups * TILE, B_BASE = 4 * kGroups * TILE;
  constexpr int LDS_BYTES = B_BASE + 2 * kGroups * BIAS;
  static_assert(NI >= 1 && NI * 4 * 1024 == TILE, "tile shape");

  constexpr int NV = DT * 16 + 2;            // floats per lane handed over in the merge
  static_assert(4 * 64 * NV * 4 <= B_BASE, "merge buffer");

  // [buf][group] K tiles, then [buf][group] V^T tiles, then [buf][group][head] key-score tiles
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

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

  // ---- tile staging ----
  // Raw buffer loads with an LDS destination; each lane's byte offset is fixed
  // for the whole loop.  K gets a resource per tile (base advanced to the
  // tile, size shrunk to what is left; scalar work only), so the hardware
  // range check returns 0 for keys >= M -- the check covers the per-lane
  // offset only, not a scalar offset.  V^T and the key-score rows are padded
  // to Mp keys, so their tiles are always in range and take a scalar offset.
  const uint16_t* k_base = k + ((size_t)b * M * Hkv + g) * DH;
  const long long k_bytes = (((long long)M - 1) * Hkv + 1) * DH * 2;  // up to the end of head g's last row
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vt + ((size_t)b * Hkv + g) * DH * Mp), (short)0, (int)((size_t)DH * Mp * 2),
      kBufferConfig);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(kbias + ((size_t)b * Hq + g * G) * Mp), (short)0, G * Mp * 4, kBufferConfig);
  // Load e of this wave fills LDS bytes [1024 C, 1024 C + 1024) of the tile,
  // C = wid * NI + e: 16-byte slot Y = 64 C + lane sits at row Y / chunks-per-row,
  // position p, and holds chunk p ^ (row & 7) of that row.
  int k_off[NI], v_off[NI];
#pragma unroll
  for (int e = 0; e < NI; ++e) {
    const int Y = (wid * NI + e) * 64 + lane;
    const int kr = Y / KCH, kc = (Y % KCH) ^ (kr & 7);
    k_off[e] = kr * Hkv * DH * 2 + kc * 16;
    const int vr = Y / (VROW / 16), vc = (Y % (VROW / 16)) ^ (vr & 7);
    v_off[e] = vr * Mp * 2 + vc * 16;
  }
  auto k_tile = [&](int buf) { return smem + (buf * kGroups + grp) * TILE; };
  auto v_tile = [&](int buf) { return smem + V_BASE + (buf * kGroups + grp) * TILE; };
  auto b_tile = [&](int buf) { return reinterpret_cast<float*>(smem + B_BASE + (buf * kGroups + grp) * BIAS); };
  auto issue_tile = [&](int kb, int buf) {
    const int key0 = kb * kBK;
    const long long k_skip = (long long)key0 * Hkv * DH * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(k_base + (size_t)key0 * Hkv * DH), (short)0, (int)(k_bytes - k_skip), kBufferConfig);
    unsigned char* kd = k_tile(buf) + wid * NI * 1024;
    unsigned char* vd = v_tile(buf) + wid * NI * 1024;
#pragma unroll
    for (int e = 0; e < NI; ++e)
      buffer_load16_to_lds(k_rsrc, kd + e * 1024, k_off[e], 0);
#pragma unroll
    for (int e = 0; e < NI; ++e)
      buffer_load16_to_lds(v_rsrc, vd + e * 1024, v_off[e], key0 * 2);
    if (wid < G)  // one 256-byte row per query head
      buffer_load4_to_lds(b_rsrc, b_tile(buf) + wid * kBK, (wid * Mp + lane) * 4, key0 * 4);
  };
  // this lane's fragment chunks: K row ql (and ql + 32) chunk 2ks + gq; V^T row
  // 32t + ql chunk 2st + gq -- both swizzled by ql & 7
  const int q7 = ql & 7;
  auto k_frag_off = [&](int ks) { return ql * KROW + (((2 * ks + gq) ^ q7) << 4); };
  auto v_frag_off = [&](int st) { return ql * VROW + (((2 * st + gq) ^ q7) << 4); };

  bf16x8 qf[KS];      // this lane's Q fragments (filled in the prologue below)
  float cq = 0.0f;    // per-query logit scale in the log2 domain
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
    const unsigned char* kt = k_tile(buf);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + k_frag_off(ks));
      const bf16x8 kc = *reinterpret_cast<const bf16x8*>(kt + k_frag_off(ks) + 32 * KROW);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc, qf[ks], s1, 0, 0, 0);
    }
    // logits (log2 domain); lane holds keys 32T + 8(i/4) + 4gq + (i%4)
    auto logits = [&](f32x16& st, int T) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 bb = *reinterpret_cast<const f32x4*>(b_tile(buf) + hloc * kBK + T * 32 + i4 * 8 + gq * 4);
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
    // tile max: a max3 tree over the 32 logits, then the partner lane's
    float x[11];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      x[2 * j] = max3f(s0[3 * j], s0[3 * j + 1], s0[3 * j + 2]);
      x[2 * j + 1] = max3f(s1[3 * j], s1[3 * j + 1], s1[3 * j + 2]);
    }
    x[10] = max3f(s0[15], s1[15], s1[15]);
    float mloc = max3f(max3f(x[0], x[1], x[2]), max3f(x[3], x[4], x[5]), max3f(x[6], x[7], max3f(x[8], x[9], x[10])));
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
      mloc = max3f(__uint_as_float(pr[0]), __uint_as_float(pr[1]), __uint_as_float(pr[1]));
    }
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
        const u32x4 vw = *reinterpret_cast<const u32x4*>(v_tile(buf) + t * 32 * VROW + v_frag_off(st));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vw), pf, o[t], 0, 0, 0);
      }
    }
  };

  // group grp owns tiles grp, grp + 2, ...; both groups meet at every barrier
  // (a buffer is refilled only after the barrier that ends its last use, and
  // read only after the barrier that follows its loads' completion)
  const int nit = (nkb + kGroups - 1) / kGroups;
  if (grp < nkb) issue_tile(grp, 0);
  // Q fragments and the original position are requested while the first
  // tile is in flight; one wait covers all of them
  {
    const uint16_t* qp = q + (((size_t)b * M + (q_ok ? qi : 0)) * Hq + hq) * DH + gq * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(q_ok ? load16(qp + ks * 16) : u32x4{0, 0, 0, 0});
  }
  const int p_orig = pos[(size_t)b * M + (q_ok ? qi : 0)];
  const float t_h = temp[hq];
  wait_vmem();
  if (q_ok) {
    float ratio = 1.0f;
    if (p_orig != qi) ratio = logf((float)max(p_orig + 1, 2)) / logf((float)max(qi + 1, 2));
    cq = sm_scale * kLog2e / (t_h * ratio);
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int buf = it & 1;
    const int kb = it * kGroups + grp;
    if (kb + kGroups < nkb) issue_tile(kb + kGroups, buf ^ 1);
    const int key0 = kb * kBK;
    if (kb < nkb && wave_rows && key0 <= rbase + 31) tile(buf, key0, key0 + kBK - 1 > rbase);  // wave-uniform
    wait_vmem();
    __syncthreads();
  }

  // merge the two groups' online-softmax states (the tile buffers are free
  // now): group 1 hands over m, l and O as 16-byte vectors per lane
  f32x4* sm4 = reinterpret_cast<f32x4*>(smem);
  const int slot = wid * 64 + lane;
  if (grp == 1) {
    sm4[slot] = f32x4{m_run, l_run, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        sm4[(1 + t * 4 + i4) * 256 + slot] =
            f32x4{o[t][i4 * 4], o[t][i4 * 4 + 1], o[t][i4 * 4 + 2], o[t][i4 * 4 + 3]};
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const f32x4 ml = sm4[slot];
    const float m1 = ml[0], l1 = ml[1];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    m_run = m;
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 o1 = sm4[(1 + t * 4 + i4) * 256 + slot];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i4 * 4 + i] = o[t][i4 * 4 + i] * a0 + o1[i] * a1;
      }
  }

  if (!wave_rows) return;
  const float l_tot = pair_sum(l_run);
  const float inv = (float)(1 << kVScaleLog2) / l_tot;
  // Output rows leave through LDS so that each store writes whole 16-byte
  // pieces of a row: the wave's 32 x DH bf16 block is written row-major with
  // the 16-byte chunks of row r XOR-swizzled by r & 15, then read back 16
  // bytes per lane.  The region lies past the merge vectors and belongs to
  // this wave alone, and LDS operations of one wave complete in order.
  constexpr int OROW = DH * 2;  // bytes of an output row
  unsigned char* ob = smem + (1 + DT * 4) * 256 * 16 + wid * 32 * OROW;
  static_assert((1 + DT * 4) * 256 * 16 + 4 * 32 * OROW <= LDS_BYTES, "output staging");
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      // d = 32t + 8 i4 + 4gq + (0..3): chunk 4t + i4 of the row, half gq
      u32x2 w;
      w[0] = pack_bf16x2(o[t][i4 * 4 + 0] * inv, o[t][i4 * 4 + 1] * inv);
      w[1] = pack_bf16x2(o[t][i4 * 4 + 2] * inv, o[t][i4 * 4 + 3] * inv);
      const int chunk = (t * 4 + i4) ^ (ql & (KCH - 1));
      *reinterpret_cast<u32x2*>(ob + ql * OROW + chunk * 16 + gq * 8) = w;
    }
  constexpr int RPI = 64 / KCH;  // rows per 64-lane store
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + lane / KCH, c = lane % KCH;
    const u32x4 w = *reinterpret_cast<const u32x4*>(ob + r * OROW + ((c ^ (r & (KCH - 1))) * 16));
    if (rbase + r < M) store16(out + (((size_t)b * M + rbase + r) * Hq + hq) * DH + c * 8, w);
  }
  if (lse != nullptr && gq == 0 && q_ok) lse[((size_t)b * Hq + hq) * M + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int DH, int G>
hipError_t launch_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq, int Hkv,
                    const float* ks, const int32_t* pos, const float* gain, const float* temp, float sm_scale,
                    uint16_t* out, float* lse, uint16_t* vt, float* kbias, hipStream_t s) {
  constexpr int BQ = 32 * (4 / G);
  const int Mp = (M + kBK - 1) / kBK * kBK;
  hipLaunchKernelGGL((attn_prepass_kernel<DH>), dim3(Mp / kBK, Hkv, B), dim3(kThreads), 0, s, v, ks, gain, M, Mp,
                     Hkv, G, vt, kbias);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (M + BQ - 1) / BQ;
  const long long total = (long long)nqb * Hkv * B;
  if (total <= 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gated_attn_kernel<DH, G>), dim3((unsigned)total), dim3(kAttnThreads), 0, s, q, k, vt, kbias, M,
                     Mp, Hq, Hkv, pos, temp, sm_scale, out, lse, nqb, (int)total);
  return hipGetLastError();
}

}  // namespace

// fp16 V^T [B, Hkv, dh, Mp], then the fp32 key-score terms [B, Hq, Mp]
size_t gated_attention_workspace(int B, int M, int Hq, int Hkv, int dh) {
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  return (size_t)B * Mp * ((size_t)Hkv * dh * 2 + (size_t)Hq * 4);
}

hipError_t launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq,
                                  int Hkv, int dh, const float* key_score, const int32_t* pos, const float* gain,
                                  const float* temp, float sm_scale, uint16_t* out, float* lse, void* ws,
                                  hipStream_t s) {
  const int G = Hq / Hkv;
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  uint16_t* vt = static_cast<uint16_t*>(ws);
  float* kbias = reinterpret_cast<float*>(vt + (size_t)B * Hkv * dh * Mp);
#define TG_ATTN_CASE(DHV, GV)                                                                                   \
  if (dh == DHV && G == GV)                                                                                     \
    return launch_t<DHV, GV>(q, k, v, B, M, Hq, Hkv, key_score, pos, gain, temp, sm_scale, out, lse, vt, kbias, \
                             s);
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
