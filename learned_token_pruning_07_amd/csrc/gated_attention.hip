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
//    16 keys of a 32-key half tile, so the row max/sum is an in-lane
//    reduction plus one exchange with the partner lane (l ^ 32).  The softmax
//    numerator P^T is then already in B-fragment layout for O^T += V^T P^T;
//    the key order inside each 16-key step is permuted identically on both
//    operands.
//  * Software pipeline over 32-key half tiles: step h issues the score MFMAs
//    of half h + 1 and the P.V MFMAs of half h - 1 while the vector ALUs run
//    the softmax of half h, so the matrix cores never wait for the wave's own
//    softmax.  In steady state the step is a fixed issue order (scheduling
//    fences): every slot holds one MFMA, the LDS read of the fragment three
//    slots ahead and a share of the softmax.
//  * Steady-state scores are relative to the running max m: the score
//    accumulator starts from -m / (scale of the query) instead of 0, so the
//    logit FMA yields z - m and feeds exp2 directly.  The max is not
//    recomputed every half: a half whose row sum exceeds 2^15 (a numerator
//    that may leave fp16's range) takes a rare path that moves m to the
//    row's true max and redoes that half.
//  * The P.V product runs in fp16 (v_mfma_f32_32x32x16_f16): the softmax
//    numerator P lies in [0, 2^15], where fp16 keeps 11 significant bits
//    against bf16's 8, so rounding P costs 8x less.  V is converted once per
//    call by a prepass into V^T (key-contiguous) fp16 scaled by 2^-8: bf16
//    values convert exactly up to |v| = 65504 * 2^8 (larger values saturate),
//    values below 2^-6 land in fp16's subnormal range with an absolute error
//    under 2^-16.  The 2^8 is folded into the final 1/l.  Inside every 16-key
//    group of V^T the middle two quads of keys are swapped, so that the 8
//    keys one lane contributes to a 16-key P.V step (4 at 4*gq, 4 at
//    8 + 4*gq) form one 16-byte chunk.
//  * Tiles travel from global memory straight into LDS (buffer loads with the
//    LDS-destination bit: each lane's 16 bytes land at the wave's LDS base +
//    16 * lane), so staging costs no registers and no LDS store
//    instructions.  Every load is issued one iteration before the first
//    iteration that reads it; K and V^T tiles are read within one iteration
//    (two-slot rings per group), key scores across two (three-slot ring).
//    K rows (bf16) and V^T rows (fp16, 64 keys) are unpadded with their
//    16-byte chunks XOR-swizzled by (row & 7), which keeps the fragment reads
//    free of bank conflicts; the lane-to-chunk map of each load applies the
//    same swizzle.  The prepass also writes the key-score term of every query
//    head, gain_h * log2(e) * b_j, so that tile too is a plain copy.
//  * Grid: heaviest causal query blocks first, remapped so that every
//    workgroup of one KV head lands on the same XCD (shared L2 for its K/V).
#include <math.h>

#include <algorithm>
#include <vector>

#include "rope_device.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;  // keys per tile

constexpr int kVScaleLog2 = 8;  // V^T holds fp16(V * 2^-8)
constexpr int kBufferConfig = 0x00020000;  // raw buffer resource word 3 (gfx9 family, 32-bit data)
// Outside the steady state the running max is only moved (and the
// accumulator rescaled) when a half tile's max exceeds it by more than this
// many log2 units; P stays <= 2^8 there.
constexpr float kRescaleSlack = 8.0f;

template <int V>
struct IntConst {
  static constexpr int value = V;
};

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

// Rotary position embedding inputs of the prepass: q, k and the positions,
// the base, and where the rotated copies go (same layouts as q and k).
struct RopeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* pos;
  double base;
  uint16_t* qr;
  uint16_t* kr;
};

// Sequences of one varying-length launch, longest first.  Sequence s owns
// packed rows t0[s] .. t0[s] + m[s] - 1 of q, k, v, out, key_score and pos,
// padded key slots p0[s] .. p0[s] + roundup(m[s], 64) - 1 of V^T and the
// key-score terms, prepass blocks pb0[s] .. pb0[s+1] - 1 and attention
// workgroups wg0[s] .. wg0[s+1] - 1 (before the XCD remap).  Passed by value:
// the kernel reads it from its argument segment.
constexpr int kMaxSeqsPerLaunch = 64;
struct SeqTable {
  int n;
  int t0[kMaxSeqsPerLaunch];
  int m[kMaxSeqsPerLaunch];
  int p0[kMaxSeqsPerLaunch];
  int pb0[kMaxSeqsPerLaunch + 1];
  int wg0[kMaxSeqsPerLaunch + 1];
};

// Prepass, per 64-key block of KV head g:
//   V [B, M, Hkv, DH] bf16 -> V^T [B, Hkv, DH, Mp] fp16 (scaled by 2^-8, keys
//   in slot order, zero beyond M);
//   key-score term kb [B, Hq, Mp] fp32 = gain_h * log2(e) * key_score for the
//   G query heads of g (zero beyond M);
//   with ROPE, also the rotary embedding of the block's K rows (head g) and Q
//   rows (the G query heads of g) at their original positions (the rotate-
//   half form: pair (x_i, x_{i+DH/2}) turns by pos * base^(-2i/DH)).  The
//   angle is formed and reduced modulo 2 pi in fp64, so that its fp32 sine
//   and cosine are accurate to a few ulp at any position.
// VARLEN: the blocks of the table's sequences, one grid row per KV head.
template <int DH, bool ROPE, bool VARLEN>
__global__ __launch_bounds__(kThreads) void attn_prepass_kernel(const uint16_t* __restrict__ v,
                                                                const float* __restrict__ key_score,
                                                                const float* __restrict__ gain, int M_all,
                                                                int Mp_all, int Hkv, int G,
                                                                uint16_t* __restrict__ vt,
                                                                float* __restrict__ kbias, RopeArgs ra,
                                                                const SeqTable st) {
  __shared__ uint16_t sT[DH][kBK + 2];
  __shared__ double s_freq[DH / 2];
  const int g = blockIdx.y;
  int m0, M, Mp;
  size_t T0, P0;  // first packed row and first padded key slot of this sequence
  if constexpr (VARLEN) {
    const int sq = seq_of(st.pb0, st.n, blockIdx.x);
    M = st.m[sq];
    Mp = (M + kBK - 1) / kBK * kBK;
    m0 = (blockIdx.x - st.pb0[sq]) * kBK;
    T0 = (size_t)st.t0[sq];
    P0 = (size_t)st.p0[sq];
  } else {
    M = M_all;
    Mp = Mp_all;
    m0 = blockIdx.x * kBK;
    T0 = (size_t)blockIdx.z * M;
    P0 = (size_t)blockIdx.z * Mp;
  }
  const int tid = threadIdx.x;
  if (ROPE && tid < DH / 2) s_freq[tid] = rope::inv_freq(ra.base, tid, DH);  // (ordered by the barrier below)
  const float scale = 1.0f / (float)(1 << kVScaleLog2);
  constexpr int NL = kBK * DH / 8 / kThreads;  // 16-byte loads per thread, all issued before any use
  u32x4 w[NL];
#pragma unroll
  for (int e = 0; e < NL; ++e) {
    const int c = tid + e * kThreads;
    const int key = c / (DH / 8), part = c % (DH / 8);
    const int m = m0 + key;
    w[e] = m < M ? load16(v + ((T0 + m) * Hkv + g) * DH + part * 8) : u32x4{0, 0, 0, 0};
  }
  const int Hq = Hkv * G;
  for (int c = tid; c < G * kBK; c += kThreads) {
    const int hq = g * G + c / kBK, m = m0 + c % kBK;
    kbias[P0 * Hq + (size_t)hq * Mp + m] = m < M ? key_score[T0 + m] * (gain[hq] * kLog2e) : 0.0f;
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
    store16(vt + P0 * Hkv * DH + ((size_t)g * DH + d) * Mp + m0 + kc * 8, o);
  }
  if constexpr (ROPE) {
    constexpr int PG = DH / 2 / 8;  // groups of 8 pairs per head row
    const int Hq = Hkv * G;
    for (int t = tid; t < kBK * PG; t += kThreads) {
      const int key = t / PG, i0 = (t % PG) * 8, m = m0 + key;
      if (m >= M) continue;
      float c[8], sn[8];
      rope::sincos8((double)ra.pos[T0 + m], s_freq, i0, c, sn);
      const size_t krow = ((T0 + m) * Hkv + g) * DH;
      rope::row8<DH>(ra.k + krow, ra.kr + krow, i0, c, sn);
      for (int hh = 0; hh < G; ++hh) {
        const size_t qrow = ((T0 + m) * Hq + g * G + hh) * DH;
        rope::row8<DH>(ra.q + qrow, ra.qr + qrow, i0, c, sn);
      }
    }
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

template <int DH, int G, bool VARLEN>
__global__ __launch_bounds__(kAttnThreads, 1) void gated_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const float* __restrict__ kbias, int M_all, int Mp_all, int Hq, int Hkv, const int32_t* __restrict__ pos,
    const float* __restrict__ temp, float sm_scale, uint16_t* __restrict__ out, float* __restrict__ lse, int nqb_all,
    int total_wg, const SeqTable st) {
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
  constexpr int LDS_BYTES = B_BASE + 3 * kGroups * BIAS;
  static_assert(NI >= 1 && NI * 4 * 1024 == TILE, "tile shape");


  // [buf][group] K tiles, then [buf][group] V^T tiles, then [buf][group][head] key-score tiles
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wall = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: branches stay scalar
  const int grp = wall >> 2;       // key-range group of this wave
  const int wid = wall & 3;        // wave index inside the group
  const int tid = threadIdx.x & (kThreads - 1);  // thread index inside the group
  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  // this workgroup's sequence (its length M, first packed row T0, first
  // padded key slot P0), KV head g and query block qb (the longest first)
  int M, Mp, g, qb;
  size_t T0, P0;
  if constexpr (VARLEN) {
    const int sq = seq_of(st.wg0, st.n, logical);
    M = st.m[sq];
    Mp = (M + kBK - 1) / kBK * kBK;
    const int nqb = (M + BQ - 1) / BQ, local = logical - st.wg0[sq];
    g = local / nqb;
    qb = nqb - 1 - (local - g * nqb);
    T0 = (size_t)st.t0[sq];
    P0 = (size_t)st.p0[sq];
  } else {
    M = M_all;
    Mp = Mp_all;
    const int bg = logical / nqb_all;
    qb = nqb_all - 1 - (logical - bg * nqb_all);
    const int b = bg / Hkv;
    g = bg - b * Hkv;
    T0 = (size_t)b * M;
    P0 = (size_t)b * Mp;
  }
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
  const uint16_t* k_base = k + (T0 * Hkv + g) * DH;
  const long long k_bytes = (((long long)M - 1) * Hkv + 1) * DH * 2;  // up to the end of head g's last row
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vt + P0 * Hkv * DH + (size_t)g * DH * Mp), (short)0, (int)((size_t)DH * Mp * 2),
      kBufferConfig);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(kbias + P0 * Hq + (size_t)g * G * Mp), (short)0, G * Mp * 4, kBufferConfig);
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
  // Group tile t is key tile grp + 2 t.  Its K rows, V^T rows and key-score
  // rows are requested at different iterations (see the loop below): K and
  // V^T into two-slot rings (slot t & 1), key scores into a three-slot ring
  // (slot t % 3).
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    const int key0 = (grp + kGroups * t) * kBK;
    const long long k_skip = (long long)key0 * Hkv * DH * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(k_base + (size_t)key0 * Hkv * DH), (short)0, (int)(k_bytes - k_skip), kBufferConfig);
    unsigned char* kd = k_tile(t & 1) + wid * NI * 1024;
#pragma unroll
    for (int e = 0; e < NI; ++e) buffer_load16_to_lds(k_rsrc, kd + e * 1024, k_off[e], 0);
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) {
    unsigned char* vd = v_tile(t & 1) + wid * NI * 1024;
#pragma unroll
    for (int e = 0; e < NI; ++e)
      buffer_load16_to_lds(v_rsrc, vd + e * 1024, v_off[e], (grp + kGroups * t) * kBK * 2);
  };
  auto issue_b = [&](int t) __attribute__((always_inline)) {
    if (wid < G)  // one 256-byte row per query head
      buffer_load4_to_lds(b_rsrc, b_tile(t % 3) + wid * kBK, (wid * Mp + lane) * 4, (grp + kGroups * t) * kBK * 4);
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

  // The pipeline runs over half tiles of 32 keys: half h of the group is keys
  // [key0, key0 + 32) of group tile h >> 1, key0 = (grp + 2 (h >> 1)) * 64 + 32 (h & 1).
  auto h_key0 = [&](int h) { return (grp + kGroups * (h >> 1)) * kBK + 32 * (h & 1); };
  // the wave computes half h: its tile exists and it starts at or before the wave's last query
  auto h_mine = [&](int h) { return h >= 0 && grp + kGroups * (h >> 1) < nkb && wave_rows && h_key0(h) <= rbase + 31; };

  // S^T = K Q^T of half h: one 32 x 32 accumulation chain over DH
  auto qk = [&](int h, f32x16& s) __attribute__((always_inline)) {
    const unsigned char* kt = k_tile((h >> 1) & 1) + (h & 1) * 32 * KROW;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + k_frag_off(ks));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
    }
  };
  // O^T += V^T P^T over the two 16-key steps of half h
  auto pv = [&](int h, const uint32_t (&pk)[8]) __attribute__((always_inline)) {
    const unsigned char* vt_l = v_tile((h >> 1) & 1);
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      const u32x4 pw = {pk[sh * 4], pk[sh * 4 + 1], pk[sh * 4 + 2], pk[sh * 4 + 3]};
      const f16x8 pf = as_f16x8(pw);
      const int st = (h & 1) * 2 + sh;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const u32x4 vw = *reinterpret_cast<const u32x4*>(vt_l + t * 32 * VROW + v_frag_off(st));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vw), pf, o[t], 0, 0, 0);
      }
    }
  };
  // Online softmax of half h's scores, without branches: the running max
  // moves by a select, and the accumulator rescale this implies is left to
  // the caller, which applies `alpha` after the P.V products issued before
  // it.  `diag`: keys after the lane's query are masked.
  auto softmax = [&](int h, f32x16& s, bool diag, uint32_t (&pk)[8], bool& resc,
                     float& alpha) __attribute__((always_inline)) {
    const float* bt = b_tile((h >> 1) % 3) + hloc * kBK + (h & 1) * 32 + gq * 4;
    // logits (log2 domain); lane holds keys key0 + 8(i/4) + 4gq + (i%4)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 bb = *reinterpret_cast<const f32x4*>(bt + i4 * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i4 * 4 + i] = fmaf(s[i4 * 4 + i], cq, bb[i]);
    }
    if (diag) {
      // key offset inside the half (minus this lane's 4*gq) beyond thr => masked
      const int thr = qi - h_key0(h) - gq * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (i >> 2) * 8 + (i & 3) > thr ? -INFINITY : s[i];
    }
    // max: a max3 tree over the 16 logits, then the partner lane's
    const float x0 = max3f(s[0], s[1], s[2]), x1 = max3f(s[3], s[4], s[5]), x2 = max3f(s[6], s[7], s[8]);
    const float x3 = max3f(s[9], s[10], s[11]), x4 = max3f(s[12], s[13], s[14]);
    float mloc = max3f(max3f(x0, x1, x2), x3, max3f(x4, s[15], s[15]));
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
      mloc = max3f(__uint_as_float(pr[0]), __uint_as_float(pr[1]), __uint_as_float(pr[1]));
    }
    resc = __ballot(mloc > m_run + kRescaleSlack) != 0;  // wave-uniform
    const float m_new = resc ? fmaxf(m_run, mloc) : m_run;
    alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    // (a lane with no visible key yet keeps m_run = -inf; its logits are all
    // -inf too, and a finite reference keeps exp2 at 0 instead of NaN)
    const float mref = m_run == -INFINITY ? 0.0f : m_run;
    // numerators (rounded to fp16 for the P.V product) and their fp32 row sum
    float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const float p0 = __builtin_amdgcn_exp2f(s[i] - mref), p1 = __builtin_amdgcn_exp2f(s[i + 1] - mref);
      const float p2 = __builtin_amdgcn_exp2f(s[i + 2] - mref), p3 = __builtin_amdgcn_exp2f(s[i + 3] - mref);
      l0 += p0 + p1;
      l1 += p2 + p3;
      pk[i / 2] = pack_f16x2(p0, p1);
      pk[i / 2 + 1] = pack_f16x2(p2, p3);
    }
    l_run = fmaf(l_run, alpha, l0 + l1);
  };
  auto rescale = [&](bool resc, float alpha) __attribute__((always_inline)) {
    if (resc) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    }
  };
  // Pipeline step h: the scores of half h + 1 and the P.V product of half
  // h - 1 run on the matrix cores while the vector ALUs run the softmax of
  // half h, so the wave always has MFMA work that does not wait on its own
  // softmax.  fast_step is the steady state (half h + 1 is computed by the
  // wave, hence half h lies wholly before its first query and h - 1 >= 0 is
  // computed too); step handles every case.
  // Steady-state scores are kept relative to the running max: the score
  // MFMA starts from cm = -m_run / cq instead of 0, so the logit FMA yields
  // z - m_run directly.  The running max is then not recomputed every half:
  // a half whose numerators could leave fp16 range (row sum > 2^15) takes a
  // rare path that rescales with the true max.
  f32x16 cm;
  auto cm_value = [&]() { return (m_run == -INFINITY || cq == 0.0f) ? 0.0f : -m_run / cq; };
  // This lane's fragment chunks, as loop-invariant LDS offsets: with
  // c = q7 >> 1 and e = q7 & 1, chunk (2j + gq) ^ q7 = 2 (j ^ c) + (gq ^ e),
  // so K k-step ks sits at k_lane[ks & 3] + 128 (ks >> 2) and V^T step st at
  // v_lane[st]; ring slot and half tile only add constants.
  int k_lane[4], v_lane[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sw = 32 * (j ^ (q7 >> 1)) + 16 * (gq ^ (q7 & 1));
    k_lane[j] = grp * TILE + ql * KROW + sw;
    v_lane[j] = V_BASE + grp * TILE + ql * VROW + sw;
  }
  // Steady-state step: SB = 0 for an iteration's first step (h = 2i + 1),
  // 1 for its second (h = 2i + 2); kb / vb are the lane bases of the
  // iteration's K slot (tile i + 1) and V^T slot (tile i).
  auto fast_step = [&](int h, f32x16& s, f32x16& sn, uint32_t (&pc)[8], const uint32_t (&pp)[8],
                       const int (&kb)[4], const int (&vb)[4], auto step_c) __attribute__((always_inline)) {
    // NS = 2 KS issue slots: even slot k runs k-step k/2 of the scores of
    // half h + 1, odd slot k runs P.V step k/2 of half h - 1 (16-key step
    // (k/2) / DT, output tile (k/2) % DT).  Each slot also issues the LDS
    // read of the fragment three slots ahead and a share of the softmax of
    // half h (13 shares spread over the slots).  Scheduling fences keep
    // this order.
    constexpr int SB = decltype(step_c)::value;
    constexpr int NS = 2 * KS;
    static_assert(2 * DT == KS && 16 % NS == 0, "slot plan");
    const float* bt = b_tile((h >> 1) % 3) + hloc * kBK + (1 - SB) * 32 + gq * 4;
    u32x4 fr[NS];
    auto read_frag = [&](int r) __attribute__((always_inline)) {
      if (r & 1) {
        const int p = r >> 1;
        fr[r] = *reinterpret_cast<const u32x4*>(smem + vb[2 * SB + p / DT] + (p % DT) * 32 * VROW);
      } else {
        const int ks = r >> 1;
        fr[r] = *reinterpret_cast<const u32x4*>(smem + kb[ks & 3] + SB * 32 * KROW + 128 * (ks >> 2));
      }
    };
    f32x4 bb[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) bb[i4] = *reinterpret_cast<const f32x4*>(bt + i4 * 8);
#pragma unroll
    for (int r = 0; r < 3 && r < NS; ++r) read_frag(r);
    f16x8 pf[2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      const u32x4 pw = {pp[sh * 4], pp[sh * 4 + 1], pp[sh * 4 + 2], pp[sh * 4 + 3]};
      pf[sh] = as_f16x8(pw);
    }
    const float l_prev = l_run;
    __builtin_amdgcn_sched_barrier(0);
    float l = 0.f;
    bool ovf = false;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k + 3 < NS) read_frag(k + 3);
      if ((k & 1) == 0) {
        sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[k]), qf[k >> 1], k == 0 ? cm : sn, 0, 0, 0);
      } else {
        const int p = k >> 1;
        o[p % DT] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(fr[k]), pf[p / DT], o[p % DT], 0, 0, 0);
      }
#pragma unroll
      for (int v = k * 16 / NS; v < (k + 1) * 16 / NS; ++v) {  // softmax shares of this slot
        if (v < 4) {  // z - m_run (log2 domain) of keys 8v + 4gq + (0..3)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[v * 4 + i] = fmaf(s[v * 4 + i], cq, bb[v][i]);
        }
        if (v >= 4 && v < 12) {  // numerators 2(v-4), 2(v-4)+1
          const int e = 2 * (v - 4);
          const float p0 = __builtin_amdgcn_exp2f(s[e]), p1 = __builtin_amdgcn_exp2f(s[e + 1]);
          l += p0 + p1;
          pc[e / 2] = pack_f16x2(p0, p1);
          asm volatile("" ::"v"(pc[e / 2]));  // computed in this slot, not sunk to its later use
        }
        if (v == 12) {
          ovf = __ballot(!(l <= 32768.0f)) != 0;  // wave-uniform; catches inf too
          l_run = l_prev + l;
          asm volatile("" ::"v"(l_run));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ovf) {
      // some numerator left the safe range: move the reference up to the
      // row's true max and redo this half's numerators
      const float x0 = max3f(s[0], s[1], s[2]), x1 = max3f(s[3], s[4], s[5]), x2 = max3f(s[6], s[7], s[8]);
      const float x3 = max3f(s[9], s[10], s[11]), x4 = max3f(s[12], s[13], s[14]);
      float mloc = max3f(max3f(x0, x1, x2), x3, max3f(x4, s[15], s[15]));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float d = fmaxf(mloc, 0.0f);
      const float alpha = __builtin_amdgcn_exp2f(-d);
      m_run += d;
      float l2 = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[e] - d), p1 = __builtin_amdgcn_exp2f(s[e + 1] - d);
        l2 += p0 + p1;
        pc[e / 2] = pack_f16x2(p0, p1);
      }
      l_run = fmaf(l_prev, alpha, l2);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
      // the scores of half h + 1 were started from the old reference
      const float dq = cq == 0.0f ? 0.0f : d / cq;
      const float mc = cm_value();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sn[i] -= dq;
        cm[i] = mc;
      }
    }
  };
  auto step = [&](int h, f32x16& s_cur, f32x16& s_next, uint32_t (&p_cur)[8],
                  const uint32_t (&p_prev)[8]) __attribute__((always_inline)) {
    bool resc = false;
    float alpha = 1.0f;
    if (h_mine(h - 1)) pv(h - 1, p_prev);
    if (h_mine(h)) softmax(h, s_cur, h_key0(h) + 31 > rbase, p_cur, resc, alpha);
    if (h_mine(h + 1)) qk(h + 1, s_next);
    rescale(resc, alpha);
  };

  // Staging: iteration i (pipeline steps 2i + 1 and 2i + 2) reads K of group
  // tile i + 1, V^T of tile i and key scores of tiles i and i + 1, and
  // requests K of tile i + 2, V^T of tile i + 1 and key scores of tile i + 2
  // into the slots whose last reads ended at the previous iteration's
  // barrier; its loads complete before its own closing barrier.
  const int nit = (nkb + kGroups - 1) / kGroups;  // tiles of group 0 (group 1 has as many or one fewer)
  auto t_exists = [&](int t) { return grp + kGroups * t < nkb; };
  // Leading iterations in which every wave of the workgroup is in steady
  // state for both steps: half 2i + 3 must be computed by the wave with the
  // lowest rows (rbase = q0) in either group.
  int n_steady = nit;
#pragma unroll
  for (int gg = 0; gg < kGroups; ++gg) {
    const int nt = (nkb - gg + kGroups - 1) / kGroups;  // tiles of group gg
    const int X = q0 + 31 - kBK * gg;                   // last visible key offset past the group's first tile
    int hmax = -1;                                      // last half the lowest wave of group gg computes
    if (X >= 0 && nt > 0) {
      const int tm = min(nt - 1, X / (kGroups * kBK));
      hmax = 2 * tm + ((X - kGroups * kBK * tm) >= 32 ? 1 : 0);
    }
    n_steady = min(n_steady, hmax >= 3 ? ((hmax - 3) >> 1) + 1 : 0);
  }
  n_steady = __builtin_amdgcn_readfirstlane(n_steady);
  if (t_exists(0)) {
    issue_k(0);
    issue_b(0);
  }
  // Q fragments and the original position are requested while the first
  // tile is in flight; one wait covers all of them
  {
    const uint16_t* qp = q + ((T0 + (q_ok ? qi : 0)) * Hq + hq) * DH + gq * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(q_ok ? load16(qp + ks * 16) : u32x4{0, 0, 0, 0});
  }
  const int p_orig = pos[T0 + (q_ok ? qi : 0)];
  const float t_h = temp[hq];
  wait_vmem();
  if (q_ok) {
    float ratio = 1.0f;
    if (p_orig != qi) ratio = logf((float)max(p_orig + 1, 2)) / logf((float)max(qi + 1, 2));
    cq = sm_scale * kLog2e / (t_h * ratio);
  }
  __syncthreads();
  if (t_exists(1)) {
    issue_k(1);
    issue_b(1);
  }
  if (t_exists(0)) issue_v(0);
  f32x16 sa, sb;
  uint32_t pa[8], pb[8];
  if (h_mine(0)) qk(0, sa);
  step(0, sa, sb, pa, pb);  // no P.V yet: half -1 is never computed
  wait_vmem();
  __syncthreads();
  auto stage = [&](int i) __attribute__((always_inline)) {
    if (t_exists(i + 2)) {
      issue_k(i + 2);
      issue_b(i + 2);
    }
    if (t_exists(i + 1)) issue_v(i + 1);
  };
  int i = 0;
  if (n_steady > 0) {
    // enter the relative form: the pending scores of half 1 and the
    // accumulator start value
    const float mc = cm_value();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      cm[e] = mc;
      sb[e] += mc;
    }
    // The two groups issue their loads at different points: group 1 at the
    // top of the iteration, group 0 between the two steps.  The two waves
    // sharing a SIMD (one of each group) then leave the barrier out of
    // phase -- one issues loads while the other starts its matrix work --
    // instead of contending for the same slots in lockstep, and the wave
    // that the SIMD favours (group 0) takes the later load slot.
    auto iter = [&](int it) __attribute__((always_inline)) {
      // ring slots of this iteration: K of tile it + 1, V^T of tile it
      int kb[4], vb[4];
      const int koff = ((it + 1) & 1) * kGroups * TILE, voff = (it & 1) * kGroups * TILE;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kb[j] = k_lane[j] + koff;
        vb[j] = v_lane[j] + voff;
      }
      if (grp == 1) stage(it);
      fast_step(2 * it + 1, sb, sa, pb, pa, kb, vb, IntConst<0>{});
      if (grp == 0) stage(it);
      fast_step(2 * it + 2, sa, sb, pa, pb, kb, vb, IntConst<1>{});
      wait_vmem();
      __syncthreads();
    };
    for (; i < n_steady; ++i) iter(i);
    // leave it: the pending scores go back to the plain form
#pragma unroll
    for (int e = 0; e < 16; ++e) sb[e] -= cm[e];
  }
  for (; i < nit; ++i) {
    stage(i);
    step(2 * i + 1, sb, sa, pb, pa);
    step(2 * i + 2, sa, sb, pa, pb);
    wait_vmem();
    __syncthreads();
  }

  // Merge the two groups' online-softmax states (the tile buffers are free
  // now).  Each group finalises half of the output columns: group g keeps
  // O^T tiles [g DT/2, (g+1) DT/2) and hands its other tiles, with m and l,
  // to the other group as 16-byte vectors per lane.  (The group number is
  // made a constant of each branch so that o[] keeps static indices.)
  constexpr int DH2 = DT / 2;  // O^T tiles finalised per group
  static_assert(2 * DH2 == DT, "column split");
  f32x4* sm4 = reinterpret_cast<f32x4*>(smem);
  const int slot = wid * 64 + lane;
  // LDS: [group][256] (m, l), then [receiving group][tile][i4][256] O values
  auto o_slot = [&](int dst, int j, int i4) { return 512 + ((dst * DH2 + j) * 4 + i4) * 256 + slot; };
  // Output rows leave through LDS so that each store writes whole 16-byte
  // pieces: the wave's 32 rows x (its group's DH/2 columns) bf16 block is
  // written row-major with the 16-byte chunks of row r XOR-swizzled by r,
  // then read back 16 bytes per lane.  The region lies past the merge
  // vectors and belongs to this wave alone, and LDS operations of one wave
  // complete in order.
  constexpr int HROW = DH;        // bytes of half an output row
  constexpr int HCH = HROW / 16;  // its 16-byte chunks
  static_assert((512 + 2 * DH2 * 4 * 256) * 16 + kGroups * 4 * 32 * HROW <= LDS_BYTES, "merge and output staging");
  auto hand_over = [&](auto gc) __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value, og = 1 - g;
    sm4[g * 256 + slot] = f32x4{m_run, l_run, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < DH2; ++j)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int t = og * DH2 + j;
        sm4[o_slot(og, j, i4)] = f32x4{o[t][i4 * 4], o[t][i4 * 4 + 1], o[t][i4 * 4 + 2], o[t][i4 * 4 + 3]};
      }
  };
  auto finish = [&](auto gc) __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value, og = 1 - g;
    const f32x4 ml = sm4[og * 256 + slot];
    const float m1 = ml[0], l1 = ml[1];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    m_run = m;
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int j = 0; j < DH2; ++j)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int t = g * DH2 + j;
        const f32x4 o1 = sm4[o_slot(g, j, i4)];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i4 * 4 + i] = o[t][i4 * 4 + i] * a0 + o1[i] * a1;
      }
    if (!wave_rows) return;
    const float l_tot = pair_sum(l_run);
    const float inv = (float)(1 << kVScaleLog2) / l_tot;
    unsigned char* ob = smem + (512 + 2 * DH2 * 4 * 256) * 16 + wall * 32 * HROW;
#pragma unroll
    for (int j = 0; j < DH2; ++j)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        // d = 32t + 8 i4 + 4gq + (0..3), t = g DH2 + j: chunk 4j + i4 of the half row, half gq
        const int t = g * DH2 + j;
        u32x2 w;
        w[0] = pack_bf16x2(o[t][i4 * 4 + 0] * inv, o[t][i4 * 4 + 1] * inv);
        w[1] = pack_bf16x2(o[t][i4 * 4 + 2] * inv, o[t][i4 * 4 + 3] * inv);
        const int chunk = (j * 4 + i4) ^ (ql & (HCH - 1));
        *reinterpret_cast<u32x2*>(ob + ql * HROW + chunk * 16 + gq * 8) = w;
      }
    constexpr int RPI = 64 / HCH;  // rows per 64-lane store
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPI) {
      const int r = r0 + lane / HCH, c = lane % HCH;
      const u32x4 w = *reinterpret_cast<const u32x4*>(ob + r * HROW + ((c ^ (r & (HCH - 1))) * 16));
      if (rbase + r < M) store16(out + ((T0 + rbase + r) * Hq + hq) * DH + g * (DH / 2) + c * 8, w);
    }
    if (lse != nullptr && g == 0 && gq == 0 && q_ok)
      lse[T0 * Hq + (size_t)hq * M + qi] = (m_run + __log2f(l_tot)) * kLn2;
  };
  if (grp == 0)
    hand_over(IntConst<0>{});
  else
    hand_over(IntConst<1>{});
  __syncthreads();
  if (grp == 0)
    finish(IntConst<0>{});
  else
    finish(IntConst<1>{});
}

template <int DH, int G>
hipError_t launch_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq, int Hkv,
                    const float* ks, const int32_t* pos, const float* gain, const float* temp, float sm_scale,
                    uint16_t* out, float* lse, uint16_t* vt, float* kbias, const RopeArgs* rope, hipStream_t s) {
  constexpr int BQ = 32 * (4 / G);
  const int Mp = (M + kBK - 1) / kBK * kBK;
  if (rope != nullptr) {
    hipLaunchKernelGGL((attn_prepass_kernel<DH, true, false>), dim3(Mp / kBK, Hkv, B), dim3(kThreads), 0, s, v, ks,
                       gain, M, Mp, Hkv, G, vt, kbias, *rope, SeqTable{});
    q = rope->qr;  // the main kernel reads the rotated copies
    k = rope->kr;
  } else {
    hipLaunchKernelGGL((attn_prepass_kernel<DH, false, false>), dim3(Mp / kBK, Hkv, B), dim3(kThreads), 0, s, v, ks,
                       gain, M, Mp, Hkv, G, vt, kbias, RopeArgs{}, SeqTable{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (M + BQ - 1) / BQ;
  const long long total = (long long)nqb * Hkv * B;
  if (total <= 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gated_attn_kernel<DH, G, false>), dim3((unsigned)total), dim3(kAttnThreads), 0, s, q, k, vt,
                     kbias, M, Mp, Hq, Hkv, pos, temp, sm_scale, out, lse, nqb, (int)total, SeqTable{});
  return hipGetLastError();
}

// One prepass and one attention launch over the sequences of a table.
template <int DH, int G>
hipError_t launch_varlen_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, const SeqTable& st, int Hq,
                           int Hkv, const float* ks, const int32_t* pos, const float* gain, const float* temp,
                           float sm_scale, uint16_t* out, float* lse, uint16_t* vt, float* kbias, hipStream_t s) {
  hipLaunchKernelGGL((attn_prepass_kernel<DH, false, true>), dim3((unsigned)st.pb0[st.n], Hkv, 1), dim3(kThreads), 0,
                     s, v, ks, gain, 0, 0, Hkv, G, vt, kbias, RopeArgs{}, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = st.wg0[st.n];
  hipLaunchKernelGGL((gated_attn_kernel<DH, G, true>), dim3((unsigned)total), dim3(kAttnThreads), 0, s, q, k, vt,
                     kbias, 0, 0, Hq, Hkv, pos, temp, sm_scale, out, lse, 0, total, st);
  return hipGetLastError();
}

}  // namespace

// fp16 V^T [B, Hkv, dh, Mp], then the fp32 key-score terms [B, Hq, Mp]
size_t gated_attention_workspace(int B, int M, int Hq, int Hkv, int dh) {
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  return (size_t)B * Mp * ((size_t)Hkv * dh * 2 + (size_t)Hq * 4);
}

// ... then the rotated q [B, M, Hq, dh] and k [B, M, Hkv, dh] (bf16)
size_t gated_attention_rope_workspace(int B, int M, int Hq, int Hkv, int dh) {
  return gated_attention_workspace(B, M, Hq, Hkv, dh) + (size_t)B * M * (Hq + Hkv) * dh * 2;
}

size_t gated_attention_varlen_slots(int B, const int32_t* cu_seqlens) {
  size_t slots = 0;
  for (int b = 0; b < B; ++b) slots += (size_t)(cu_seqlens[b + 1] - cu_seqlens[b] + kBK - 1) / kBK * kBK;
  return slots;
}

hipError_t launch_gated_attention_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B,
                                         const int32_t* cu_seqlens, int Hq, int Hkv, int dh, const float* key_score,
                                         const int32_t* pos, const float* gain, const float* temp, float sm_scale,
                                         uint16_t* out, float* lse, void* ws, hipStream_t s) {
  const int G = Hq / Hkv;
  constexpr int BQ_G[5] = {0, 128, 64, 0, 32};  // query rows per workgroup by group size
  if (G != 1 && G != 2 && G != 4) return hipErrorInvalidValue;
  // the non-empty sequences, longest first: their heavy query blocks start first
  std::vector<int> order;
  for (int b = 0; b < B; ++b)
    if (cu_seqlens[b + 1] > cu_seqlens[b]) order.push_back(b);
  std::stable_sort(order.begin(), order.end(), [&](int a, int c) {
    return cu_seqlens[a + 1] - cu_seqlens[a] > cu_seqlens[c + 1] - cu_seqlens[c];
  });
  const size_t slots = gated_attention_varlen_slots(B, cu_seqlens);
  uint16_t* vt = static_cast<uint16_t*>(ws);
  float* kbias = reinterpret_cast<float*>(vt + slots * Hkv * dh);
  size_t p = 0;
  for (size_t i = 0; i < order.size(); i += kMaxSeqsPerLaunch) {
    SeqTable st{};
    st.n = (int)std::min(order.size() - i, (size_t)kMaxSeqsPerLaunch);
    long long pb = 0, wg = 0;
    for (int j = 0; j < st.n; ++j) {
      const int b = order[i + j], m = cu_seqlens[b + 1] - cu_seqlens[b];
      const int mp = (m + kBK - 1) / kBK * kBK;
      if (p + mp > 0x7FFFFFFF) return hipErrorInvalidValue;
      st.t0[j] = cu_seqlens[b];
      st.m[j] = m;
      st.p0[j] = (int)p;
      st.pb0[j] = (int)pb;
      st.wg0[j] = (int)wg;
      p += mp;
      pb += mp / kBK;
      wg += (long long)((m + BQ_G[G] - 1) / BQ_G[G]) * Hkv;
      if (wg > 0x7FFFFFFF / kAttnThreads) return hipErrorInvalidValue;
    }
    st.pb0[st.n] = (int)pb;
    st.wg0[st.n] = (int)wg;
    hipError_t e = hipErrorInvalidValue;
#define TG_ATTN_VARLEN_CASE(DHV, GV)                                                                          \
  if (dh == DHV && G == GV)                                                                                   \
    e = launch_varlen_t<DHV, GV>(q, k, v, st, Hq, Hkv, key_score, pos, gain, temp, sm_scale, out, lse, vt, kbias, \
                                 s);
    TG_ATTN_VARLEN_CASE(128, 2)
    TG_ATTN_VARLEN_CASE(128, 1)
    TG_ATTN_VARLEN_CASE(128, 4)
    TG_ATTN_VARLEN_CASE(64, 2)
    TG_ATTN_VARLEN_CASE(64, 1)
    TG_ATTN_VARLEN_CASE(64, 4)
#undef TG_ATTN_VARLEN_CASE
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq,
                                  int Hkv, int dh, const float* key_score, const int32_t* pos, const float* gain,
                                  const float* temp, float sm_scale, double rope_base, uint16_t* out, float* lse,
                                  void* ws, hipStream_t s) {
  const int G = Hq / Hkv;
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  uint16_t* vt = static_cast<uint16_t*>(ws);
  float* kbias = reinterpret_cast<float*>(vt + (size_t)B * Hkv * dh * Mp);
  RopeArgs ra{};
  const RopeArgs* rope = nullptr;
  if (rope_base > 0.0) {
    uint16_t* qr = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(ws) +
                                               gated_attention_workspace(B, M, Hq, Hkv, dh));
    ra = RopeArgs{q, k, pos, rope_base, qr, qr + (size_t)B * M * Hq * dh};
    rope = &ra;
  }
#define TG_ATTN_CASE(DHV, GV)                                                                                   \
  if (dh == DHV && G == GV)                                                                                     \
    return launch_t<DHV, GV>(q, k, v, B, M, Hq, Hkv, key_score, pos, gain, temp, sm_scale, out, lse, vt, kbias, \
                             rope, s);
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
