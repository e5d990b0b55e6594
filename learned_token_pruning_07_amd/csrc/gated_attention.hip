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
//    call by a prepass into V^T (key-contiguous) fp16.  Each 64-key tile of
//    a KV head is scaled by its own power of two 2^e, chosen from the tile's
//    largest magnitude so that it lands in [2^14, 2^15): every bf16 value
//    within 2^28 of the tile's largest converts exactly.  The factor moves
//    to the numerators: the tile's key terms carry -e, so the kernel's
//    numerator is P 2^-e and the product P 2^-e . V 2^e is unchanged, and
//    the row sum, which needs P itself, multiplies the tile's numerator sum
//    by 2^e (one product per half tile).  Inside every 16-key group of V^T
//    the middle two quads of keys are swapped, so that the 8 keys one lane
//    contributes to a 16-key P.V step (4 at 4*gq, 4 at 8 + 4*gq) form one
//    16-byte chunk.
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
//    head, gain_h * log2(e) * b_j - e, and a row holding the tile's 2^e, so
//    that those tiles too are plain copies.
//  * Grid (batched rows): a persistent grid of one workgroup per CU works
//    through the query blocks, heaviest causal blocks first, in a snake
//    order that pairs each workgroup's heavy and light blocks; every block
//    of one KV head stays on one XCD (shared L2 for its K/V).  A workgroup
//    requests its next block's Q fragments as soon as it has written the
//    current block's output.  Varying-length launches run one workgroup
//    per query block, heaviest first.
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
constexpr int kRopeRows = 16;  // rows whose rotary angles the prepass holds in LDS at a time

// V^T tile scale exponents: the tile's largest |v| times 2^e lies in
// [2^14, 2^15) when e is inside this range (tile maxima in [2^-36, 2^65)).
// The range keeps the row sum, which carries 2^e, far inside fp32, and
// bounds the spread of e between tiles (see the kernel's row sum).
constexpr int kVExpMin = -50, kVExpMax = 50;
constexpr int kBufferConfig = 0x00020000;  // raw buffer resource word 3 (gfx9 family, 32-bit data)
// Outside the steady state the running max is only moved (and the
// accumulator rescaled) when a half tile's max exceeds it by more than this
// many log2 units; P stays <= 2^8 there.
constexpr float kRescaleSlack = 8.0f;

#ifdef TG_DIAG_COUNTERS
// Test build only (libtokengate_diag.so): how often the kernel took its rare
// paths, one count per wave and event.  0: a steady-state half whose
// numerators left the fp16-safe range and was redone with a new reference;
// 1: a mid-row move of the running max outside the steady state.
__device__ unsigned long long g_diag_count[4];
#define TG_DIAG_HIT(i)                                                  \
  do {                                                                  \
    if ((threadIdx.x & 63) == 0) atomicAdd(&g_diag_count[i], 1ull);     \
  } while (0)
// Per-block timeline of the last launch (100 MHz real-time counter), by block
// id (slab * query blocks + qb, or the workgroup of a varying-length launch):
// [logical workgroup | qb << 32, start, prologue done, first step done,
// steady loop done, all key tiles done, end, round] for ids below kDiagWG.
constexpr int kDiagWG = 8192;
__device__ unsigned long long g_diag_wg[kDiagWG][8];
// finer stamps of the prologue and first step: [before the first loads,
// after their wait, after the first step's loads are issued, after its wait]
__device__ unsigned long long g_diag_pro[kDiagWG][4];
#define TG_DIAG_STAMP(k) \
  do {                   \
    diag_t[k] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define TG_DIAG_PSTAMP(k) \
  do {                    \
    diag_p[k] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define TG_DIAG_PSTAMP(k) \
  do {                    \
  } while (0)
#define TG_DIAG_STAMP(k) \
  do {                   \
  } while (0)
#define TG_DIAG_HIT(i) \
  do {                 \
  } while (0)
#endif

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
// rotated copy of k, and a table of the cosines and sines of every row's
// angles ([rows, DH/2] pairs (cos, sin), fp32) from which the attention
// kernel rotates its Q fragments.
struct RopeArgs {
  const uint16_t* k;
  const int32_t* pos;
  double base;
  float* tab;
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

// The rotary angle table, by padded key slot, in the attention kernel's
// fragment order: for slots 32 n .. 32 n + 31 (one wave's queries), piece
// (ks, u) of lane l = 32 gq + (slot & 31) is the f32x4 (cos, sin, cos, sin) of
// pairs 16 ks + 8 gq + 2u and + 1 (ks < DH / 32, u < 4), and the 64 lanes'
// pieces of one (ks, u) are 1 KiB contiguous, so each load of the kernel's
// Q rotation reads whole cache lines.  Pairs i0 .. i0 + 7 (i0 a multiple of
// 8) of a slot are pieces u = 0..3, 64 pieces apart, from the one returned.
template <int DH>
__device__ __forceinline__ f32x4* rope_tab_piece(float* tab, size_t slot, int i0) {
  const int ks = i0 >> 4, gq = (i0 >> 3) & 1;
  return reinterpret_cast<f32x4*>(tab) + ((slot >> 5) * (DH / 32) + ks) * 4 * 64 + gq * 32 + (slot & 31);
}

// One prepass workgroup per 64-key block: DH threads, thread t owning the 8
// d values 8 (t mod DH/8) .. + 7 of the 8 keys whose V^T slots form chunk
// t / (DH/8) of the block's rows (keys 16 n + 4 v + {0..3, 8..11}, n = chunk / 2,
// v = chunk mod 2, in slot order).  Its 8 loads read those keys' 16-byte
// pieces (DH/8 consecutive lanes read one whole row), and the transposition
// to V^T rows happens in registers: word p of its piece of row d packs the
// keys of slots 8 chunk + 2p and + 1.
template <int DH>
constexpr int kPreThreads = DH;

// Prepass, per 64-key block of KV head g:
//   e = the block's scale exponent: 141 - (exponent field of the largest
//   bf16 magnitude), clamped to [kVExpMin, kVExpMax], so that the largest
//   |v| 2^e lies in [2^14, 2^15);
//   V [B, M, Hkv, DH] bf16 -> V^T [B, Hkv, DH, Mp] fp16 = V 2^e (round to
//   nearest even, keys in slot order, zero beyond M);
//   key-score rows kb [B, Hkv, G + 1, Mp] fp32: row hh < G holds
//   gain_h * log2(e) * key_score - e for query head h = g G + hh (zero
//   beyond M), row G holds 2^e for every key of the block;
//   with ROPE, also the rotary embedding of the block's K rows (head g) at
//   their original positions (the rotate-half form: pair (x_i, x_{i+DH/2})
//   turns by pos * base^(-2i/DH)) and, in the blocks of KV head 0, the
//   table of those angles' cosines and sines for the attention kernel's Q
//   rotation.  The angle is formed and reduced modulo 2 pi in fp64, so that
//   its fp32 sine and cosine are accurate to a few ulp at any position.
// VARLEN: the blocks of the table's sequences, one grid row per KV head.
template <int DH, bool ROPE, bool VARLEN>
__global__ __launch_bounds__(kPreThreads<DH>) void attn_prepass_kernel(const uint16_t* __restrict__ v,
                                                                       const float* __restrict__ key_score,
                                                                       const float* __restrict__ gain, int M_all,
                                                                       int Mp_all, int Hkv, int G,
                                                                       uint16_t* __restrict__ vt,
                                                                       float* __restrict__ kbias, RopeArgs ra,
                                                                       const SeqTable st,
                                                                       const int32_t* __restrict__ m_dev) {
  constexpr int kT = kPreThreads<DH>;
  constexpr int kNW = kT / 64;
  static_assert(kT % 64 == 0 && kBK == 64, "prepass layout");
  __shared__ double s_freq[DH / 2];
  __shared__ uint32_t s_mag[kNW];
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
    if (m_dev != nullptr) {  // this row's kept length; its blocks past it have nothing to do
      M = min(max(m_dev[blockIdx.z], 0), M_all);
      if (m0 >= M) return;
    }
    T0 = (size_t)blockIdx.z * M_all;
    P0 = (size_t)blockIdx.z * Mp;
  }
  const int tid = threadIdx.x;
  if (ROPE && tid < DH / 2) s_freq[tid] = rope::inv_freq(ra.base, tid, DH);
  constexpr int CPR = DH / 8;       // 16-byte pieces per row
  const int dc = tid % CPR;         // this thread's d values: 8 dc .. 8 dc + 7
  const int ch = tid / CPR;         // its chunk of the block's V^T rows (slots 8 ch .. 8 ch + 7)
  const int kbase = 16 * (ch >> 1) + 4 * (ch & 1);
  auto key_of = [&](int j) { return kbase + (j & 3) + 8 * (j >> 2); };  // key in slot 8 ch + j
  // The block's rows of head g through a range-checked resource that ends
  // with row M - 1: a key at or past M reads zeros, with no select.
  const int nvalid = min(M - m0, kBK);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(v + ((T0 + m0) * Hkv + g) * DH), (short)0, ((nvalid - 1) * Hkv + 1) * DH * 2,
      kBufferConfig);
  u32x4 w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, key_of(j) * Hkv * DH * 2 + dc * 16, 0, 0));
  // The key-score rows: value c of the block is row c / 64, key m0 + c mod 64;
  // thread t writes c = t + u kT, all of key mk.  Its key score and gains are
  // requested with the V loads (clamped in-bounds, masked later), so that
  // nothing waits on a load once the scale is known.  (G <= 4.)
  constexpr int kKbIt = (5 * kBK + kT - 1) / kT;
  const int mk = m0 + (tid & (kBK - 1));
  const float ksv = key_score[T0 + min(mk, M - 1)];
  float gk[kKbIt];
#pragma unroll
  for (int u = 0; u < kKbIt; ++u) gk[u] = gain[g * G + min((tid + u * kT) / kBK, G - 1)];
  // the block's largest bf16 magnitude (sign cleared; NaN and inf compare
  // above every finite value), as an integer max over the bit patterns
  uint32_t mag = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) mag = max(mag, max(w[j][i] & 0x7FFFu, (w[j][i] >> 16) & 0x7FFFu));
  mag = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max_u32(mag), 63);
  if constexpr (kNW > 1) {
    if ((tid & 63) == 0) s_mag[tid >> 6] = mag;
    __syncthreads();
#pragma unroll
    for (int wv = 0; wv < kNW; ++wv) mag = max(mag, s_mag[wv]);
  }
  const int ex = min(max(141 - (int)(mag >> 7), kVExpMin), kVExpMax);
  const float scale = __uint_as_float((uint32_t)(ex + 127) << 23);  // 2^ex, exact
  // fp16 V 2^ex, round to nearest even: exact for every value within 2^28
  // below the block's largest.  Row 8 dc + i, word p: keys of slots 8 ch + 2p, + 1.
  uint16_t* vt_row = vt + P0 * Hkv * DH + ((size_t)g * DH + dc * 8) * Mp + m0 + ch * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = w[2 * p][i >> 1], b = w[2 * p + 1][i >> 1];
      o[p] = (i & 1) ? pack_f16x2(bf16_hi(a) * scale, bf16_hi(b) * scale)
                     : pack_f16x2(bf16_lo(a) * scale, bf16_lo(b) * scale);
    }
    store16(vt_row + (size_t)i * Mp, o);
  }
  const int Hq = Hkv * G;
  float* kb = kbias + P0 * (size_t)(Hq + Hkv) + (size_t)g * (G + 1) * Mp + mk;
#pragma unroll
  for (int u = 0; u < kKbIt; ++u) {
    const int hh = (tid + u * kT) / kBK;
    if (hh <= G) kb[(size_t)hh * Mp] = hh == G ? scale : (mk < M ? fmaf(ksv, gk[u] * kLog2e, (float)-ex) : 0.0f);
  }
  if constexpr (ROPE) {
    // The angles of a row are formed once, by one of the Hkv blocks of its
    // 64-key block (rows g R .. g R + R - 1, R = ceil(64 / Hkv)), which then
    // turns that row's K for every KV head and writes its table row; up to
    // kRopeRows rows at a time, their (cos, sin) pairs in LDS.  Item t of a
    // pass is pairs 8 (t mod PG) .. + 7 of row t / (PG Hkv), head
    // (t / PG) mod Hkv (consecutive threads: one row's heads in memory
    // order).  A thread's first kIt items of a pass request their K pieces
    // before the angles are formed (clamped to row M - 1; rows at or past M
    // are skipped), so that the loads overlap that work.
    constexpr int PG = DH / 2 / 8;  // groups of 8 pairs per head row
    constexpr int kIt = 4;
    __shared__ f32x2 s_cs[kRopeRows][DH / 2];
    const int R = (kBK + Hkv - 1) / Hkv;
    const int r_hi = min(kBK, (g + 1) * R);
    __syncthreads();  // s_freq is written
    for (int c0 = g * R; c0 < r_hi; c0 += kRopeRows) {  // (block-uniform)
      const int nr = min(kRopeRows, r_hi - c0);
      const int n_items = nr * PG * Hkv;
      u32x4 ka[kIt], kp[kIt];
      auto item_row = [&](int t) { return ((T0 + min(m0 + c0 + t / (PG * Hkv), M - 1)) * Hkv + (t / PG) % Hkv) * DH; };
      auto load_items = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kIt; ++u) {
          const int t = t0 + u * kT, i0 = (t % PG) * 8;
          const uint16_t* src = ra.k + item_row(t);
          ka[u] = load16(src + i0);
          kp[u] = load16(src + DH / 2 + i0);
        }
      };
      load_items(tid);
      for (int t = tid; t < nr * PG; t += kT) {
        const int rr = t / PG, i0 = (t % PG) * 8, m = m0 + c0 + rr;
        // the table holds pairs i0 .. i0 + 7 of slot P0 + m as 4 pieces (the
        // padding slots past M hold zeros: their queries turn into 0)
        f32x4* tb = rope_tab_piece<DH>(ra.tab, P0 + m, i0);
        if (m >= M) {
#pragma unroll
          for (int u = 0; u < 4; ++u) tb[u * 64] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          continue;
        }
        float c[8], sn[8];
        rope::sincos8((double)ra.pos[T0 + m], s_freq, i0, c, sn);
#pragma unroll
        for (int u = 0; u < 4; ++u) tb[u * 64] = f32x4{c[2 * u], sn[2 * u], c[2 * u + 1], sn[2 * u + 1]};
#pragma unroll
        for (int i = 0; i < 8; ++i) s_cs[rr][i0 + i] = f32x2{c[i], sn[i]};
      }
      __syncthreads();
      for (int t0 = tid; t0 < n_items; t0 += kIt * kT) {
        if (t0 != tid) load_items(t0);
#pragma unroll
        for (int u = 0; u < kIt; ++u) {
          const int t = t0 + u * kT, i0 = (t % PG) * 8, rr = t / (PG * Hkv);
          if (t >= n_items || m0 + c0 + rr >= M) continue;
          float c[8], sn[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const f32x2 cs = s_cs[rr][i0 + i];
            c[i] = cs[0];
            sn[i] = cs[1];
          }
          rope::row8_rotate<DH>(ka[u], kp[u], ra.kr + item_row(t), i0, c, sn);
        }
      }
      __syncthreads();  // (before the next rows' pairs overwrite LDS)
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

// The attention kernel's scalar arguments.  The kernel reads them from its
// argument segment at the start of every block it works on (not once), so
// that its loop over blocks carries only the segment's address in registers.
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;
  const float* kbias;
  const int32_t* pos;
  const float* temp;
  uint16_t* out;
  float* lse;
  const int32_t* m_dev;
  const float* rope_tab;  // the angle table (rope_tab_piece layout), or null: q is used as given
  int M_all, Mp_all, Hq, Hkv, nqb_all, total_wg, n_slabs;
  float sm_scale;
};
typedef const __attribute__((address_space(4))) AttnArgs* AttnArgsPtr;

// The persistent schedule of the batched launch.  Slab = batch row x KV head;
// level L of a slab is its query block nqb - 1 - L (the heaviest first).
// Round r hands rank r P + w to workgroup w when r is even and rank
// r P + P - 1 - w when it is odd (P workgroups deal out a partition), so each
// workgroup's heavy and light blocks pair up and a workgroup moves to its
// next block without a new dispatch.  When the slabs divide evenly over the
// 8 XCDs, XCD x deals out only the slabs x, x + 8, ... among its own
// workgroups (consecutive logical ids share an XCD), so each KV head's K/V
// tiles stay in one L2.  Returns 0 past the workgroup's last block, 1 when
// round r has nothing for it (a query block past a short row's kept length),
// 2 with the block's batch row b, KV head g, query block qb and the row's
// kept length M.  Everything is derived from the argument segment here, so
// no schedule value stays live while a block runs.
template <int BQ>
__device__ __forceinline__ int sched_block(AttnArgsPtr ap, int rnd, int& b, int& g, int& qb, int& M) {
  const int total_wg = ap->total_wg, n_slabs = ap->n_slabs, nqb_all = ap->nqb_all, Hkv = ap->Hkv;
  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  const bool by_xcd = n_slabs % 8 == 0 && total_wg % 8 == 0;
  const int sched_p = by_xcd ? total_wg / 8 : total_wg;  // workgroups dealing out one partition
  const int sched_x = logical / sched_p, sched_w = logical - sched_x * sched_p;
  const int slabs_here = by_xcd ? n_slabs / 8 : n_slabs;
  const int rank = rnd * sched_p + ((rnd & 1) ? sched_p - 1 - sched_w : sched_w);
  if (rank >= slabs_here * nqb_all) return 0;
  const int level = rank / slabs_here, j = rank - level * slabs_here;
  const int slab = by_xcd ? sched_x + 8 * j : j;
  b = slab / Hkv;
  g = slab - b * Hkv;
  M = ap->M_all;
  int nqb = nqb_all;
  if (ap->m_dev != nullptr) {  // this row's kept length (M_all is the padded length)
    M = min(max(ap->m_dev[b], 0), M);
    nqb = (M + BQ - 1) / BQ;
  }
  if (level >= nqb) return 1;
  qb = nqb - 1 - level;
  return 2;
}

// The (cos, sin) pieces of one lane's query fragments from the angle table
// (rope_tab_piece's layout): slot0 = the wave's first query slot (a multiple
// of 32), rt[ks][u] covers pairs 16 ks + 8 gq + 2u and + 1 of query slot0 +
// (lane & 31).  Every load reads 1 KiB contiguous.
template <int DH>
__device__ __forceinline__ void load_rope_row(const float* tab, size_t slot0, int lane, f32x4 (&rt)[DH / 32][4]) {
  const f32x4* tb = reinterpret_cast<const f32x4*>(tab) + (slot0 >> 5) * (DH / 32) * 4 * 64 + lane;
#pragma unroll
  for (int ks = 0; ks < DH / 32; ++ks)
#pragma unroll
    for (int u = 0; u < 4; ++u) rt[ks][u] = tb[(ks * 4 + u) * 64];
}

// ROPE: the Q fragments are rotated by the prepass's angle table after they
// land (the plain instance carries none of that code or its registers).
template <int DH, int G, bool VARLEN, bool ROPE>
__global__ __launch_bounds__(kAttnThreads, 1) void gated_attn_kernel(const AttnArgs args, const SeqTable st) {
  (void)args;  // read through the argument segment below (it is the first argument)
  const AttnArgsPtr args_seg = (AttnArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int RG = 4 / G;        // 32-row groups per head
  constexpr int BQ = 32 * RG;      // query rows per workgroup
  constexpr int KS = DH / 16;      // k-steps of S^T = K Q^T
  constexpr int DT = DH / 32;      // 32-row tiles of O^T
  constexpr int KROW = DH * 2;      // bytes of a K row in LDS (unpadded, swizzled)
  constexpr int KCH = DH / 8;       // its 16-byte chunks
  // LDS swizzles: row r of a tile holds its 16-byte chunk u at position
  // u ^ h(r).  With h = r & 7 the fragment reads (32 rows x 2 chunks per
  // MFMA) conflict 2-way on gfx950; folding row bit 3 in removes that: into
  // chunk bit 3 for 256-byte K rows (h = r & 15), into chunk bit 0 for
  // 128-byte rows (V^T, and K at DH = 64).
  auto swz_k = [](int r) { return DH == 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1)); };
  auto swz_v = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
  constexpr int VROW = kBK * 2;     // bytes of a V^T row (64 keys, fp16)
  constexpr int TILE = kBK * DH * 2;           // bytes of a K tile = bytes of a V^T tile
  constexpr int NI = TILE / 1024 / 4;          // 1 KiB loads per wave per tile, for each of K and V^T
  constexpr int BIAS = (G + 1) * kBK * 4;      // bytes of a key-score tile (G heads, then the V^T scale row)
  constexpr int V_BASE = 2 * kGroups * TILE, B_BASE = 4 * kGroups * TILE;
  constexpr int LDS_BYTES = B_BASE + 3 * kGroups * BIAS;
  static_assert(NI >= 1 && NI * 4 * 1024 == TILE, "tile shape");


  // [buf][group] K tiles, then [buf][group] V^T tiles, then [buf][group][head] key-score tiles
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

  // This lane's Q fragments and the original position of its query.  The
  // next block's are requested as soon as the current block has written its
  // output (they then belong to round pre_round).
  bf16x8 qf[DH / 16];
  int p_pre = 0, pre_round = -1;
  for (int round = 0;; ++round) {
  // Every value of the block is derived afresh inside the loop (the thread
  // index and the argument segment pass through empty asm statements), so
  // nothing is hoisted out of it and kept live across the whole block.
  unsigned tix = threadIdx.x;
  asm volatile("" : "+v"(tix));
  const int lane = tix & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tix >> 6);  // wave-uniform: branches stay scalar
  const int grp = wall >> 2;       // key-range group of this wave
  const int wid = wall & 3;        // wave index inside the group
  const int tid = tix & (kThreads - 1);  // thread index inside the group
  AttnArgsPtr ap = args_seg;
  asm volatile("" : "+s"(ap));  // reload the arguments for this block
  const uint16_t* __restrict__ q = ap->q;
  const uint16_t* __restrict__ k = ap->k;
  const uint16_t* __restrict__ vt = ap->vt;
  const float* __restrict__ kbias = ap->kbias;
  const int32_t* __restrict__ pos = ap->pos;
  const float* __restrict__ temp = ap->temp;
  uint16_t* __restrict__ out = ap->out;
  float* __restrict__ lse = ap->lse;
  const int32_t* __restrict__ m_dev = ap->m_dev;
  const int M_all = ap->M_all, Mp_all = ap->Mp_all, Hq = ap->Hq, Hkv = ap->Hkv, nqb_all = ap->nqb_all;
  const int total_wg = ap->total_wg, n_slabs = ap->n_slabs;
  const float sm_scale = ap->sm_scale;
  // this block's sequence (its length M, first packed row T0, first padded
  // key slot P0), KV head g and query block qb
  int M, Mp, g, qb;
  size_t T0, P0;
  int item;  // a unique id of the block (timeline of the counting build)
  if constexpr (VARLEN) {
    if (round > 0) break;
    const int logical = xcd_logical_id(blockIdx.x, total_wg);
    const int sq = seq_of(st.wg0, st.n, logical);
    M = st.m[sq];
    Mp = (M + kBK - 1) / kBK * kBK;
    const int nqb = (M + BQ - 1) / BQ, local = logical - st.wg0[sq];
    g = local / nqb;
    qb = nqb - 1 - (local - g * nqb);
    T0 = (size_t)st.t0[sq];
    P0 = (size_t)st.p0[sq];
    item = logical;
  } else {
    int b;
    const int st_b = sched_block<BQ>(ap, round, b, g, qb, M);
    if (st_b == 0) break;
    if (st_b == 1) continue;  // (the whole workgroup)
    Mp = Mp_all;
    T0 = (size_t)b * M_all;
    P0 = (size_t)b * Mp;
    item = (b * Hkv + g) * nqb_all + qb;
  }
  if (round > 0) __syncthreads();  // every wave is done with the previous block's LDS
  const int lse_ld = VARLEN ? M : M_all;  // lse rows: [Hq, M] per sequence, [Hq, M_all] per batch row
#ifdef TG_DIAG_COUNTERS
  unsigned long long diag_t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  unsigned long long diag_p[4] = {0, 0, 0, 0};
  diag_t[0] = (unsigned long long)blockIdx.x | ((unsigned long long)(unsigned)qb << 32);
  diag_t[7] = (unsigned long long)(unsigned)round;
#endif
  TG_DIAG_STAMP(1);
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
      const_cast<float*>(kbias + P0 * (Hq + Hkv) + (size_t)g * (G + 1) * Mp), (short)0, (G + 1) * Mp * 4,
      kBufferConfig);
  // Load e of this wave fills LDS bytes [1024 C, 1024 C + 1024) of the tile,
  // C = wid * NI + e: 16-byte slot Y = 64 C + lane sits at row Y / chunks-per-row,
  // position p, and holds chunk p ^ (row & 7) of that row.
  int k_off[NI], v_off[NI];
#pragma unroll
  for (int e = 0; e < NI; ++e) {
    const int Y = (wid * NI + e) * 64 + lane;
    const int kr = Y / KCH, kc = (Y % KCH) ^ swz_k(kr);
    k_off[e] = kr * Hkv * DH * 2 + kc * 16;
    const int vr = Y / (VROW / 16), vc = (Y % (VROW / 16)) ^ swz_v(vr);
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
    const int soff = (grp + kGroups * t) * kBK * 4;
    if (wid < G)  // one 256-byte row per query head
      buffer_load4_to_lds(b_rsrc, b_tile(t % 3) + wid * kBK, (wid * Mp + lane) * 4, soff);
    if (wid == G % 4)  // and the tile's V^T scale row
      buffer_load4_to_lds(b_rsrc, b_tile(t % 3) + G * kBK, (G * Mp + lane) * 4, soff);
  };
  // this lane's fragment chunks: K row ql (and ql + 32) chunk 2ks + gq; V^T row
  // 32t + ql chunk 2st + gq -- both swizzled by ql & 7
  const int q7 = ql & 7;
  auto k_frag_off = [&](int ks) { return ql * KROW + (((2 * ks + gq) ^ swz_k(ql)) << 4); };
  auto v_frag_off = [&](int st) { return ql * VROW + (((2 * st + gq) ^ swz_v(ql)) << 4); };

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
  // (Every fragment read of qk and pv is issued before the first product:
  // read-then-use per product left one LDS latency exposed per MFMA in the
  // steps outside the steady loop.)
  auto qk = [&](int h, f32x16& s) __attribute__((always_inline)) {
    const unsigned char* kt = k_tile((h >> 1) & 1) + (h & 1) * 32 * KROW;
    bf16x8 ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(kt + k_frag_off(ks));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(ka[ks]));  // all reads issued, then one wait
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s, 0, 0, 0);
  };
  // O^T += V^T P^T over the two 16-key steps of half h
  auto pv = [&](int h, const uint32_t (&pk)[8]) __attribute__((always_inline)) {
    const unsigned char* vt_l = v_tile((h >> 1) & 1);
    u32x4 vw[2][DT];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
      for (int t = 0; t < DT; ++t)
        vw[sh][t] = *reinterpret_cast<const u32x4*>(vt_l + t * 32 * VROW + v_frag_off((h & 1) * 2 + sh));
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
      for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(vw[sh][t]));
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      const u32x4 pw = {pk[sh * 4], pk[sh * 4 + 1], pk[sh * 4 + 2], pk[sh * 4 + 3]};
      const f16x8 pf = as_f16x8(pw);
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vw[sh][t]), pf, o[t], 0, 0, 0);
    }
  };
  // Online softmax of half h's scores, without branches: the running max
  // moves by a select, and the accumulator rescale this implies is left to
  // the caller, which applies `alpha` after the P.V products issued before
  // it.  `diag`: keys after the lane's query are masked.
  auto softmax = [&](int h, f32x16& s, bool diag, uint32_t (&pk)[8], bool& resc,
                     float& alpha) __attribute__((always_inline)) {
    const float* bt = b_tile((h >> 1) % 3) + hloc * kBK + (h & 1) * 32 + gq * 4;
    const float sc = b_tile((h >> 1) % 3)[G * kBK];  // the tile's V^T scale 2^e
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
    if (resc && m_run != -INFINITY) TG_DIAG_HIT(1);
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
    l_run = fmaf(l0 + l1, sc, l_run * alpha);
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
  // c = q7 >> 1, e = q7 & 1 and b3 = bit 3 of ql, V^T chunk (2j + gq) ^ swz_v(ql)
  // = 2 (j ^ c) + (gq ^ e ^ b3), so V^T step st sits at v_lane[st].  K chunk
  // (2 ks + gq) ^ swz_k(ql) adds 8 ((ks >> 2) ^ b3) at DH = 128: k_lane[j]
  // holds the b3 term, whose 128-byte bit is the only set bit 7 of the
  // offset, so k-step ks sits at k_lane[ks & 3] ^ (128 (ks >> 2)).  Ring slot
  // and half tile only add constants.
  int k_lane[4], v_lane[4];
  const int b3 = (ql >> 3) & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int swv = 32 * (j ^ (q7 >> 1)) + 16 * (gq ^ (q7 & 1) ^ b3);
    const int swk = DH == 128 ? 32 * (j ^ (q7 >> 1)) + 16 * (gq ^ (q7 & 1)) + 128 * b3 : swv;
    k_lane[j] = grp * TILE + ql * KROW + swk;
    v_lane[j] = V_BASE + grp * TILE + ql * VROW + swv;
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
    const float sc = b_tile((h >> 1) % 3)[G * kBK];  // the tile's V^T scale 2^e
    u32x4 fr[NS];
    auto read_frag = [&](int r) __attribute__((always_inline)) {
      if (r & 1) {
        const int p = r >> 1;
        fr[r] = *reinterpret_cast<const u32x4*>(smem + vb[2 * SB + p / DT] + (p % DT) * 32 * VROW);
      } else {
        const int ks = r >> 1;
        fr[r] = *reinterpret_cast<const u32x4*>(smem + (kb[ks & 3] ^ (128 * (ks >> 2))) + SB * 32 * KROW);
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
          l_run = fmaf(l, sc, l_prev);
          asm volatile("" ::"v"(l_run));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ovf) {
      // some numerator left the safe range: move the reference up to the
      // row's true max and redo this half's numerators
      TG_DIAG_HIT(0);
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
      l_run = fmaf(l2, sc, l_prev * alpha);
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
  TG_DIAG_PSTAMP(0);
  if (t_exists(0)) {
    issue_k(0);
    issue_b(0);
  }
  // Q fragments and the original position are requested while the first
  // tile is in flight (unless the previous block requested them); one wait
  // covers all of them
  int p_orig = p_pre;
  if (pre_round != round) {
    const uint16_t* qp = q + ((T0 + (q_ok ? qi : 0)) * Hq + hq) * DH + gq * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(q_ok ? load16(qp + ks * 16) : u32x4{0, 0, 0, 0});
    p_orig = pos[T0 + (q_ok ? qi : 0)];
  }
  const float t_h = temp[hq];
  // rotary embedding: this lane's fragments ks and ks + KS/2 hold the pairs
  // (x_i, x_{i + DH/2}), i = 16 ks + 8 gq + e; their cosines and sines come
  // from the prepass's table of this query's slot (held only in the prologue:
  // a copy carried over from the previous block would not fit the registers)
  f32x4 rt[KS / 2][4];
  if constexpr (ROPE) {
    if (wave_rows) {  // (the wave's 32 slots lie inside the sequence's padded slots)
      load_rope_row<DH>(ap->rope_tab, P0 + rbase, lane, rt);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int u = 0; u < 4; ++u) rt[ks][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  wait_vmem();
  TG_DIAG_PSTAMP(1);
  if constexpr (ROPE) {  // exactly the prepass's rotation of k: fused fp32 products, bf16 nearest even
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      const u32x4 a = __builtin_bit_cast(u32x4, qf[ks]), bv = __builtin_bit_cast(u32x4, qf[ks + KS / 2]);
      u32x4 oa, ob;
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // word j: elements e = 2j (low half) and 2j + 1 (high half)
        const float cl = rt[ks][j][0], sl = rt[ks][j][1], ch = rt[ks][j][2], sh = rt[ks][j][3];
        const float x1l = bf16_lo(a[j]), x1h = bf16_hi(a[j]), x2l = bf16_lo(bv[j]), x2h = bf16_hi(bv[j]);
        oa[j] = pack_bf16x2(fmaf(x1l, cl, -(x2l * sl)), fmaf(x1h, ch, -(x2h * sh)));
        ob[j] = pack_bf16x2(fmaf(x2l, cl, x1l * sl), fmaf(x2h, ch, x1h * sh));
      }
      qf[ks] = as_bf16x8(oa);
      qf[ks + KS / 2] = as_bf16x8(ob);
    }
  }
  if (q_ok) {
    float ratio = 1.0f;
    if (p_orig != qi) ratio = logf((float)max(p_orig + 1, 2)) / logf((float)max(qi + 1, 2));
    cq = sm_scale * kLog2e / (t_h * ratio);
  }
  __syncthreads();
  TG_DIAG_STAMP(2);
  if (t_exists(1)) {
    issue_k(1);
    issue_b(1);
  }
  if (t_exists(0)) issue_v(0);
  f32x16 sa, sb;
  uint32_t pa[8], pb[8];
  if (h_mine(0)) qk(0, sa);
  step(0, sa, sb, pa, pb);  // no P.V yet: half -1 is never computed
  TG_DIAG_PSTAMP(2);
  wait_vmem();
  TG_DIAG_PSTAMP(3);
  __syncthreads();
  TG_DIAG_STAMP(3);
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
    TG_DIAG_STAMP(4);
    // leave it: the pending scores go back to the plain form
#pragma unroll
    for (int e = 0; e < 16; ++e) sb[e] -= cm[e];
  }
  // The next block's schedule and the offsets of its Q fragments and
  // position (scalar reads from the argument segment), taken before the
  // tail iterations so that their latency passes under them; the loads
  // themselves wait until this block's last scores are computed.
  // Unconditional loads through a range-checked resource: a row past the
  // kept length (or no next block) reads zeros, with no select.  The
  // fragments then load straight into the registers they live in; a
  // conditional load (zero default, then a masked load) made the compiler
  // copy them over and wait for the loads, which exposed their whole
  // latency at every block transition.
  __amdgpu_buffer_rsrc_t q_rsrc_n;
  int q_off_n = 0;
  const int32_t* pos_n = nullptr;
  bool has_next = false;
  if constexpr (!VARLEN) {
    AttnArgsPtr an = args_seg;
    asm volatile("" : "+s"(an));
    int b_n = 0, g_n = 0, qb_n = 0, M_n = 0;
    has_next = sched_block<BQ>(an, round + 1, b_n, g_n, qb_n, M_n) == 2;
    const int qi_n = qb_n * BQ + (wid % RG) * 32 + ql;
    const bool ok = has_next && qi_n < M_n;
    pos_n = an->pos + (size_t)b_n * an->M_all + (ok ? qi_n : 0);
    const uint16_t* qbase = an->q + (size_t)b_n * an->M_all * an->Hq * DH;
    q_rsrc_n = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qbase), (short)0,
                                                 (int)((size_t)M_n * an->Hq * DH * 2), kBufferConfig);
    q_off_n = ok ? (int)(((size_t)qi_n * an->Hq + g_n * G + hloc) * DH * 2 + gq * 16) : (int)0x7FFFFFF0;
  }
  for (; i < nit; ++i) {
    stage(i);
    step(2 * i + 1, sb, sa, pb, pa);
    step(2 * i + 2, sa, sb, pa, pb);
    wait_vmem();
    __syncthreads();
  }
  TG_DIAG_STAMP(5);
  if constexpr (!VARLEN) {
    // request the next block's Q fragments and position now (this block's
    // scores are all done, so its Q fragments are free): they land while the
    // groups merge, the output is written and the next block sets up
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc_n, q_off_n, ks * 32, 0)));
    p_pre = *pos_n;
    pre_round = has_next ? round + 1 : -1;
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
    const float inv = 1.0f / l_tot;
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
      lse[T0 * Hq + (size_t)hq * lse_ld + qi] = (m_run + __log2f(l_tot)) * kLn2;
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

#ifdef TG_DIAG_COUNTERS
  TG_DIAG_STAMP(6);
  if (tix == 0 && item < kDiagWG) {
    for (int k = 0; k < 8; ++k) g_diag_wg[item][k] = diag_t[k];
    for (int k = 0; k < 4; ++k) g_diag_pro[item][k] = diag_p[k];
  }
#endif
  }  // the next block of this workgroup
}


template <int DH, int G>
hipError_t launch_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq, int Hkv,
                    const float* ks, const int32_t* pos, const float* gain, const float* temp, float sm_scale,
                    uint16_t* out, float* lse, uint16_t* vt, float* kbias, const RopeArgs* rope, hipStream_t s,
                    const int32_t* m_dev) {
  constexpr int BQ = 32 * (4 / G);
  const int Mp = (M + kBK - 1) / kBK * kBK;
  if (rope != nullptr) {
    hipLaunchKernelGGL((attn_prepass_kernel<DH, true, false>), dim3(Mp / kBK, Hkv, B), dim3(kPreThreads<DH>), 0, s, v, ks,
                       gain, M, Mp, Hkv, G, vt, kbias, *rope, SeqTable{}, m_dev);
    k = rope->kr;  // the main kernel reads the rotated k and rotates its Q fragments itself
  } else {
    hipLaunchKernelGGL((attn_prepass_kernel<DH, false, false>), dim3(Mp / kBK, Hkv, B), dim3(kPreThreads<DH>), 0, s, v, ks,
                       gain, M, Mp, Hkv, G, vt, kbias, RopeArgs{}, SeqTable{}, m_dev);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (M + BQ - 1) / BQ;
  const long long total = (long long)nqb * Hkv * B;
  if (total <= 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  // a persistent grid of one workgroup per CU (each holds a CU's LDS)
  const int grid = (int)std::min<long long>(total, device_cu_count());
  const AttnArgs a{q,   k,   vt,  kbias, pos,  temp,     out, lse, m_dev, rope != nullptr ? rope->tab : nullptr,
                   M,   Mp,  Hq,  Hkv,   nqb,  grid,     Hkv * B,  sm_scale};
  if (rope != nullptr)
    hipLaunchKernelGGL((gated_attn_kernel<DH, G, false, true>), dim3((unsigned)grid), dim3(kAttnThreads), 0, s, a,
                       SeqTable{});
  else
    hipLaunchKernelGGL((gated_attn_kernel<DH, G, false, false>), dim3((unsigned)grid), dim3(kAttnThreads), 0, s, a,
                       SeqTable{});
  return hipGetLastError();
}

// One prepass and one attention launch over the sequences of a table.
template <int DH, int G>
hipError_t launch_varlen_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, const SeqTable& st, int Hq,
                           int Hkv, const float* ks, const int32_t* pos, const float* gain, const float* temp,
                           float sm_scale, uint16_t* out, float* lse, uint16_t* vt, float* kbias,
                           const RopeArgs* rope, hipStream_t s) {
  if (rope != nullptr) {
    hipLaunchKernelGGL((attn_prepass_kernel<DH, true, true>), dim3((unsigned)st.pb0[st.n], Hkv, 1), dim3(kPreThreads<DH>),
                       0, s, v, ks, gain, 0, 0, Hkv, G, vt, kbias, *rope, st, nullptr);
    k = rope->kr;
  } else {
    hipLaunchKernelGGL((attn_prepass_kernel<DH, false, true>), dim3((unsigned)st.pb0[st.n], Hkv, 1), dim3(kPreThreads<DH>),
                       0, s, v, ks, gain, 0, 0, Hkv, G, vt, kbias, RopeArgs{}, st, nullptr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = st.wg0[st.n];
  const AttnArgs a{q, k, vt, kbias, pos, temp, out, lse, nullptr, rope != nullptr ? rope->tab : nullptr,
                   0, 0, Hq, Hkv, 0, total, 0, sm_scale};
  if (rope != nullptr)
    hipLaunchKernelGGL((gated_attn_kernel<DH, G, true, true>), dim3((unsigned)total), dim3(kAttnThreads), 0, s, a, st);
  else
    hipLaunchKernelGGL((gated_attn_kernel<DH, G, true, false>), dim3((unsigned)total), dim3(kAttnThreads), 0, s, a,
                       st);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// fp16 V^T [B, Hkv, dh, Mp], then the fp32 key-score rows [B, Hkv, G + 1, Mp]
size_t gated_attention_workspace(int B, int M, int Hq, int Hkv, int dh) {
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  return (size_t)B * Mp * ((size_t)Hkv * dh * 2 + (size_t)(Hq + Hkv) * 4);
}

// ... then the rotated k [B, M, Hkv, dh] (bf16) and the angle table, dh / 2
// (cos, sin) pairs of every padded slot [B, Mp] (fp32)
size_t gated_attention_rope_workspace(int B, int M, int Hq, int Hkv, int dh) {
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  return gated_attention_workspace(B, M, Hq, Hkv, dh) + (size_t)B * M * dh * Hkv * 2 + (size_t)B * Mp * dh * 4;
}

// the varying-length rotary call: after the other workspace (slots padded
// rows), the rotated k of the T packed rows and the angle table of the slots
size_t gated_attention_rope_varlen_workspace(int B, const int32_t* cu_seqlens, int Hq, int Hkv, int dh) {
  const size_t slots = gated_attention_varlen_slots(B, cu_seqlens);
  return gated_attention_workspace(1, (int)slots, Hq, Hkv, dh) + (size_t)cu_seqlens[B] * dh * Hkv * 2 +
         slots * dh * 4;
}

size_t gated_attention_varlen_slots(int B, const int32_t* cu_seqlens) {
  size_t slots = 0;
  for (int b = 0; b < B; ++b) slots += (size_t)(cu_seqlens[b + 1] - cu_seqlens[b] + kBK - 1) / kBK * kBK;
  return slots;
}

hipError_t launch_gated_attention_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B,
                                         const int32_t* cu_seqlens, int Hq, int Hkv, int dh, const float* key_score,
                                         const int32_t* pos, const float* gain, const float* temp, float sm_scale,
                                         double rope_base, uint16_t* out, float* lse, void* ws, hipStream_t s) {
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
  RopeArgs ra{};
  const RopeArgs* rope = nullptr;
  if (rope_base > 0.0) {  // rotated k and the angle table, by packed row, after the other workspace
    unsigned char* rw = static_cast<unsigned char*>(ws) + gated_attention_workspace(1, (int)slots, Hq, Hkv, dh);
    const size_t T = (size_t)cu_seqlens[B];
    uint16_t* kr = reinterpret_cast<uint16_t*>(rw);
    ra = RopeArgs{k, pos, rope_base, reinterpret_cast<float*>(kr + T * Hkv * dh), kr};
    rope = &ra;
  }
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
                                 rope, s);
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
                                  void* ws, hipStream_t s, const int32_t* m_dev) {
  const int G = Hq / Hkv;
  const size_t Mp = (size_t)(M + kBK - 1) / kBK * kBK;
  uint16_t* vt = static_cast<uint16_t*>(ws);
  float* kbias = reinterpret_cast<float*>(vt + (size_t)B * Hkv * dh * Mp);
  RopeArgs ra{};
  const RopeArgs* rope = nullptr;
  if (rope_base > 0.0) {  // rotated k, then the angle table
    uint16_t* kr = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(ws) +
                                               gated_attention_workspace(B, M, Hq, Hkv, dh));
    ra = RopeArgs{k, pos, rope_base, reinterpret_cast<float*>(kr + (size_t)B * M * Hkv * dh), kr};
    rope = &ra;
  }
#define TG_ATTN_CASE(DHV, GV)                                                                                   \
  if (dh == DHV && G == GV)                                                                                     \
    return launch_t<DHV, GV>(q, k, v, B, M, Hq, Hkv, key_score, pos, gain, temp, sm_scale, out, lse, vt, kbias, \
                             rope, s, m_dev);
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

#ifdef TG_DIAG_COUNTERS
// Reads (and with reset != 0 clears) the rare-path counters of the test
// build on the current device.  Not part of the library's interface.
extern "C" int tg_diag_attention_timeline(unsigned long long* out, int n_wg) {
  if (n_wg < 0 || n_wg > tg::kDiagWG) return 1;
  return hipMemcpyFromSymbol(out, HIP_SYMBOL(tg::g_diag_wg), (size_t)n_wg * 8 * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : 3;
}

extern "C" int tg_diag_attention_prologue(unsigned long long* out, int n_wg) {
  if (n_wg < 0 || n_wg > tg::kDiagWG) return 1;
  return hipMemcpyFromSymbol(out, HIP_SYMBOL(tg::g_diag_pro), (size_t)n_wg * 4 * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : 3;
}

extern "C" int tg_diag_attention_counters(unsigned long long* out4, int reset) {
  if (hipMemcpyFromSymbol(out4, HIP_SYMBOL(tg::g_diag_count), 4 * sizeof(unsigned long long), 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return 3;
  if (reset) {
    const unsigned long long zero[4] = {0, 0, 0, 0};
    if (hipMemcpyToSymbol(HIP_SYMBOL(tg::g_diag_count), zero, sizeof(zero), 0, hipMemcpyHostToDevice) != hipSuccess)
      return 3;
  }
  return 0;
}
#endif
