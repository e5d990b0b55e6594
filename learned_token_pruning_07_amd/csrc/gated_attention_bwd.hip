// Backward of token-gated causal GQA attention (TokenGate paper, Section 4:
// token-gated attention, Eq. 8).  The key score b_j enters every logit of
// key j through gain_h * b_j; that term is the gradient path that trains the
// scorer although the top-K selection itself has no gradient.  The per-head
// gain and the temperature are trainable scale factors too ("Putting
// everything together").
//
// With c_i = sm_scale / (temp_h ratio_i), z_ij = (q_i . k_j) c_i + gain_h b_j
// (j <= i), P = exp(z - lse) and the upstream gradient dO:
//   D_i   = dO_i . O_i,   dZ_ij = P_ij (dO_i . v_j - D_i)
//   dq_i  = c_i sum_j dZ_ij k_j
//   dk_j  = sum_{h in group, i} c_i dZ_ij q_i,   dv_j = sum_{h in group, i} P_ij dO_i
//   db_j  = sum_h gain_h sum_i dZ_{h,ij}
//   dgain_h = sum_{b,i,j} dZ_{h,ij} b_j,   dtemp_h = -(1/temp_h) sum_{b,i,j} dZ_{h,ij} (q_i . k_j) c_i
//
// Four kernels on one stream, all bf16 MFMA 32x32x16 with fp32 accumulation:
//  * bwd_rows: per query row and head, D_i and the exponent constants
//    c_i log2(e) and lse_i log2(e) (+inf beyond M, so padded rows get P = 0).
//  * bwd_dkdv: a workgroup owns 64 keys of one KV head, keeps their K and V
//    fragments in registers and walks every 32-query tile of each of the G
//    query heads from the diagonal down.  S = Q K^T and dP = dO V^T come out
//    with one lane per key, so P and dS = dZ c are at once the B fragments of
//    dV^T += dO^T P and dK^T += Q^T dS; their A fragments (dO^T, Q^T) are read
//    from the row-major tiles with the LDS transpose load (ds_read_b64_tr_b16:
//    a 16-lane group whose lanes point at 4 rows x 4 consecutive columns gets,
//    per lane, one column's 4 rows).  An accumulator hands a lane the rows
//    {4 gq .. 4 gq + 3, 8 + 4 gq .. 8 + 4 gq + 3} of each 16-wide k-step, so
//    the two transpose loads of an A fragment start at rows 4 gq and 8 + 4 gq.
//    Four waves: two key halves x two query-tile parities, merged through LDS
//    at the end.  The lane's running column sums of dZ give the key-score,
//    gain and temperature partials.
//  * bwd_dq: a workgroup owns 32 (4/G) query rows of each of the G heads,
//    keeps their Q and dO fragments in registers and walks the 32-key tiles
//    up to the diagonal.  S^T = K Q^T and dP^T = V dO^T come out with one
//    lane per query, so dZ^T is the B fragment of dQ^T += K^T dZ^T (K^T again
//    by transpose loads) and c_i is applied once at the end.
//  * bwd_reduce: db as the sum of the per-KV-head partials, dgain and dtemp
//    as fixed-order sums of the per-block partials.  No atomics anywhere:
//    the results are deterministic.
// Tiles travel global -> LDS by buffer loads with the LDS-destination bit
// into three-slot rings: the loads of step p + 2 are issued, between the
// first and the second products of step p, while the matrix cores work.
#include <math.h>

#include <algorithm>
#include <vector>

#include "rope_device.h"
#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kPB = 64;   // rows per prepass block (Mp is a multiple of it)
constexpr int kKB = 64;   // keys per dK/dV workgroup
constexpr int kT = 32;    // queries per dK/dV tile, keys per dQ tile
constexpr int kRsrcCfg = 0x00020000;  // raw buffer resource word 3 (gfx9 family, 32-bit data)

size_t base_ws_bytes(int B, int M, int Hq, int Hkv) {
  const size_t Mp = (size_t)(M + kPB - 1) / kPB * kPB;
  return (size_t)B * Mp * ((size_t)3 * Hq * 4 + (size_t)Hkv * 4) + (size_t)2 * B * (Mp / kKB) * Hq * 4;
}
// where the rotary variant's buffers start in the workspace
size_t rope_ws_offset(int B, int M, int Hq, int Hkv, int dh) {
  (void)dh;
  return (base_ws_bytes(B, M, Hq, Hkv) + 15) / 16 * 16;
}
size_t rope_varlen_ws_offset(int B, const int32_t* cu_seqlens, int Hq, int Hkv) {
  return (gated_attention_backward_varlen_workspace(B, cu_seqlens, Hq, Hkv) + 15) / 16 * 16;
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}
// s_waitcnt vmcnt(0): every load of this wave, LDS-destination ones included
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, kRsrcCfg);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 lds_frag(const unsigned char* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  return as_bf16x8(w);
}

// Four consecutive results at element idx of a bf16 (nearest even) or fp32 output.
template <bool F32>
__device__ __forceinline__ void store4(void* base, size_t idx, float a, float b, float c, float d) {
  if constexpr (F32)
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = f32x4{a, b, c, d};
  else
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// Row r of a staged [32 rows x DH] bf16 tile holds its 16-byte chunk c at
// position c ^ tile_swz(r).  gfx950 serves 16 lanes of an LDS read per
// cycle from 64 four-byte banks (a 256-byte period), so a read is
// conflict-free when those 16 lanes cover distinct banks.  The fragment
// reads (16 rows, one chunk each) need tile_swz to be one-to-one on r mod 16
// (on each parity of r for 128-byte rows); the transpose loads (4 rows x 32
// bytes per 16 lanes) need tile_swz(r) >> 1 to differ within every aligned
// group of 4 rows (of 2 same-parity rows for 128-byte rows).  r & 7 met
// neither at DH = 128 (both reads conflicted 2-way).
template <int DH>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (DH == 128) return ((r >> 2) & 1) | ((r & 3) << 1) | (r & 8);  // bits b2 b0 b1 b3
  else return (r & 7) ^ ((r >> 3) & 1);
}
// The byte-offset bit holding the chunk bit that row bit 3 flips (chunk bit
// 3 at DH = 128, chunk bit 0 at DH = 64): rows r and r + 8 of the same lane
// differ in their offsets by 8 rows and this bit.
template <int DH>
constexpr int kRow8Flip = DH == 128 ? 128 : 16;

// Byte offset, inside a staged [32 rows x DH] bf16 tile, of row r's 16-byte chunk c.
template <int DH>
__device__ __forceinline__ int row_tile_off(int r, int c) {
  return r * (2 * DH) + ((c ^ tile_swz<DH>(r)) << 4);
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// A fragment of X^T (rows d = 32 blk + (lane & 31), k = 16 tile rows) from a
// staged row-major [32 x DH] tile X: two transpose loads, rows
// 16 s + 4 gq + {0..3} then 16 s + 8 + 4 gq + {0..3} (the accumulator order
// of the B fragment it meets).  Lane j of each 16-lane group points at row
// base + (j >> 2), columns c0 + 4 (j & 3) .. + 3.
template <int DH>
__device__ __forceinline__ int tr_off(int blk, int s, int hf, int lane) {
  const int j = lane & 15, gq = lane >> 5;
  const int col = 32 * blk + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int row = 16 * s + 8 * hf + 4 * gq + (j >> 2);
  return row * (2 * DH) + (((col >> 3) ^ tile_swz<DH>(row)) << 4) + (((col >> 2) & 1) << 3);
}
// the same fragment from precomputed offsets (tr_off of hf = 0 and 1)
__device__ __forceinline__ bf16x8 tr_frag_at(const unsigned char* tile, int off0, int off1) {
  const v4s h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(tile + off0));
  const v4s h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(tile + off1));
  const u32x4 w = {__builtin_bit_cast(u32x2, h0)[0], __builtin_bit_cast(u32x2, h0)[1],
                   __builtin_bit_cast(u32x2, h1)[0], __builtin_bit_cast(u32x2, h1)[1]};
  return as_bf16x8(w);
}
template <int DH>
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* tile, int blk, int s, int lane) {
  v4s h[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    h[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(tile + tr_off<DH>(blk, s, hf, lane)));
  const u32x4 w = {__builtin_bit_cast(u32x2, h[0])[0], __builtin_bit_cast(u32x2, h[0])[1],
                   __builtin_bit_cast(u32x2, h[1])[0], __builtin_bit_cast(u32x2, h[1])[1]};
  return as_bf16x8(w);
}

// s_waitcnt vmcnt(N): at most N loads of this wave still in flight (loads
// complete in issue order)
template <int N>
__device__ __forceinline__ void wait_loads_le() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Stages `n` 1 KiB DMA loads of a [32 x DH] row-major tile: load e fills LDS
// slots 64 e + lane, slot Y holding row Y / (DH/8), chunk (Y % (DH/8)) ^ tile_swz(row).
template <int DH>
__device__ __forceinline__ void stage_rows(__amdgpu_buffer_rsrc_t r, unsigned char* tile, int row_bytes, int e,
                                           int lane) {
  constexpr int CH = DH / 8;
  const int Y = e * 64 + lane;
  const int row = Y / CH, c = (Y % CH) ^ tile_swz<DH>(row);
  dma16(r, tile + e * 1024, row * row_bytes + c * 16, 0);
}

// Sequences of one varying-length backward launch (longest first; empty ones
// take no work).  Sequence s owns packed rows t0[s] .. t0[s] + m[s] - 1,
// padded row slots p0[s] .. p0[s] + roundup(m[s], 64) - 1 of the row
// constants and partials, 64-row blocks pb0[s] .. pb0[s+1] - 1 (the rows
// kernel; the dK/dV workgroups are Hkv per block), dQ workgroups qb0[s] ..
// qb0[s+1] - 1, and row out_row[s] of the gain and temperature gradients.
// n = 0: an equal-length batch, indexed by the grid's batch coordinate.
constexpr int kMaxBwdSeqs = 64;
struct BwdSeqTable {
  int n;
  int t0[kMaxBwdSeqs];
  int m[kMaxBwdSeqs];
  int p0[kMaxBwdSeqs];
  int out_row[kMaxBwdSeqs];
  int pb0[kMaxBwdSeqs + 1];
  int qb0[kMaxBwdSeqs + 1];
};

// ---------------------------------------------------------------------------
// Per (query row, head): D_i = dO_i . O_i (fp32, fixed order: four threads per
// row), c_i log2(e), lse_i log2(e); rows M .. Mp-1 get 0, +inf, 0.
template <int DH>
__global__ __launch_bounds__(kBwdThreads) void bwd_rows_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const int32_t* __restrict__ pos, const float* __restrict__ temp, float sm_scale, int M_all, int Mp_all, int Hq,
    float* __restrict__ rowc, float* __restrict__ rowl, float* __restrict__ rowD, const BwdSeqTable st) {
  const int h = blockIdx.y;
  int M = M_all, Mp = Mp_all, blk = blockIdx.x;
  size_t T0 = (size_t)blockIdx.z * M_all, P0 = (size_t)blockIdx.z * Mp_all;
  if (st.n > 0) {
    const int sq = seq_of(st.pb0, st.n, blockIdx.x);
    M = st.m[sq];
    Mp = (M + kPB - 1) / kPB * kPB;
    blk = blockIdx.x - st.pb0[sq];
    T0 = (size_t)st.t0[sq];
    P0 = (size_t)st.p0[sq];
  }
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int i = blk * kPB + r;
  float acc = 0.0f;
  if (i < M) {
    const size_t off = ((T0 + i) * Hq + h) * DH + part * (DH / 4);
#pragma unroll
    for (int c = 0; c < DH / 32; ++c) {
      const u32x4 ov = load16(o + off + c * 8), dv = load16(dout + off + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf16_lo(ov[e]), bf16_lo(dv[e]), acc);
        acc = fmaf(bf16_hi(ov[e]), bf16_hi(dv[e]), acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  if (part == 0) {
    const size_t idx = P0 * Hq + (size_t)h * Mp + i;
    if (i < M) {
      const int p = pos[T0 + i];
      float ratio = 1.0f;
      if (p != i) ratio = logf((float)max(p + 1, 2)) / logf((float)max(i + 1, 2));
      rowc[idx] = sm_scale * kLog2e / (temp[h] * ratio);
      rowl[idx] = lse[T0 * Hq + (size_t)h * M + i] * kLog2e;
      rowD[idx] = acc;
    } else {
      rowc[idx] = 0.0f;
      rowl[idx] = INFINITY;
      rowD[idx] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
template <int DH, int G, bool F32OUT>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ rowc, const float* __restrict__ rowl,
    const float* __restrict__ rowD, const float* __restrict__ kscore, const float* __restrict__ gain, int M_all,
    int Mp_all, int Hq, int Hkv, int nkb, int total_wg, void* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ dbp, float* __restrict__ gpart, float* __restrict__ tpart, const BwdSeqTable st) {
  constexpr int KS = DH / 16;       // k-steps over dh
  constexpr int DT = DH / 32;       // 32-row blocks of dK^T and dV^T
  constexpr int TB = kT * DH * 2;   // bytes of a 32 x DH bf16 tile
  constexpr int NI = TB / 1024;     // 1 KiB DMA loads per tile
  constexpr int RC = 2 * TB, RL = RC + 256, RD = RL + 256;
  constexpr int UB = RD + 256;      // bytes of one staged unit (Q, dO, row constants)
  constexpr int NBUF = 3;
  constexpr int RED = 2 * DT * 2 * 16 * 64;  // floats of the parity merge area
  static_assert(NBUF * 2 * UB >= (RED + 2 * 2 * G * 64 + 4 * G) * 4, "merge area");
  __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * 2 * UB];  // [slot][parity] units

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = w & 1, par = w >> 1;
  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  // sequence (length M, first packed row T0, first padded slot P0), KV head
  // g and key block kb: the lowest key blocks (most query tiles) first
  int M = M_all, Mp = Mp_all, g, kb;
  size_t T0, P0;
  if (st.n > 0) {
    const int sq = seq_of(st.pb0, st.n, logical / Hkv);
    M = st.m[sq];
    Mp = (M + kPB - 1) / kPB * kPB;
    const int nk = st.pb0[sq + 1] - st.pb0[sq], local = logical - Hkv * st.pb0[sq];
    g = local / nk;
    kb = local - g * nk;
    T0 = (size_t)st.t0[sq];
    P0 = (size_t)st.p0[sq];
  } else {
    const int bg = logical / nkb;
    kb = logical - bg * nkb;
    const int b = bg / Hkv;
    g = bg - b * Hkv;
    T0 = (size_t)b * M;
    P0 = (size_t)b * Mp;
  }
  const int key0 = kb * kKB, kw0 = key0 + 32 * kh;
  const int kl = lane & 31, gq = lane >> 5;
  const int j = kw0 + kl;  // this lane's key
  const bool j_ok = j < M;
  const int nt = (M + kT - 1) / kT;
  const int t0 = key0 / kT;
  const int U = G * (nt - t0);      // units: (head, query tile) pairs, head fastest
  const int nsteps = (U + 1) / 2;   // a step holds one unit per parity

  bf16x8 kf[KS], vf[KS];
  {
    const size_t off = ((T0 + (j_ok ? j : 0)) * Hkv + g) * DH + gq * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = as_bf16x8(j_ok ? load16(k + off + s * 16) : u32x4{0, 0, 0, 0});
      vf[s] = as_bf16x8(j_ok ? load16(v + off + s * 16) : u32x4{0, 0, 0, 0});
    }
  }
  const float bj = j_ok ? kscore[T0 + j] : 0.0f;
  float kbias[G];  // gain_h log2(e) b_j of each head of the group
#pragma unroll
  for (int i = 0; i < G; ++i) kbias[i] = gain[g * G + i] * kLog2e * bj;

  // Unit u = 2 step + parity is staged by the two waves of that parity: key
  // half 0 brings the Q tile and the row constants (NI + 3 loads), key half 1
  // the dO tile (NI loads).  Rows >= M read 0.
  auto stage = [&](int step, int slot) __attribute__((always_inline)) {
    const int u = 2 * step + par;
    if (u >= U) return;
    const int hl = u % G, t = t0 + u / G;
    const int h = g * G + hl;
    unsigned char* base = smem + (slot * 2 + par) * UB;
    const size_t row0 = ((T0 + t * kT) * Hq + h) * DH;
    const int nrec = (int)(((long long)(M - 1 - t * kT) * Hq + 1) * DH * 2);
    if (kh == 0) {
      const auto rq = rsrc(q + row0, nrec);
#pragma unroll
      for (int e = 0; e < NI; ++e) stage_rows<DH>(rq, base, Hq * DH * 2, e, lane);
      const size_t rr = P0 * Hq + (size_t)h * Mp + t * kT;  // 32 constants; lanes 32..63 read 0
      dma4(rsrc(rowc + rr, kT * 4), base + RC, lane * 4, 0);
      dma4(rsrc(rowl + rr, kT * 4), base + RL, lane * 4, 0);
      dma4(rsrc(rowD + rr, kT * 4), base + RD, lane * 4, 0);
    } else {
      const auto rdo = rsrc(dout + row0, nrec);
#pragma unroll
      for (int e = 0; e < NI; ++e) stage_rows<DH>(rdo, base + TB, Hq * DH * 2, e, lane);
    }
  };

  f32x16 dKt[DT], dVt[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dKt[i][r] = dVt[i][r] = 0.0f;
  float cs[G], ta[G];
#pragma unroll
  for (int i = 0; i < G; ++i) cs[i] = ta[i] = 0.0f;

  // This lane's LDS offsets inside a staged tile, formed once: the swizzled
  // chunk of fragment s is row_tile_off(kl, 2 s + gq) = rto[s & 3] ^ 128 (s >> 2)
  // (chunk bit 3 is offset bit 7, clear in rto), and the transpose loads of
  // tr_frag sit at o = tro[blk & 1] + 128 (blk >> 1) + 16 s 2 DH for the first
  // 8 rows and (o ^ kRow8Flip) + 8 2 DH for the next 8 (the swizzle sees only
  // the row's low 4 bits: the lane's own, and bit 3 for the second 8 rows).
  // The empty asm statements keep them in registers rather than re-derived
  // at every use.
  int rto[4], tro[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rto[i] = row_tile_off<DH>(kl, 2 * i + gq);
    asm volatile("" : "+v"(rto[i]));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    tro[i] = tr_off<DH>(i, 0, 0, lane);
    asm volatile("" : "+v"(tro[i]));
  }
  auto frag_off = [&](int s_) { return rto[s_ & 3] ^ (128 * (s_ >> 2)); };
  auto trf = [&](const unsigned char* tile, int blk, int s_) __attribute__((always_inline)) {
    const int o = tro[blk & 1] + 128 * (blk >> 1) + 16 * s_ * 2 * DH;
    return tr_frag_at(tile, o, (o ^ kRow8Flip<DH>) + 8 * 2 * DH);
  };

  // One unit: S = Q K^T and dP = dO V^T, the softmax terms, then
  // dV^T += dO^T P and dK^T += Q^T dS.  Fragments are read in batches ahead
  // of their products.
  auto step_dkdv = [&](const unsigned char* base, int hl, int t, bool run) __attribute__((always_inline)) {
    f32x16 S, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
    {
      bf16x8 fq[KS], fd[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int off = frag_off(s);
        fq[s] = lds_frag(base + off);
        fd[s] = lds_frag(base + TB + off);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        S = mfma(fq[s], kf[s], S);
        dP = mfma(fd[s], vf[s], dP);
      }
    }
    float kbh = kbias[0];
#pragma unroll
    for (int i = 1; i < G; ++i) kbh = i == hl ? kbias[i] : kbh;
    // rows of S and dP: queries t*32 + 8 i4 + 4 gq + jj; column: key j
    float Pv[16], Sv[16];
    float csum = 0.0f, tsum = 0.0f;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int ro = (8 * i4 + 4 * gq) * 4;
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(base + RC + ro);
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(base + RL + ro);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(base + RD + ro);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * i4 + jj;
        const int qi = t * kT + 8 * i4 + 4 * gq + jj;
        const float z = fmaf(S[r], c4[jj], kbh) - l4[jj];
        const float P = run && j <= qi ? __builtin_amdgcn_exp2f(z) : 0.0f;
        const float dZ = P * (dP[r] - d4[jj]);
        const float dS = dZ * c4[jj];
        csum += dZ;
        tsum = fmaf(dS, S[r], tsum);
        Pv[r] = P;
        Sv[r] = dS;
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (i == hl) {
        cs[i] += csum;
        ta[i] += tsum;
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 pb = pack8(Pv + 8 * s), sb = pack8(Sv + 8 * s);
#pragma unroll
      for (int blk = 0; blk < DT; ++blk) {
        const bf16x8 fdo = trf(base + TB, blk, s), fqt = trf(base, blk, s);
        dVt[blk] = mfma(fdo, pb, dVt[blk]);
        dKt[blk] = mfma(fqt, sb, dKt[blk]);
      }
    }
  };

  // Every step runs its products (a skipped unit contributes exact zeros: its
  // P is 0), so a slot that is never staged -- the last unit of an odd count
  // -- must hold finite values: the staging area starts zeroed.
  for (int i = threadIdx.x; i < NBUF * 2 * UB / 16; i += kBwdThreads)
    reinterpret_cast<u32x4*>(smem)[i] = u32x4{0, 0, 0, 0};
  __syncthreads();
  stage(0, 0);
  stage(1, 1);
  int slot = 0;  // p % NBUF, carried instead of divided
  for (int p = 0; p < nsteps; ++p) {
    // step p's loads are done once at most step p + 1's remain in flight
    if (2 * (p + 1) + par < U) {
      if (kh == 0) wait_loads_le<NI + 3>();
      else wait_loads_le<NI>();
    } else {
      wait_loads_le<0>();
    }
    __syncthreads();  // step p is in LDS; every wave is done with the slot step p + 2 reuses
    const int u = 2 * p + par;
    const int hl = u % G, t = t0 + u / G;
    const bool run = u < U && t * kT + kT - 1 >= kw0 && kw0 < M;  // some key of this wave lies on/below the tile
    const unsigned char* base = smem + (slot * 2 + par) * UB;
    step_dkdv(base, hl, t, run);
    // Issued after this step's transpose loads: the compiler makes an LDS
    // transpose load wait for every LDS-destination load issued before it.
    stage(p + 2, slot == 0 ? NBUF - 1 : slot - 1);
    slot = slot == NBUF - 1 ? 0 : slot + 1;
  }
  // ---- merge the two parities, write dK and dV, the key-score and scale partials ----
  __syncthreads();  // the staging slots are free
  float* red = reinterpret_cast<float*>(smem);
  float* s_x = red + RED + 2 * 2 * G * 64;  // per-wave sums of the two key halves
  float* mine = red + kh * (DT * 2 * 16 * 64);
  float* sums = red + RED + kh * (2 * G * 64);
  if (par == 1) {
#pragma unroll
    for (int blk = 0; blk < DT; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        mine[((blk * 2 + 0) * 16 + r) * 64 + lane] = dKt[blk][r];
        mine[((blk * 2 + 1) * 16 + r) * 64 + lane] = dVt[blk][r];
      }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      sums[i * 64 + lane] = cs[i];
      sums[(G + i) * 64 + lane] = ta[i];
    }
  }
  __syncthreads();
  float gw[G], tw[G];
  if (par == 0) {
#pragma unroll
    for (int blk = 0; blk < DT; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dKt[blk][r] += mine[((blk * 2 + 0) * 16 + r) * 64 + lane];
        dVt[blk][r] += mine[((blk * 2 + 1) * 16 + r) * 64 + lane];
      }
    if (j_ok) {
      const size_t row = ((T0 + j) * Hkv + g) * DH;
#pragma unroll
      for (int blk = 0; blk < DT; ++blk)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * blk + 8 * i4 + 4 * gq;
          const int r = 4 * i4;
          // dS carried c log2(e); dk takes the factor ln 2 back
          store4<F32OUT>(dk, row + d0, dKt[blk][r] * kLn2, dKt[blk][r + 1] * kLn2, dKt[blk][r + 2] * kLn2,
                         dKt[blk][r + 3] * kLn2);
          store4<false>(dv, row + d0, dVt[blk][r], dVt[blk][r + 1], dVt[blk][r + 2], dVt[blk][r + 3]);
        }
    }
    float dbs = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float c = cs[i] + sums[i * 64 + lane];
      c += __shfl_xor(c, 32, 64);  // the partner lane holds the key's other 16 queries of each tile
      dbs = fmaf(gain[g * G + i], c, dbs);
      gw[i] = wave_sum_f32(gq == 0 ? bj * c : 0.0f);
      tw[i] = wave_sum_f32(ta[i] + sums[(G + i) * 64 + lane]);
    }
    if (gq == 0 && j_ok) dbp[P0 * Hkv + (size_t)g * Mp + j] = dbs;
  }
  __syncthreads();
  if (par == 0 && lane == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      s_x[(kh * 2 + 0) * G + i] = gw[i];
      s_x[(kh * 2 + 1) * G + i] = tw[i];
    }
  }
  __syncthreads();
  if (w == 0 && lane < G) {
    const size_t o = (P0 / kKB + kb) * Hq + g * G + lane;
    gpart[o] = s_x[lane] + s_x[2 * G + lane];
    tpart[o] = s_x[G + lane] + s_x[3 * G + lane];
  }
}

// ---------------------------------------------------------------------------
// Query block of the idx-th dQ workgroup of a slab (n blocks, heaviest =
// last): the first p (the CUs of an XCD, which dispatches the slab's first
// p workgroups one per CU and the next p into the same CUs' second slots)
// take the blocks heaviest first, the rest lightest first, so a CU's two
// workgroups pair a heavy block with a light one.  A bijection of [0, n)
// for any p >= 1.
__device__ __forceinline__ int paired_block(int idx, int n, int p) {
  return idx < p ? n - 1 - idx : idx - p;
}

template <int DH, int G, bool F32OUT>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ rowc, const float* __restrict__ rowl,
    const float* __restrict__ rowD, const float* __restrict__ kscore, const float* __restrict__ gain, int M_all,
    int Mp_all, int Hq, int Hkv, int nqb, int total_wg, int pair_p, void* __restrict__ dq, const BwdSeqTable st) {
  constexpr int RG = 4 / G;
  constexpr int BQ = 32 * RG;
  constexpr int KS = DH / 16, DT = DH / 32;
  constexpr int TB = kT * DH * 2;
  constexpr int NI = TB / 1024;
  constexpr int BO = 2 * TB, UB = BO + 256;
  constexpr int NBUF = 3;
  constexpr int NX = 2 * NI / 4;  // DMA loads per wave per tile (K and V); wave 0 adds the key scores
  static_assert(2 * NI % 4 == 0, "staging split");
  __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * UB];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  // sequence, KV head g and query block qb: the heaviest (latest) first
  int M = M_all, Mp = Mp_all, g, qb;
  size_t T0, P0;
  if (st.n > 0) {
    const int sq = seq_of(st.qb0, st.n, logical);
    M = st.m[sq];
    Mp = (M + kPB - 1) / kPB * kPB;
    const int nq = (M + BQ - 1) / BQ, local = logical - st.qb0[sq];
    g = local / nq;
    qb = paired_block(local - g * nq, nq, pair_p);
    T0 = (size_t)st.t0[sq];
    P0 = (size_t)st.p0[sq];
  } else {
    const int bg = logical / nqb;
    qb = paired_block(logical - bg * nqb, nqb, pair_p);
    const int b = bg / Hkv;
    g = bg - b * Hkv;
    T0 = (size_t)b * M;
    P0 = (size_t)b * Mp;
  }
  const int q0 = qb * BQ;
  const int h = g * G + w / RG;
  const int qw0 = q0 + 32 * (w % RG);
  const int ql = lane & 31, gq = lane >> 5;
  const int qi = qw0 + ql;
  const bool q_ok = qi < M;
  const int ntk = (min(M, q0 + BQ) + kT - 1) / kT;

  bf16x8 qf[KS], df[KS];
  {
    const size_t off = ((T0 + (q_ok ? qi : 0)) * Hq + h) * DH + gq * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = as_bf16x8(q_ok ? load16(q + off + s * 16) : u32x4{0, 0, 0, 0});
      df[s] = as_bf16x8(q_ok ? load16(dout + off + s * 16) : u32x4{0, 0, 0, 0});
    }
  }
  const size_t ridx = P0 * Hq + (size_t)h * Mp + (q_ok ? qi : 0);
  const float cq = q_ok ? rowc[ridx] : 0.0f;
  const float lq = q_ok ? rowl[ridx] : INFINITY;
  const float Dq = q_ok ? rowD[ridx] : 0.0f;
  const float gl2 = gain[h] * kLog2e;

  const uint16_t* kbase = k + (T0 * Hkv + g) * DH;
  const uint16_t* vbase = v + (T0 * Hkv + g) * DH;
  const auto rks = rsrc(kscore + T0, M * 4);
  // Tile t: K and V rows (rows >= M read 0) and 64 key scores (those >= M
  // read 0); load x = w + 4 n of the 2 NI goes to wave w.
  auto stage = [&](int t, int slot_t) __attribute__((always_inline)) {
    if (t >= ntk) return;
    unsigned char* base = smem + slot_t * UB;
    const int nrec = (int)(((long long)(M - 1 - t * kT) * Hkv + 1) * DH * 2);
    const size_t roff = (size_t)t * kT * Hkv * DH;
    const auto rk = rsrc(kbase + roff, nrec), rv = rsrc(vbase + roff, nrec);
#pragma unroll
    for (int n = 0; n < NX; ++n) {
      const int x = w + 4 * n;
      const int which = x / NI, e = x - (x / NI) * NI;
      stage_rows<DH>(which == 0 ? rk : rv, base + which * TB, Hkv * DH * 2, e, lane);
    }
    if (w == 0) dma4(rks, base + BO, (t * kT + lane) * 4, 0);
  };

  f32x16 dQt[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQt[i][r] = 0.0f;

  int toff[DT][2][2];  // transpose-load offsets of the K^T fragments, fixed per lane
#pragma unroll
  for (int blk = 0; blk < DT; ++blk)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) toff[blk][s][hf] = tr_off<DH>(blk, s, hf, lane);
  int rto[4];  // row_tile_off(ql, 2 s + gq) = rto[s & 3] ^ 128 (s >> 2), formed once
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rto[i] = row_tile_off<DH>(ql, 2 * i + gq);
    asm volatile("" : "+v"(rto[i]));
  }
  auto step_dq = [&](const unsigned char* base, int t, bool run) __attribute__((always_inline)) {
    f32x16 S, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
    {
      bf16x8 fk[KS], fv[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int off = rto[s & 3] ^ (128 * (s >> 2));
        fk[s] = lds_frag(base + off);
        fv[s] = lds_frag(base + TB + off);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        S = mfma(fk[s], qf[s], S);
        dP = mfma(fv[s], df[s], dP);
      }
    }
    // rows of S^T and dP^T: keys t*32 + 8 i4 + 4 gq + jj; column: query qi
    float Z[16];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(base + BO + (8 * i4 + 4 * gq) * 4);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * i4 + jj;
        const int key = t * kT + 8 * i4 + 4 * gq + jj;
        const float z = fmaf(S[r], cq, gl2 * b4[jj]) - lq;
        const float P = run && key <= qi ? __builtin_amdgcn_exp2f(z) : 0.0f;
        Z[r] = P * (dP[r] - Dq);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 zb = pack8(Z + 8 * s);
#pragma unroll
      for (int blk = 0; blk < DT; ++blk)
        dQt[blk] = mfma(tr_frag_at(base, toff[blk][s][0], toff[blk][s][1]), zb, dQt[blk]);
    }
  };

  const bool wave_rows = qw0 < M;
  stage(0, 0);
  stage(1, 1);
  int slot = 0;  // t % NBUF, carried instead of divided
  for (int t = 0; t < ntk; ++t) {
    if (t + 1 < ntk) {
      if (w == 0) wait_loads_le<NX + 1>();
      else wait_loads_le<NX>();
    } else {
      wait_loads_le<0>();
    }
    __syncthreads();
    // every step runs its products (every tile t < ntk is staged; a tile
    // past this wave's queries has P = 0 and contributes exact zeros)
    const bool run = wave_rows && t * kT <= qw0 + 31;  // some query of this wave reaches the tile
    step_dq(smem + slot * UB, t, run);
    stage(t + 2, slot == 0 ? NBUF - 1 : slot - 1);  // after this step's transpose loads (see the dK/dV kernel)
    slot = slot == NBUF - 1 ? 0 : slot + 1;
  }
  if (q_ok) {
    const float sc = cq * kLn2;  // c_i (the exponent constant carries log2(e))
    const size_t row = ((T0 + qi) * Hq + h) * DH;
#pragma unroll
    for (int blk = 0; blk < DT; ++blk)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * blk + 8 * i4 + 4 * gq;
        const int r = 4 * i4;
        store4<F32OUT>(dq, row + d0, dQt[blk][r] * sc, dQt[blk][r + 1] * sc, dQt[blk][r + 2] * sc,
                       dQt[blk][r + 3] * sc);
      }
  }
}

// ---------------------------------------------------------------------------
// Rotary embedding for the backward of the rotary variant, per 64-row block,
// its rows shared out over the grid's Hkv blocks: ROTATE_BACK false rotates
// the K rows of every KV head and the Q rows of every query head into bf16
// copies, exactly as the forward rotates them (so the products see the
// forward's operands); true applies the transposed rotation to the fp32
// gradients with respect to the rotated q and k and rounds them to bf16.
template <int DH, bool ROTATE_BACK>
__global__ __launch_bounds__(kBwdThreads) void bwd_rope_kernel(const void* __restrict__ q_in,
                                                                const void* __restrict__ k_in,
                                                                const int32_t* __restrict__ pos, double base, int M,
                                                                int Hq, int Hkv, uint16_t* __restrict__ q_out,
                                                                uint16_t* __restrict__ k_out) {
  constexpr int kRows = 16;  // rows whose angles sit in LDS at a time
  __shared__ double s_freq[DH / 2];
  __shared__ f32x2 s_cs[kRows][DH / 2];
  constexpr int PG = DH / 16;  // groups of 8 pairs per head row
  // The angles of a row are formed once, by one of the Hkv blocks of its
  // 64-row block (rows g R .. g R + R - 1, R = ceil(64 / Hkv)), which turns
  // that row of every K and Q head.
  const int m0 = blockIdx.x * kPB, g = blockIdx.y, b = blockIdx.z;
  const int nh = Hkv + Hq;  // head rows of one position: K heads first, then Q heads
  if (threadIdx.x < DH / 2) s_freq[threadIdx.x] = rope::inv_freq(base, threadIdx.x, DH);
  __syncthreads();
  const int R = (kPB + Hkv - 1) / Hkv;
  const int r_hi = min(kPB, (g + 1) * R);
  for (int c0 = g * R; c0 < r_hi; c0 += kRows) {  // (block-uniform)
    const int nr = min(kRows, r_hi - c0);
    for (int t = threadIdx.x; t < nr * PG; t += kBwdThreads) {
      const int rr = t / PG, i0 = (t % PG) * 8, m = m0 + c0 + rr;
      if (m >= M) continue;
      float c[8], sn[8];
      rope::sincos8((double)pos[(size_t)b * M + m], s_freq, i0, c, sn);
#pragma unroll
      for (int i = 0; i < 8; ++i) s_cs[rr][i0 + i] = f32x2{c[i], sn[i]};
    }
    __syncthreads();
    for (int t = threadIdx.x; t < nr * PG * nh; t += kBwdThreads) {
      const int i0 = (t % PG) * 8, hh = (t / PG) % nh, rr = t / (PG * nh), m = m0 + c0 + rr;
      if (m >= M) continue;
      float c[8], sn[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x2 cs = s_cs[rr][i0 + i];
        c[i] = cs[0];
        sn[i] = cs[1];
      }
      const size_t row = (size_t)b * M + m;
      if (hh < Hkv) {
        const size_t krow = (row * Hkv + hh) * DH;
        if constexpr (ROTATE_BACK)
          rope::row8_transposed<DH>(static_cast<const float*>(k_in) + krow, k_out + krow, i0, c, sn);
        else
          rope::row8<DH>(static_cast<const uint16_t*>(k_in) + krow, k_out + krow, i0, c, sn);
      } else {
        const size_t qrow = (row * Hq + (hh - Hkv)) * DH;
        if constexpr (ROTATE_BACK)
          rope::row8_transposed<DH>(static_cast<const float*>(q_in) + qrow, q_out + qrow, i0, c, sn);
        else
          rope::row8<DH>(static_cast<const uint16_t*>(q_in) + qrow, q_out + qrow, i0, c, sn);
      }
    }
    __syncthreads();  // (before the next rows' pairs overwrite LDS)
  }
}

// ---------------------------------------------------------------------------
// db_j = sum over KV heads of the partials.  The last block forms dgain and
// dtemp: one wave per head, lanes over (batch, key block) partials, fp64 and
// a fixed butterfly order.
__global__ __launch_bounds__(kBwdThreads) void bwd_reduce_kernel(const float* __restrict__ dbp,
                                                                  const float* __restrict__ gpart,
                                                                  const float* __restrict__ tpart,
                                                                  const float* __restrict__ temp, int B, int M,
                                                                  int Mp, int Hq, int Hkv, int nkb,
                                                                  float* __restrict__ db, float* __restrict__ dgain,
                                                                  float* __restrict__ dtemp, const BwdSeqTable st) {
  if (st.n > 0) {
    // the last n blocks: sequence s's gain and temperature gradients, in the
    // order a batch-of-one call takes; the others: db over its padded slots
    const int first_gain_block = gridDim.x - st.n;
    if ((int)blockIdx.x >= first_gain_block) {
      const int sq = blockIdx.x - first_gain_block;
      const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
      const int nk = st.pb0[sq + 1] - st.pb0[sq];
      const size_t x0 = (size_t)st.p0[sq] / kKB;
      for (int h = wv; h < Hq; h += kBwdThreads / 64) {
        double gs = 0.0, ts = 0.0;
        for (int x = lane; x < nk; x += 64) {
          gs += gpart[(x0 + x) * Hq + h];
          ts += tpart[(x0 + x) * Hq + h];
        }
        gs = wave_sum_f64(gs);
        ts = wave_sum_f64(ts);
        if (lane == 0) {
          dgain[(size_t)st.out_row[sq] * Hq + h] = (float)gs;
          dtemp[(size_t)st.out_row[sq] * Hq + h] = (float)(-(double)kLn2 * ts / (double)temp[h]);
        }
      }
      return;
    }
    const int slot = blockIdx.x * blockDim.x + threadIdx.x;
    if (slot >= st.pb0[st.n] * kPB) return;
    const int sq = seq_of(st.pb0, st.n, slot / kPB);
    const int m = st.m[sq], mp = (m + kPB - 1) / kPB * kPB, jj = slot - st.pb0[sq] * kPB;
    if (jj >= m) return;
    const size_t P0 = (size_t)st.p0[sq];
    float s = 0.0f;
    for (int g = 0; g < Hkv; ++g) s += dbp[P0 * Hkv + (size_t)g * mp + jj];
    db[(size_t)st.t0[sq] + jj] = s;
    return;
  }
  if (blockIdx.x == gridDim.x - 1) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int h = wv; h < Hq; h += kBwdThreads / 64) {
      double gs = 0.0, ts = 0.0;
      for (int x = lane; x < B * nkb; x += 64) {
        gs += gpart[(size_t)x * Hq + h];
        ts += tpart[(size_t)x * Hq + h];
      }
      gs = wave_sum_f64(gs);
      ts = wave_sum_f64(ts);
      if (lane == 0) {
        dgain[h] = (float)gs;
        dtemp[h] = (float)(-(double)kLn2 * ts / (double)temp[h]);
      }
    }
    return;
  }
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)B * M) return;
  const size_t bi = idx / M, jj = idx - bi * M;
  float s = 0.0f;
  for (int g = 0; g < Hkv; ++g) s += dbp[(bi * Hkv + g) * Mp + jj];
  db[idx] = s;
}

template <int DH, int G>
hipError_t launch_bwd_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                        const float* lse, const uint16_t* dout, int B, int M, int Hq, int Hkv, const float* ks,
                        const int32_t* pos, const float* gain, const float* temp, float sm_scale, double rope_base,
                        uint16_t* dq, uint16_t* dk, uint16_t* dv, float* db, float* dgain, float* dtemp, void* ws,
                        hipStream_t s) {
  const int Mp = (M + kPB - 1) / kPB * kPB;
  const int nkb = Mp / kKB;
  const size_t rn = (size_t)B * Hq * Mp;
  float* rowc = static_cast<float*>(ws);
  float* rowl = rowc + rn;
  float* rowD = rowl + rn;
  float* dbp = rowD + rn;
  float* gpart = dbp + (size_t)B * Hkv * Mp;
  float* tpart = gpart + (size_t)B * nkb * Hq;
  // rotary variant: rotated bf16 q and k, then fp32 gradients with respect to them
  const bool rope = rope_base > 0.0;
  unsigned char* rws = static_cast<unsigned char*>(ws) + rope_ws_offset(B, M, Hq, Hkv, DH);
  uint16_t* qr = reinterpret_cast<uint16_t*>(rws);
  uint16_t* kr = qr + (size_t)B * M * Hq * DH;
  float* dq32 = reinterpret_cast<float*>(kr + (size_t)B * M * Hkv * DH);
  float* dk32 = dq32 + (size_t)B * M * Hq * DH;

  if (M > 0) {
    const dim3 rope_grid(Mp / kPB, Hkv, B);
    if (rope) {
      hipLaunchKernelGGL((bwd_rope_kernel<DH, false>), rope_grid, dim3(kBwdThreads), 0, s, q, k, pos, rope_base, M,
                         Hq, Hkv, qr, kr);
      q = qr;
      k = kr;
    }
    hipLaunchKernelGGL((bwd_rows_kernel<DH>), dim3(Mp / kPB, Hq, B), dim3(kBwdThreads), 0, s, o, dout, lse, pos,
                       temp, sm_scale, M, Mp, Hq, rowc, rowl, rowD, BwdSeqTable{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long ta = (long long)nkb * Hkv * B;
    const int nqb = (M + 32 * (4 / G) - 1) / (32 * (4 / G));
    const long long tb = (long long)nqb * Hkv * B;
    if (ta > 0x7FFFFFFF || tb > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (rope)
      hipLaunchKernelGGL((bwd_dkdv_kernel<DH, G, true>), dim3((unsigned)ta), dim3(kBwdThreads), 0, s, q, k, v, dout,
                         rowc, rowl, rowD, ks, gain, M, Mp, Hq, Hkv, nkb, (int)ta, dk32, dv, dbp, gpart, tpart,
                         BwdSeqTable{});
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<DH, G, false>), dim3((unsigned)ta), dim3(kBwdThreads), 0, s, q, k, v, dout,
                         rowc, rowl, rowD, ks, gain, M, Mp, Hq, Hkv, nkb, (int)ta, dk, dv, dbp, gpart, tpart,
                         BwdSeqTable{});
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int pair_p = std::max(1, device_cu_count() / 8);  // CUs of one XCD
    if (rope)
      hipLaunchKernelGGL((bwd_dq_kernel<DH, G, true>), dim3((unsigned)tb), dim3(kBwdThreads), 0, s, q, k, v, dout,
                         rowc, rowl, rowD, ks, gain, M, Mp, Hq, Hkv, nqb, (int)tb, pair_p, dq32, BwdSeqTable{});
    else
      hipLaunchKernelGGL((bwd_dq_kernel<DH, G, false>), dim3((unsigned)tb), dim3(kBwdThreads), 0, s, q, k, v, dout,
                         rowc, rowl, rowD, ks, gain, M, Mp, Hq, Hkv, nqb, (int)tb, pair_p, dq, BwdSeqTable{});
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (rope) {
      hipLaunchKernelGGL((bwd_rope_kernel<DH, true>), rope_grid, dim3(kBwdThreads), 0, s, dq32, dk32, pos,
                         rope_base, M, Hq, Hkv, dq, dk);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const size_t n = (size_t)B * M;
  const unsigned grid = (unsigned)((n + kBwdThreads - 1) / kBwdThreads) + 1;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(grid), dim3(kBwdThreads), 0, s, dbp, gpart, tpart, temp, B, M, Mp, Hq,
                     Hkv, M > 0 ? nkb : 0, db, dgain, dtemp, BwdSeqTable{});
  return hipGetLastError();
}

// One launch of each kernel over the sequences of a table.  With dq32 and
// dk32 set (the rotary variant, q and k already rotated), dq and dk go out
// in fp32 with respect to the rotated q and k.
template <int DH, int G>
hipError_t launch_bwd_varlen_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                               const float* lse, const uint16_t* dout, const BwdSeqTable& st, int Hq, int Hkv,
                               const float* ks, const int32_t* pos, const float* gain, const float* temp,
                               float sm_scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, float* db, float* dgain,
                               float* dtemp, size_t slots, void* ws, float* dq32, float* dk32, hipStream_t s) {
  const size_t rn = (size_t)Hq * slots;
  float* rowc = static_cast<float*>(ws);
  float* rowl = rowc + rn;
  float* rowD = rowl + rn;
  float* dbp = rowD + rn;
  float* gpart = dbp + (size_t)Hkv * slots;
  float* tpart = gpart + slots / kKB * Hq;
  const int nblk = st.pb0[st.n];
  hipError_t e;
  if (nblk > 0) {
    hipLaunchKernelGGL((bwd_rows_kernel<DH>), dim3(nblk, Hq, 1), dim3(kBwdThreads), 0, s, o, dout, lse, pos, temp,
                       sm_scale, 0, 0, Hq, rowc, rowl, rowD, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int ta = nblk * Hkv;
    if (dk32 != nullptr)
      hipLaunchKernelGGL((bwd_dkdv_kernel<DH, G, true>), dim3(ta), dim3(kBwdThreads), 0, s, q, k, v, dout, rowc,
                         rowl, rowD, ks, gain, 0, 0, Hq, Hkv, 0, ta, dk32, dv, dbp, gpart, tpart, st);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<DH, G, false>), dim3(ta), dim3(kBwdThreads), 0, s, q, k, v, dout, rowc,
                         rowl, rowD, ks, gain, 0, 0, Hq, Hkv, 0, ta, dk, dv, dbp, gpart, tpart, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int pair_p = std::max(1, device_cu_count() / 8);  // CUs of one XCD
    if (dq32 != nullptr)
      hipLaunchKernelGGL((bwd_dq_kernel<DH, G, true>), dim3(st.qb0[st.n]), dim3(kBwdThreads), 0, s, q, k, v, dout,
                         rowc, rowl, rowD, ks, gain, 0, 0, Hq, Hkv, 0, st.qb0[st.n], pair_p, dq32, st);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<DH, G, false>), dim3(st.qb0[st.n]), dim3(kBwdThreads), 0, s, q, k, v, dout,
                         rowc, rowl, rowD, ks, gain, 0, 0, Hq, Hkv, 0, st.qb0[st.n], pair_p, dq, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)(((size_t)nblk * kPB + kBwdThreads - 1) / kBwdThreads) + st.n;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(grid), dim3(kBwdThreads), 0, s, dbp, gpart, tpart, temp, 0, 0, 0, Hq, Hkv,
                     0, db, dgain, dtemp, st);
  return hipGetLastError();
}

}  // namespace

// fp32 c log2(e), lse log2(e) and D [B, Hq, Mp] each, the key-score partials
// [B, Hkv, Mp], and the gain and temperature partials [B, Mp/64, Hq] each.
size_t gated_attention_backward_workspace(int B, int M, int Hq, int Hkv, int dh) {
  (void)dh;
  if (M <= 0) return 0;
  return base_ws_bytes(B, M, Hq, Hkv);
}

// ... rounded up to 16 bytes, then the rotated q and k (bf16) and the fp32
// gradients with respect to them
size_t gated_attention_rope_backward_workspace(int B, int M, int Hq, int Hkv, int dh) {
  if (M <= 0) return 0;
  return rope_ws_offset(B, M, Hq, Hkv, dh) + (size_t)B * M * (Hq + Hkv) * dh * (2 + 4);
}

size_t gated_attention_backward_varlen_workspace(int B, const int32_t* cu_seqlens, int Hq, int Hkv) {
  size_t slots = 0;
  for (int b = 0; b < B; ++b) slots += (size_t)(cu_seqlens[b + 1] - cu_seqlens[b] + kPB - 1) / kPB * kPB;
  return slots * (size_t)(12 * Hq + 4 * Hkv) + 8 * (slots / kKB) * Hq;
}

// ... rounded up to 16 bytes, then the rotated q and k (bf16) and the fp32
// gradients with respect to them, by packed row
size_t gated_attention_rope_backward_varlen_workspace(int B, const int32_t* cu_seqlens, int Hq, int Hkv, int dh) {
  return rope_varlen_ws_offset(B, cu_seqlens, Hq, Hkv) + (size_t)cu_seqlens[B] * (Hq + Hkv) * dh * (2 + 4);
}

hipError_t launch_gated_attention_backward_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                                  const uint16_t* out, const float* lse, const uint16_t* d_out, int B,
                                                  const int32_t* cu_seqlens, int Hq, int Hkv, int dh,
                                                  const float* key_score, const int32_t* pos, const float* gain,
                                                  const float* temp, float sm_scale, double rope_base, uint16_t* dq,
                                                  uint16_t* dk, uint16_t* dv, float* d_key_score, float* d_gain,
                                                  float* d_temp, void* ws, hipStream_t s) {
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4) return hipErrorInvalidValue;
  if (dh != 64 && dh != 128) return hipErrorInvalidValue;
  const int BQ = 32 * (4 / G);
  // rotary variant: every packed row of q and k turned by its own position
  // (the rows of all sequences at once, as one row block of T rows), the
  // kernels on the rotated copies with fp32 gradients, then the transposed
  // rotation of those
  const size_t T = (size_t)cu_seqlens[B];
  const bool rope = rope_base > 0.0 && T > 0;
  uint16_t *qr = nullptr, *kr = nullptr;
  float *dq32 = nullptr, *dk32 = nullptr;
  const dim3 rope_grid((unsigned)((T + kPB - 1) / kPB), Hkv, 1);
  if (rope) {
    unsigned char* rws = static_cast<unsigned char*>(ws) + rope_varlen_ws_offset(B, cu_seqlens, Hq, Hkv);
    qr = reinterpret_cast<uint16_t*>(rws);
    kr = qr + T * Hq * dh;
    dq32 = reinterpret_cast<float*>(kr + T * Hkv * dh);
    dk32 = dq32 + T * Hq * dh;
    if (dh == 128)
      hipLaunchKernelGGL((bwd_rope_kernel<128, false>), rope_grid, dim3(kBwdThreads), 0, s, q, k, pos, rope_base,
                         (int)T, Hq, Hkv, qr, kr);
    else
      hipLaunchKernelGGL((bwd_rope_kernel<64, false>), rope_grid, dim3(kBwdThreads), 0, s, q, k, pos, rope_base,
                         (int)T, Hq, Hkv, qr, kr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    q = qr;
    k = kr;
  }
  // every sequence (the empty ones get zero gain and temperature gradients), longest first
  std::vector<int> order(B);
  for (int b = 0; b < B; ++b) order[b] = b;
  std::stable_sort(order.begin(), order.end(), [&](int a, int c) {
    return cu_seqlens[a + 1] - cu_seqlens[a] > cu_seqlens[c + 1] - cu_seqlens[c];
  });
  size_t slots = 0;
  for (int b = 0; b < B; ++b) slots += (size_t)(cu_seqlens[b + 1] - cu_seqlens[b] + kPB - 1) / kPB * kPB;
  size_t p = 0;
  for (size_t i = 0; i < order.size(); i += kMaxBwdSeqs) {
    BwdSeqTable st{};
    st.n = (int)std::min(order.size() - i, (size_t)kMaxBwdSeqs);
    long long pb = 0, qw = 0;
    for (int j = 0; j < st.n; ++j) {
      const int b = order[i + j], m = cu_seqlens[b + 1] - cu_seqlens[b];
      const int mp = (m + kPB - 1) / kPB * kPB;
      if (p + mp > 0x7FFFFFFF) return hipErrorInvalidValue;
      st.t0[j] = cu_seqlens[b];
      st.m[j] = m;
      st.p0[j] = (int)p;
      st.out_row[j] = b;
      st.pb0[j] = (int)pb;
      st.qb0[j] = (int)qw;
      p += mp;
      pb += mp / kPB;
      qw += (long long)((m + BQ - 1) / BQ) * Hkv;
      if (pb * Hkv > 0x7FFFFFFF / kBwdThreads || qw > 0x7FFFFFFF / kBwdThreads) return hipErrorInvalidValue;
    }
    st.pb0[st.n] = (int)pb;
    st.qb0[st.n] = (int)qw;
    hipError_t e = hipErrorInvalidValue;
#define TG_BWD_VARLEN_CASE(DHV, GV)                                                                              \
  if (dh == DHV && G == GV)                                                                                      \
    e = launch_bwd_varlen_t<DHV, GV>(q, k, v, out, lse, d_out, st, Hq, Hkv, key_score, pos, gain, temp, sm_scale, \
                                     dq, dk, dv, d_key_score, d_gain, d_temp, slots, ws, dq32, dk32, s);
    TG_BWD_VARLEN_CASE(128, 2)
    TG_BWD_VARLEN_CASE(128, 1)
    TG_BWD_VARLEN_CASE(128, 4)
    TG_BWD_VARLEN_CASE(64, 2)
    TG_BWD_VARLEN_CASE(64, 1)
    TG_BWD_VARLEN_CASE(64, 4)
#undef TG_BWD_VARLEN_CASE
    if (e != hipSuccess) return e;
  }
  if (rope) {
    if (dh == 128)
      hipLaunchKernelGGL((bwd_rope_kernel<128, true>), rope_grid, dim3(kBwdThreads), 0, s, dq32, dk32, pos,
                         rope_base, (int)T, Hq, Hkv, dq, dk);
    else
      hipLaunchKernelGGL((bwd_rope_kernel<64, true>), rope_grid, dim3(kBwdThreads), 0, s, dq32, dk32, pos, rope_base,
                         (int)T, Hq, Hkv, dq, dk);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_gated_attention_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                           const uint16_t* out, const float* lse, const uint16_t* d_out, int B, int M,
                                           int Hq, int Hkv, int dh, const float* key_score, const int32_t* pos,
                                           const float* gain, const float* temp, float sm_scale, double rope_base,
                                           uint16_t* dq,
                                           uint16_t* dk, uint16_t* dv, float* d_key_score, float* d_gain,
                                           float* d_temp, void* ws, hipStream_t s) {
  const int G = Hq / Hkv;
#define TG_BWD_CASE(DHV, GV)                                                                                        \
  if (dh == DHV && G == GV)                                                                                         \
    return launch_bwd_t<DHV, GV>(q, k, v, out, lse, d_out, B, M, Hq, Hkv, key_score, pos, gain, temp, sm_scale,   \
                                 rope_base, dq, dk, dv, d_key_score, d_gain, d_temp, ws, s);
  TG_BWD_CASE(128, 2)
  TG_BWD_CASE(128, 1)
  TG_BWD_CASE(128, 4)
  TG_BWD_CASE(64, 2)
  TG_BWD_CASE(64, 1)
  TG_BWD_CASE(64, 4)
#undef TG_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tg
