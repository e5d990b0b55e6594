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
//  * bwd_prepass: per 64-row block of a query head, D_i and the exponent
//    constants c_i log2(e) and lse_i log2(e) (+inf beyond M, so padded rows
//    get P = 0), and transposed copies Q^T and dO^T [B, Hq, dh, Mp]; per
//    64-row block of a KV head, K^T [B, Hkv, dh, Mp].  Inside every 16-row
//    group of a transposed row the middle two quads are swapped: that is the
//    order in which an MFMA accumulator hands a lane its 8 rows of a 16-wide
//    k-step, so accumulators feed the next product as B fragments directly.
//  * bwd_dkdv: a workgroup owns 64 keys of one KV head, keeps their K and V
//    fragments in registers and walks every 32-query tile of each of the G
//    query heads from the diagonal down.  S = Q K^T and dP = dO V^T come out
//    with one lane per key, so P and dS = dZ c are at once the B fragments of
//    dV^T += dO^T P and dK^T += Q^T dS.  Four waves: two key halves x two
//    query-tile parities, merged through LDS at the end.  The lane's running
//    column sums of dZ give the key-score, gain and temperature partials.
//    Tiles travel global -> LDS by buffer loads with the LDS-destination bit,
//    double-buffered: step p + 1 is in flight while step p is computed.
//  * bwd_dq: a workgroup owns 32 (4/G) query rows of each of the G heads,
//    keeps their Q and dO fragments in registers and walks the 32-key tiles
//    up to the diagonal.  S^T = K Q^T and dP^T = V dO^T come out with one
//    lane per query, so dZ^T is the B fragment of dQ^T += K^T dZ^T and c_i
//    is applied once at the end.
//  * bwd_reduce: db as the sum of the per-KV-head partials, dgain and dtemp
//    as fixed-order sums of the per-block partials.  No atomics anywhere:
//    the results are deterministic.
#include <math.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kPB = 64;   // rows per prepass block (Mp is a multiple of it)
constexpr int kKB = 64;   // keys per dK/dV workgroup
constexpr int kT = 32;    // queries per dK/dV tile, keys per dQ tile
constexpr int kRsrcCfg = 0x00020000;  // raw buffer resource word 3 (gfx9 family, 32-bit data)

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

// Row held by slot s of a transposed 16-row group (self-inverse).
__device__ __forceinline__ int slot_row(int s) {
  const int q = (s >> 2) & 3;
  const int kq = q == 1 ? 2 : (q == 2 ? 1 : q);
  return (s & ~15) | (kq << 2) | (s & 3);
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

// Byte offset, inside a staged [32 rows x DH] bf16 tile, of row r's 16-byte
// chunk c (chunks swizzled by r & 7: conflict-free fragment reads).
template <int DH>
__device__ __forceinline__ int row_tile_off(int r, int c) {
  return r * (2 * DH) + ((c ^ (r & 7)) << 4);
}
// ... and inside a staged [DH rows x 32] transposed tile (64-byte rows,
// chunks swizzled by (d >> 2) & 3).
__device__ __forceinline__ int tr_tile_off(int d, int c) { return d * 64 + ((c ^ ((d >> 2) & 3)) << 4); }

// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(kBwdThreads) void bwd_prepass_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const int32_t* __restrict__ pos,
    const float* __restrict__ temp, float sm_scale, int M, int Mp, int Hq, int Hkv, uint16_t* __restrict__ qT,
    uint16_t* __restrict__ doT, uint16_t* __restrict__ kTo, float* __restrict__ rowc, float* __restrict__ rowl,
    float* __restrict__ rowD) {
  constexpr int LS = DH + 2;  // LDS row stride in bf16 (odd word stride: conflict-free column reads)
  constexpr int CH = DH / 8;
  __shared__ __attribute__((aligned(16))) uint16_t s_t[kPB * LS];
  const int b = blockIdx.z, y = blockIdx.y, i0 = blockIdx.x * kPB;
  const int tid = threadIdx.x;
  const bool is_kv = y >= Hq;
  const int hh = is_kv ? y - Hq : y;
  const int H = is_kv ? Hkv : Hq;

  // src rows (b, i0 .. i0 + 63, head hh) -> dst [b, hh, d, i0 + slot]; rows >= M give 0
  auto transpose = [&](const uint16_t* src, uint16_t* dst) {
    for (int c = tid; c < kPB * CH; c += kBwdThreads) {
      const int r = c / CH, ch = c - (c / CH) * CH;
      const int i = i0 + r;
      const u32x4 v = i < M ? load16(src + (((size_t)b * M + i) * H + hh) * DH + ch * 8) : u32x4{0, 0, 0, 0};
      uint32_t* wp = reinterpret_cast<uint32_t*>(s_t + r * LS + ch * 8);
      wp[0] = v[0];
      wp[1] = v[1];
      wp[2] = v[2];
      wp[3] = v[3];
    }
    __syncthreads();
    uint16_t* base = dst + ((size_t)b * H + hh) * DH * Mp + i0;
    for (int c = tid; c < DH * (kPB / 8); c += kBwdThreads) {
      const int d = c / (kPB / 8), ch = c % (kPB / 8);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r0 = slot_row(ch * 8 + 2 * e), r1 = slot_row(ch * 8 + 2 * e + 1);
        w[e] = (uint32_t)s_t[r0 * LS + d] | ((uint32_t)s_t[r1 * LS + d] << 16);
      }
      store16(base + (size_t)d * Mp + ch * 8, w);
    }
    __syncthreads();
  };

  if (is_kv) {
    transpose(k, kTo);
    return;
  }
  transpose(q, qT);
  transpose(dout, doT);  // s_t keeps the dO block for D below

  // D_i = dO_i . O_i: four threads per row, fixed order
  const int r = tid >> 2, part = tid & 3;
  const int i = i0 + r;
  float acc = 0.0f;
  if (i < M) {
    const uint16_t* op = o + (((size_t)b * M + i) * Hq + hh) * DH + part * (DH / 4);
    const uint16_t* dp = s_t + r * LS + part * (DH / 4);
#pragma unroll
    for (int c = 0; c < DH / 32; ++c) {
      const u32x4 ov = load16(op + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf16_lo(ov[e]), bf16_to_f32(dp[c * 8 + 2 * e]), acc);
        acc = fmaf(bf16_hi(ov[e]), bf16_to_f32(dp[c * 8 + 2 * e + 1]), acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  if (part == 0) {
    const size_t idx = ((size_t)b * Hq + hh) * Mp + i;
    if (i < M) {
      const int p = pos[(size_t)b * M + i];
      float ratio = 1.0f;
      if (p != i) ratio = logf((float)max(p + 1, 2)) / logf((float)max(i + 1, 2));
      rowc[idx] = sm_scale * kLog2e / (temp[hh] * ratio);
      rowl[idx] = lse[((size_t)b * Hq + hh) * M + i] * kLog2e;
      rowD[idx] = acc;
    } else {
      rowc[idx] = 0.0f;
      rowl[idx] = INFINITY;
      rowD[idx] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
template <int DH, int G>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ qT, const uint16_t* __restrict__ doT,
    const float* __restrict__ rowc, const float* __restrict__ rowl, const float* __restrict__ rowD,
    const float* __restrict__ kscore, const float* __restrict__ gain, int M, int Mp, int Hq, int Hkv, int nkb,
    int total_wg, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ dbp,
    float* __restrict__ gpart, float* __restrict__ tpart) {
  constexpr int KS = DH / 16;       // k-steps over dh
  constexpr int DT = DH / 32;       // 32-row blocks of dK^T and dV^T
  constexpr int CH = DH / 8;        // 16-byte chunks per row
  constexpr int TB = kT * DH * 2;   // bytes of a 32 x DH bf16 tile
  constexpr int NI = TB / 1024;     // 1 KiB DMA instructions per tile
  constexpr int RC = 4 * TB, RL = RC + 256, RD = RL + 256;
  constexpr int UB = RD + 256;      // bytes of one staged unit (Q, dO, Q^T, dO^T, row constants)
  constexpr int RED = 2 * DT * 2 * 16 * 64;  // floats of the parity merge area
  static_assert(4 * UB >= (RED + 2 * 2 * G * 64) * 4, "merge area");
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * UB];  // [buffer][parity] units
  __shared__ float s_x[4 * G];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = w & 1, par = w >> 1;
  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  const int bg = logical / nkb;
  const int kb = logical - bg * nkb;  // lowest key blocks (most query tiles) first
  const int b = bg / Hkv, g = bg - b * Hkv;
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
    const size_t off = (((size_t)b * M + (j_ok ? j : 0)) * Hkv + g) * DH + gq * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = as_bf16x8(j_ok ? load16(k + off + s * 16) : u32x4{0, 0, 0, 0});
      vf[s] = as_bf16x8(j_ok ? load16(v + off + s * 16) : u32x4{0, 0, 0, 0});
    }
  }
  const float bj = j_ok ? kscore[(size_t)b * M + j] : 0.0f;

  // Unit u = 2 step + parity is staged by the two waves of that parity: key
  // half 0 brings the row-major Q and dO tiles and the row constants, key
  // half 1 the transposed tiles.
  auto stage = [&](int step, int buf) __attribute__((always_inline)) {
    const int u = 2 * step + par;
    if (u >= U) return;
    const int hl = u % G, t = t0 + u / G;
    const int h = g * G + hl;
    unsigned char* base = smem + (buf * 2 + par) * UB;
    if (kh == 0) {
      const size_t row0 = (((size_t)b * M + t * kT) * Hq + h) * DH;
      const int nrec = (int)(((long long)(M - 1 - t * kT) * Hq + 1) * DH * 2);  // rows >= M read 0
      const auto rq = rsrc(q + row0, nrec), rdo = rsrc(dout + row0, nrec);
#pragma unroll
      for (int e = 0; e < NI; ++e) {
        const int Y = e * 64 + lane;
        const int r = Y / CH, c = (Y % CH) ^ (r & 7);
        const int voff = r * Hq * DH * 2 + c * 16;
        dma16(rq, base + e * 1024, voff, 0);
        dma16(rdo, base + TB + e * 1024, voff, 0);
      }
      const size_t rr = ((size_t)b * Hq + h) * Mp + t * kT;  // 32 constants; lanes 32..63 read 0
      dma4(rsrc(rowc + rr, kT * 4), base + RC, lane * 4, 0);
      dma4(rsrc(rowl + rr, kT * 4), base + RL, lane * 4, 0);
      dma4(rsrc(rowD + rr, kT * 4), base + RD, lane * 4, 0);
    } else {
      const size_t hb = ((size_t)b * Hq + h) * DH * Mp;
      const auto rt = rsrc(qT + hb, DH * Mp * 2), rdt = rsrc(doT + hb, DH * Mp * 2);
#pragma unroll
      for (int e = 0; e < NI; ++e) {
        const int Y = e * 64 + lane;
        const int d = Y >> 2, c = (Y & 3) ^ ((d >> 2) & 3);
        const int voff = d * Mp * 2 + c * 16;
        dma16(rt, base + 2 * TB + e * 1024, voff, t * kT * 2);
        dma16(rdt, base + 3 * TB + e * 1024, voff, t * kT * 2);
      }
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

  stage(0, 0);
  for (int p = 0; p < nsteps; ++p) {
    wait_loads();
    __syncthreads();  // step p is in LDS; every wave is done with the buffer step p + 1 reuses
    if (p + 1 < nsteps) stage(p + 1, (p + 1) & 1);
    const int u = 2 * p + par;
    if (u >= U) continue;
    const int hl = u % G, t = t0 + u / G;
    if (t * kT + kT - 1 < kw0 || kw0 >= M) continue;  // every key of this wave lies above the tile
    const unsigned char* base = smem + ((p & 1) * 2 + par) * UB;
    const float kbh = gain[g * G + hl] * kLog2e * bj;

    f32x16 S, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = row_tile_off<DH>(kl, 2 * s + gq);
      S = mfma(lds_frag(base + off), kf[s], S);
      dP = mfma(lds_frag(base + TB + off), vf[s], dP);
    }
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
        const float P = j <= qi ? __builtin_amdgcn_exp2f(z) : 0.0f;
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
        const int off = tr_tile_off(32 * blk + kl, 2 * s + gq);
        dVt[blk] = mfma(lds_frag(base + 3 * TB + off), pb, dVt[blk]);
        dKt[blk] = mfma(lds_frag(base + 2 * TB + off), sb, dKt[blk]);
      }
    }
  }

  // ---- merge the two parities, write dK and dV, the key-score and scale partials ----
  __syncthreads();  // the staging buffers are free
  float* red = reinterpret_cast<float*>(smem);
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
      uint16_t* kp = dk + (((size_t)b * M + j) * Hkv + g) * DH;
      uint16_t* vp = dv + (((size_t)b * M + j) * Hkv + g) * DH;
#pragma unroll
      for (int blk = 0; blk < DT; ++blk)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * blk + 8 * i4 + 4 * gq;
          const int r = 4 * i4;
          // dS carried c log2(e); dk takes the factor ln 2 back
          *reinterpret_cast<u32x2*>(kp + d0) =
              u32x2{pack_bf16x2(dKt[blk][r] * kLn2, dKt[blk][r + 1] * kLn2),
                    pack_bf16x2(dKt[blk][r + 2] * kLn2, dKt[blk][r + 3] * kLn2)};
          *reinterpret_cast<u32x2*>(vp + d0) = u32x2{pack_bf16x2(dVt[blk][r], dVt[blk][r + 1]),
                                                     pack_bf16x2(dVt[blk][r + 2], dVt[blk][r + 3])};
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
    if (gq == 0 && j_ok) dbp[((size_t)b * Hkv + g) * Mp + j] = dbs;
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
    const size_t o = ((size_t)b * nkb + kb) * Hq + g * G + lane;
    gpart[o] = s_x[lane] + s_x[2 * G + lane];
    tpart[o] = s_x[G + lane] + s_x[3 * G + lane];
  }
}

// ---------------------------------------------------------------------------
template <int DH, int G>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ kTi, const float* __restrict__ rowc,
    const float* __restrict__ rowl, const float* __restrict__ rowD, const float* __restrict__ kscore,
    const float* __restrict__ gain, int M, int Mp, int Hq, int Hkv, int nqb, int total_wg,
    uint16_t* __restrict__ dq) {
  constexpr int RG = 4 / G;
  constexpr int BQ = 32 * RG;
  constexpr int KS = DH / 16, DT = DH / 32, CH = DH / 8;
  constexpr int TB = kT * DH * 2;
  constexpr int NI = TB / 1024;
  constexpr int BO = 3 * TB, UB = BO + 256;
  constexpr int NX = 3 * NI / 4;  // DMA instructions per wave per tile (K, V, K^T)
  static_assert(3 * NI % 4 == 0, "staging split");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * UB];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  const int bg = logical / nqb;
  const int qb = nqb - 1 - (logical - bg * nqb);  // heaviest (latest) query blocks first
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int q0 = qb * BQ;
  const int h = g * G + w / RG;
  const int qw0 = q0 + 32 * (w % RG);
  const int ql = lane & 31, gq = lane >> 5;
  const int qi = qw0 + ql;
  const bool q_ok = qi < M;
  const int ntk = (min(M, q0 + BQ) + kT - 1) / kT;

  bf16x8 qf[KS], df[KS];
  {
    const size_t off = (((size_t)b * M + (q_ok ? qi : 0)) * Hq + h) * DH + gq * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = as_bf16x8(q_ok ? load16(q + off + s * 16) : u32x4{0, 0, 0, 0});
      df[s] = as_bf16x8(q_ok ? load16(dout + off + s * 16) : u32x4{0, 0, 0, 0});
    }
  }
  const size_t ridx = ((size_t)b * Hq + h) * Mp + (q_ok ? qi : 0);
  const float cq = q_ok ? rowc[ridx] : 0.0f;
  const float lq = q_ok ? rowl[ridx] : INFINITY;
  const float Dq = q_ok ? rowD[ridx] : 0.0f;
  const float gl2 = gain[h] * kLog2e;

  const uint16_t* kbase = k + ((size_t)b * M * Hkv + g) * DH;
  const uint16_t* vbase = v + ((size_t)b * M * Hkv + g) * DH;
  const auto rkt = rsrc(kTi + ((size_t)b * Hkv + g) * DH * Mp, DH * Mp * 2);
  const auto rks = rsrc(kscore + (size_t)b * M, M * 4);
  // Tile t: K, V (row-major, rows >= M read 0), K^T (transposed) and 64 key
  // scores (those >= M read 0); instruction x = w + 4 n of the 3 NI.
  auto stage = [&](int t, int buf) __attribute__((always_inline)) {
    unsigned char* base = smem + buf * UB;
    const int nrec = (int)(((long long)(M - 1 - t * kT) * Hkv + 1) * DH * 2);
    const size_t roff = (size_t)t * kT * Hkv * DH;
    const auto rk = rsrc(kbase + roff, nrec), rv = rsrc(vbase + roff, nrec);
#pragma unroll
    for (int n = 0; n < NX; ++n) {
      const int x = w + 4 * n;
      const int which = x / NI, e = x - (x / NI) * NI;
      const int Y = e * 64 + lane;
      if (which < 2) {
        const int r = Y / CH, c = (Y % CH) ^ (r & 7);
        dma16(which == 0 ? rk : rv, base + which * TB + e * 1024, r * Hkv * DH * 2 + c * 16, 0);
      } else {
        const int d = Y >> 2, c = (Y & 3) ^ ((d >> 2) & 3);
        dma16(rkt, base + 2 * TB + e * 1024, d * Mp * 2 + c * 16, t * kT * 2);
      }
    }
    if (w == 0) dma4(rks, base + BO, (t * kT + lane) * 4, 0);
  };

  f32x16 dQt[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQt[i][r] = 0.0f;

  stage(0, 0);
  for (int t = 0; t < ntk; ++t) {
    wait_loads();
    __syncthreads();
    if (t + 1 < ntk) stage(t + 1, (t + 1) & 1);
    if (qw0 >= M || t * kT > qw0 + 31) continue;  // no query of this wave reaches the tile
    const unsigned char* base = smem + (t & 1) * UB;
    f32x16 S, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = row_tile_off<DH>(ql, 2 * s + gq);
      S = mfma(lds_frag(base + off), qf[s], S);
      dP = mfma(lds_frag(base + TB + off), df[s], dP);
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
        const float P = key <= qi ? __builtin_amdgcn_exp2f(z) : 0.0f;
        Z[r] = P * (dP[r] - Dq);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 zb = pack8(Z + 8 * s);
#pragma unroll
      for (int blk = 0; blk < DT; ++blk)
        dQt[blk] = mfma(lds_frag(base + 2 * TB + tr_tile_off(32 * blk + ql, 2 * s + gq)), zb, dQt[blk]);
    }
  }

  if (q_ok) {
    const float sc = cq * kLn2;  // c_i (the exponent constant carries log2(e))
    uint16_t* qp = dq + (((size_t)b * M + qi) * Hq + h) * DH;
#pragma unroll
    for (int blk = 0; blk < DT; ++blk)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * blk + 8 * i4 + 4 * gq;
        const int r = 4 * i4;
        *reinterpret_cast<u32x2*>(qp + d0) = u32x2{pack_bf16x2(dQt[blk][r] * sc, dQt[blk][r + 1] * sc),
                                                   pack_bf16x2(dQt[blk][r + 2] * sc, dQt[blk][r + 3] * sc)};
      }
  }
}

// ---------------------------------------------------------------------------
// db_j = sum over KV heads of the partials; the last block forms dgain and
// dtemp from the per-(batch, key block) partials in a fixed order.
__global__ __launch_bounds__(kBwdThreads) void bwd_reduce_kernel(const float* __restrict__ dbp,
                                                                  const float* __restrict__ gpart,
                                                                  const float* __restrict__ tpart,
                                                                  const float* __restrict__ temp, int B, int M,
                                                                  int Mp, int Hq, int Hkv, int nkb,
                                                                  float* __restrict__ db, float* __restrict__ dgain,
                                                                  float* __restrict__ dtemp) {
  if (blockIdx.x == gridDim.x - 1) {
    for (int h = threadIdx.x; h < Hq; h += blockDim.x) {
      double gs = 0.0, ts = 0.0;
      for (int bi = 0; bi < B; ++bi)
        for (int kb = 0; kb < nkb; ++kb) {
          gs += gpart[((size_t)bi * nkb + kb) * Hq + h];
          ts += tpart[((size_t)bi * nkb + kb) * Hq + h];
        }
      dgain[h] = (float)gs;
      dtemp[h] = (float)(-(double)kLn2 * ts / (double)temp[h]);
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
                        const int32_t* pos, const float* gain, const float* temp, float sm_scale, uint16_t* dq,
                        uint16_t* dk, uint16_t* dv, float* db, float* dgain, float* dtemp, void* ws, hipStream_t s) {
  const int Mp = (M + kPB - 1) / kPB * kPB;
  const int nkb = Mp / kKB;
  const size_t qn = (size_t)B * Hq * DH * Mp, kn = (size_t)B * Hkv * DH * Mp, rn = (size_t)B * Hq * Mp;
  uint16_t* qT = static_cast<uint16_t*>(ws);
  uint16_t* doT = qT + qn;
  uint16_t* kTw = doT + qn;
  float* rowc = reinterpret_cast<float*>(kTw + kn);
  float* rowl = rowc + rn;
  float* rowD = rowl + rn;
  float* dbp = rowD + rn;
  float* gpart = dbp + (size_t)B * Hkv * Mp;
  float* tpart = gpart + (size_t)B * nkb * Hq;

  if (M > 0) {
    hipLaunchKernelGGL((bwd_prepass_kernel<DH>), dim3(Mp / kPB, Hq + Hkv, B), dim3(kBwdThreads), 0, s, q, k, o, dout,
                       lse, pos, temp, sm_scale, M, Mp, Hq, Hkv, qT, doT, kTw, rowc, rowl, rowD);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long ta = (long long)nkb * Hkv * B;
    const int nqb = (M + 32 * (4 / G) - 1) / (32 * (4 / G));
    const long long tb = (long long)nqb * Hkv * B;
    if (ta > 0x7FFFFFFF || tb > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<DH, G>), dim3((unsigned)ta), dim3(kBwdThreads), 0, s, q, k, v, dout, qT, doT,
                       rowc, rowl, rowD, ks, gain, M, Mp, Hq, Hkv, nkb, (int)ta, dk, dv, dbp, gpart, tpart);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<DH, G>), dim3((unsigned)tb), dim3(kBwdThreads), 0, s, q, k, v, dout, kTw, rowc,
                       rowl, rowD, ks, gain, M, Mp, Hq, Hkv, nqb, (int)tb, dq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t n = (size_t)B * M;
  const unsigned grid = (unsigned)((n + kBwdThreads - 1) / kBwdThreads) + 1;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(grid), dim3(kBwdThreads), 0, s, dbp, gpart, tpart, temp, B, M, Mp, Hq,
                     Hkv, M > 0 ? nkb : 0, db, dgain, dtemp);
  return hipGetLastError();
}

}  // namespace

// Q^T and dO^T [B, Hq, dh, Mp] and K^T [B, Hkv, dh, Mp] (bf16), then fp32
// c log2(e), lse log2(e) and D [B, Hq, Mp] each, the key-score partials
// [B, Hkv, Mp], and the gain and temperature partials [B, Mp/64, Hq] each.
size_t gated_attention_backward_workspace(int B, int M, int Hq, int Hkv, int dh) {
  if (M <= 0) return 0;
  const size_t Mp = (size_t)(M + kPB - 1) / kPB * kPB;
  return (size_t)B * Mp * ((size_t)(2 * Hq + Hkv) * dh * 2 + (size_t)3 * Hq * 4 + (size_t)Hkv * 4) +
         (size_t)2 * B * (Mp / kKB) * Hq * 4;
}

hipError_t launch_gated_attention_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                           const uint16_t* out, const float* lse, const uint16_t* d_out, int B, int M,
                                           int Hq, int Hkv, int dh, const float* key_score, const int32_t* pos,
                                           const float* gain, const float* temp, float sm_scale, uint16_t* dq,
                                           uint16_t* dk, uint16_t* dv, float* d_key_score, float* d_gain,
                                           float* d_temp, void* ws, hipStream_t s) {
  const int G = Hq / Hkv;
#define TG_BWD_CASE(DHV, GV)                                                                                        \
  if (dh == DHV && G == GV)                                                                                         \
    return launch_bwd_t<DHV, GV>(q, k, v, out, lse, d_out, B, M, Hq, Hkv, key_score, pos, gain, temp, sm_scale, dq, \
                                 dk, dv, d_key_score, d_gain, d_temp, ws, s);
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
