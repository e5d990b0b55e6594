// Token-gated causal GQA attention over the kept set (TokenGate paper,
// Section 4: token-gated attention Eq. 5, head-wise gain Eq. 6, temperature
// Eq. 7, combined into the key-bias form Eq. 8; Appendix C.4).
//
//   z_ij = (q_i . k_j) * sm_scale / (temp_h * ratio_i) + gain_h * b_j,  j <= i
//   ratio_i = 1 if pos_i == i else ln(max(pos_i+1, 2)) / ln(max(i+1, 2))
//
// Flash-style forward on gfx950, bf16 MFMA 32x32x16 with fp32 accumulation.
//  * Workgroup = 4 waves = the G query heads of one KV head x (4/G) groups of
//    32 query rows, so every K/V tile staged in LDS serves G heads.
//  * Scores are computed transposed, S^T = K Q^T: a lane owns one query and
//    16 keys of a 32-key tile, so the row max/sum is an in-lane reduction
//    plus one exchange with the partner lane (l ^ 32).  The softmax numerator
//    P^T is then already in B-fragment layout for O^T += V^T P^T; the key
//    order inside each 16-key step is permuted identically on both operands.
//  * The logit is formed in the log2 domain with one FMA per element:
//    z = s * (sm_scale*log2e/tau_i) + (gain_h*log2e) * b_j, the key term
//    pre-multiplied per head when the tile is staged.
//  * K tiles are stored row-major, V tiles transposed (V^T, key-contiguous);
//    both padded so fragment reads and transposing writes avoid bank
//    conflicts.  Tiles are double-buffered through registers.
//  * Grid: heaviest causal query blocks first, remapped so that every
//    workgroup of one KV head lands on the same XCD (shared L2 for its K/V).
#include <math.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;  // keys per tile

template <int DH, int G>
__global__ __launch_bounds__(kThreads) void gated_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int M,
    int Hq, int Hkv, const float* __restrict__ key_score, const int32_t* __restrict__ pos,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nqb, int total_wg) {
  constexpr int RG = 4 / G;        // 32-row groups per head
  constexpr int BQ = 32 * RG;      // query rows per workgroup
  constexpr int KS = DH / 16;      // k-steps of S^T = K Q^T
  constexpr int DT = DH / 32;      // 32-row tiles of O^T
  constexpr int LDK = DH + 8;      // sK row stride (bf16)
  constexpr int LDV = kBK + 4;     // sVt row stride (bf16)
  constexpr int KCH = kBK * DH / 8;          // 16-byte chunks of a K tile
  constexpr int KL = KCH / kThreads;         // per thread
  constexpr int VCH = (kBK / 2) * (DH / 8);  // key-pair chunks of a V tile
  constexpr int VL = VCH / kThreads;
  static_assert(KL >= 1 && VL >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBK * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][DH * LDV];
  __shared__ __attribute__((aligned(16))) float sBias[2][G][kBK];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
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
  u32x4 rk[KL], rv0[VL], rv1[VL];
  float rb = 0.0f;
  auto load_tile = [&](int kb) {
    const int key0 = kb * kBK;
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      const int c = tid + kThreads * e;
      const int key = c / (DH / 8), part = c % (DH / 8);
      const int kk = key0 + key;
      rk[e] = kk < M ? load16(k + (((size_t)b * M + kk) * Hkv + g) * DH + part * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < VL; ++e) {
      const int c = tid + kThreads * e;
      const int kp = c % 32, j = c / 32;
      const int dc = (j & ~3) | ((j & 1) << 1) | ((j >> 1) & 1);
      const int k0 = key0 + 2 * kp;
      rv0[e] = k0 < M ? load16(v + (((size_t)b * M + k0) * Hkv + g) * DH + dc * 8) : u32x4{0, 0, 0, 0};
      rv1[e] = k0 + 1 < M ? load16(v + (((size_t)b * M + k0 + 1) * Hkv + g) * DH + dc * 8) : u32x4{0, 0, 0, 0};
    }
    if (tid < G * kBK) {
      const int kk = key0 + (tid % kBK);
      rb = kk < M ? key_score[(size_t)b * M + kk] : 0.0f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      const int c = tid + kThreads * e;
      const int key = c / (DH / 8), part = c % (DH / 8);
      store16(&sK[buf][key * LDK + part * 8], rk[e]);
    }
#pragma unroll
    for (int e = 0; e < VL; ++e) {
      const int c = tid + kThreads * e;
      const int kp = c % 32, j = c / 32;
      const int dc = (j & ~3) | ((j & 1) << 1) | ((j >> 1) & 1);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&sVt[buf][(dc * 8) * LDV + 2 * kp]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = rv0[e][w], c2 = rv1[e][w];
        dst[(2 * w) * (LDV / 2)] = (a & 0xFFFFu) | (c2 << 16);
        dst[(2 * w + 1) * (LDV / 2)] = (a >> 16) | (c2 & 0xFFFF0000u);
      }
    }
    if (tid < G * kBK) {
      const int hh = tid / kBK;
      sBias[buf][hh][tid % kBK] = rb * (gain[g * G + hh] * kLog2e);
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) load_tile(kb + 1);

    const int key0 = kb * kBK;
    if (wave_rows && key0 <= rbase + 31) {
      // S^T = K Q^T for the two 32-key halves of the tile
      f32x16 s[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[T][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(&sK[buf][(T * 32 + ql) * LDK + ks * 16 + gq * 8]);
          s[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[T], 0, 0, 0);
        }
      }
      // logits (log2 domain); lane holds keys 32T + 8(i/4) + 4gq + (i%4)
      const bool diag = key0 + kBK - 1 > rbase;
      float mloc = -INFINITY;
#pragma unroll
      for (int T = 0; T < 2; ++T) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 bb = *reinterpret_cast<const f32x4*>(&sBias[buf][hloc][T * 32 + i4 * 8 + gq * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float z = fmaf(s[T][i4 * 4 + i], cq, bb[i]);
            if (diag) {
              const int key = key0 + T * 32 + i4 * 8 + gq * 4 + i;
              z = key > qi ? -INFINITY : z;
            }
            s[T][i4 * 4 + i] = z;
            mloc = fmaxf(mloc, z);
          }
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.0f;
      uint32_t pk[2][8];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(s[T][i] - m_new);
          const float p1 = __builtin_amdgcn_exp2f(s[T][i + 1] - m_new);
          lsum += p0 + p1;
          pk[T][i / 2] = pack_bf16x2(p0, p1);
        }
      }
      l_run = fmaf(l_run, alpha, lsum);
      if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
      }
      // O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int T = st >> 1, h8 = (st & 1) * 4;
        const u32x4 pw = {pk[T][h8], pk[T][h8 + 1], pk[T][h8 + 2], pk[T][h8 + 3]};
        const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const uint16_t* vr = &sVt[buf][(t * 32 + ql) * LDV + st * 16 + gq * 4];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
          const u32x4 vw = {lo[0], lo[1], hi[0], hi[1]};
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), pf, o[t], 0, 0, 0);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_rows) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!q_ok) return;
  const float inv = 1.0f / l_tot;
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
                    uint16_t* out, float* lse, hipStream_t s) {
  constexpr int BQ = 32 * (4 / G);
  const int nqb = (M + BQ - 1) / BQ;
  const long long total = (long long)nqb * Hkv * B;
  if (total <= 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gated_attn_kernel<DH, G>), dim3((unsigned)total), dim3(kThreads), 0, s, q, k, v, M, Hq,
                     Hkv, ks, pos, gain, temp, sm_scale, out, lse, nqb, (int)total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int M, int Hq,
                                  int Hkv, int dh, const float* key_score, const int32_t* pos, const float* gain,
                                  const float* temp, float sm_scale, uint16_t* out, float* lse, hipStream_t s) {
  const int G = Hq / Hkv;
#define TG_ATTN_CASE(DHV, GV)                                                                               \
  if (dh == DHV && G == GV)                                                                                 \
    return launch_t<DHV, GV>(q, k, v, B, M, Hq, Hkv, key_score, pos, gain, temp, sm_scale, out, lse, s);
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
