// Rotary position embedding on the original positions, shared by the
// forward and the backward of the token-gated attention.  TokenGate paper,
// Appendix C.4: the kept tokens keep their original positions for the
// position encoding of the layers above the gate.  Rotate-half form: pair
// (x_i, x_{i+DH/2}) turns by pos * base^(-2i/DH).  The angle is formed and
// reduced modulo 2 pi in fp64 (2 pi split into two doubles), so that its
// fp32 sine and cosine are accurate to a few ulp at any position.
#pragma once

#include <math.h>

#include "tg_device.h"

namespace tg {
namespace rope {

// sine and cosine of pos * freq[i0 + i] for 8 consecutive pairs
__device__ __forceinline__ void sincos8(double pos, const double* freq, int i0, float (&c)[8], float (&s)[8]) {
  constexpr double kInv2Pi = 0.15915494309189535, k2PiHi = 6.283185307179586, k2PiLo = 2.4492935982947064e-16;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double th = pos * freq[i0 + i];
    const double n = rint(th * kInv2Pi);
    const double red = fma(-n, k2PiLo, fma(-n, k2PiHi, th));  // th - 2 pi n, |red| <= pi (+ rounding)
    sincosf((float)red, &s[i], &c[i]);
  }
}

// base^(-2i/DH) for the DH/2 pairs (fp64)
__device__ __forceinline__ double inv_freq(double base, int i, int DH) {
  return pow(base, -2.0 * (double)i / (double)DH);
}

// Rotates one head row, pairs i = i0 .. i0 + 7, by the angles whose cosines
// and sines are c[], s[] (fp32, products fused), rounding to bf16 (nearest
// even).
// row8_rotate takes the two 16-byte pieces already loaded: a = pairs' first
// elements x_{i0..i0+7}, bv = their partners x_{DH/2+i0..}.
template <int DH>
__device__ __forceinline__ void row8_rotate(u32x4 a, u32x4 bv, uint16_t* dst, int i0, const float (&c)[8],
                                            const float (&s)[8]) {
  constexpr int HALF = DH / 2;
  u32x4 oa, ob;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x1l = bf16_lo(a[j]), x1h = bf16_hi(a[j]), x2l = bf16_lo(bv[j]), x2h = bf16_hi(bv[j]);
    const int il = 2 * j, ih = 2 * j + 1;
    oa[j] = pack_bf16x2(fmaf(x1l, c[il], -(x2l * s[il])), fmaf(x1h, c[ih], -(x2h * s[ih])));
    ob[j] = pack_bf16x2(fmaf(x2l, c[il], x1l * s[il]), fmaf(x2h, c[ih], x1h * s[ih]));
  }
  store16(dst + i0, oa);
  store16(dst + HALF + i0, ob);
}
template <int DH>
__device__ __forceinline__ void row8(const uint16_t* src, uint16_t* dst, int i0, const float (&c)[8],
                                     const float (&s)[8]) {
  row8_rotate<DH>(load16(src + i0), load16(src + DH / 2 + i0), dst, i0, c, s);
}

// The transposed rotation of a gradient row (fp32 in, bf16 out): for the
// forward map x1' = x1 c - x2 s, x2' = x2 c + x1 s, the gradient with
// respect to (x1, x2) is (g1 c + g2 s, g2 c - g1 s).
template <int DH>
__device__ __forceinline__ void row8_transposed(const float* src, uint16_t* dst, int i0, const float (&c)[8],
                                                const float (&s)[8]) {
  constexpr int HALF = DH / 2;
  u32x4 oa, ob;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float g1[2], g2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      g1[h] = src[i0 + 2 * j + h];
      g2[h] = src[HALF + i0 + 2 * j + h];
    }
    const int il = 2 * j, ih = 2 * j + 1;
    oa[j] = pack_bf16x2(fmaf(g1[0], c[il], g2[0] * s[il]), fmaf(g1[1], c[ih], g2[1] * s[ih]));
    ob[j] = pack_bf16x2(fmaf(g2[0], c[il], -(g1[0] * s[il])), fmaf(g2[1], c[ih], -(g1[1] * s[ih])));
  }
  store16(dst + i0, oa);
  store16(dst + HALF + i0, ob);
}

}  // namespace rope
}  // namespace tg
