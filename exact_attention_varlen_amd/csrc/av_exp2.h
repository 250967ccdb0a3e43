// av_exp2.h — 2^x on the fused-multiply-add pipe (host and device).
//
// FlashAttention's newest kernels compute part of the softmax exponentials with
// a polynomial on the FMA units instead of the transcendental unit ("FA4
// head_dim=256 B200 Regression Check", Observations: exp2 emulation on FMA
// units; FlashAttention repository guide, Other Components: fast_math). The
// same idea for gfx950, from the published method of Cody and Waite (Software
// Manual for the Elementary Functions, 1980): split x = n + f with n = rint(x)
// and |f| <= 1/2, so 2^x = 2^n * 2^f; 2^f is a degree-3 polynomial fitted here
// (minimax in relative error on [-1/2, 1/2], Remez exchange, exp2_fit.py), and
// 2^n is added to the exponent field as an integer.
//
// Relative error <= 7.5e-5 (the fit) plus float32 rounding, for x >= -125;
// below -125 (and for -inf, a masked score) the result is exactly 0. The
// softmax needs P to bf16 accuracy (2^-9) and its row sum to ~1e-4 for the LSE.
// Ten VALU operations against one v_exp_f32, which on gfx950 costs about two
// VALU issue slots: the forward keeps the hardware exp2 by default and can
// emulate a share of its exponentials when built with AV_EXP2_EMU = K > 0
// (every K-th score of a tile).
#ifndef AV_EXP2_H
#define AV_EXP2_H

#include <math.h>
#include <stdint.h>
#include <string.h>

#ifndef AV_HD
#define AV_HD __host__ __device__
#endif

#ifndef AV_EXP2_EMU
#define AV_EXP2_EMU 0
#endif

namespace av {

AV_HD inline float exp2_fma(float x) {
  constexpr float c0 = 0x1.fff692p-1f, c1 = 0x1.62f31ap-1f, c2 = 0x1.f0de1ap-3f, c3 = 0x1.c3f76p-5f;
  const float xc = fmaxf(x, -125.0f);
  const float n = rintf(xc);
  const float f = xc - n;
  float p = fmaf(c3, f, c2);
  p = fmaf(p, f, c1);
  p = fmaf(p, f, c0);
  int32_t bits;
  memcpy(&bits, &p, 4);
  bits += (int32_t)n * (1 << 23);
  float r;
  memcpy(&r, &bits, 4);
  return x >= -125.0f ? r : 0.0f;
}

// Does score i of a tile take the emulated exponential (AV_EXP2_EMU = K > 0:
// every K-th score)?
AV_HD constexpr bool exp2_emulated(int i) { return AV_EXP2_EMU > 0 && (i % (AV_EXP2_EMU > 0 ? AV_EXP2_EMU : 1)) == 0; }

}  // namespace av

#endif  // AV_EXP2_H
