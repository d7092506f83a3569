// MXFP8 block encoding shared by the kernels that quantize ("Bending the
// Scaling Law Curve in Large-Scale Recommendation Systems", Mixed precision;
// OCP Microscaling formats): a block of 32 values with largest magnitude
// amax gets the shared exponent floor(log2(amax)) - 8 (E8M0 byte + 127;
// -127 for an all-zero block) and E4M3 codes of value / 2^shared, clamped to
// +-448 in fp32 and converted with round-to-nearest-even.
#pragma once

#include "common.h"

HSTU_DEV int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  // frexp: amax = f 2^x with f in [0.5, 1), so floor(log2(amax)) = x - 1
  const int s = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
  return min(max(s, -127), 127);
}

// four values -> four E4M3 codes (byte i = value i)
HSTU_DEV uint32_t mx_cvt4(float a, float b, float c, float d, int shared) {
  auto q = [&](float v) { return fminf(fmaxf(ldexpf(v, -shared), -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q(a), q(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q(c), q(d), w, true);
  return (uint32_t)w;
}
