// Fixed fp32 score recipe for the expert-selection key.
//
// With a selection bias the top-k compares score(logit) + bias ("Sparse MoE
// FFN for DFlash-family drafters", What's here: MoEGate, sqrtsoftplus routing
// with the aux-loss-free balancing bias).  The selection is an integer
// decision taken from floating point, so the score is evaluated by one fully
// specified sequence of binary32 operations, each correctly rounded, with no
// fused multiply-add:
//
//   exp32(x): NaN -> NaN, x > 89 -> +inf, x < -104 -> +0; else
//     n = rint(x * LOG2E);  r = (x - n*C1) - n*C2     (Cody-Waite reduction,
//     C1 = ln 2 truncated to 16 significant bits, C2 = fl32(ln 2 - C1));
//     p = Horner form of the degree-7 Taylor polynomial of exp(r);
//     result = (p * 2^floor(n/2)) * 2^(n - floor(n/2)).
//   log1p32(y), 0 <= y <= 1: s = y / (2 + y), z = s*s,
//     q = Horner form of sum_{i=0..8} z^i / (2i+1), result = (2*s) * q
//     (log1p(y) = 2 atanh(y / (2 + y))).
//   sigmoid32(l) = 1 / (1 + exp32(-l))
//   sqrtsoftplus32(l) = sqrt(max(l, 0) + log1p32(exp32(-|l|)))
//   softmax denominators: lane partials over strided experts, then an
//     xor-butterfly over the 64 lanes (see the router kernel).
//
// This file must be compiled with -ffp-contract=off; the pragma below
// repeats the requirement locally.
#pragma once
#include "common.h"

namespace moe {
namespace score32 {

#pragma clang fp contract(off)

constexpr float kLog2e = 1.4426950408889634f;
// ln 2 = 0.693147180559945309...; its first 16 significant bits and the rest.
constexpr float kC1 = 0.693145751953125f;
constexpr float kC2 = (float)(0.6931471805599453094172321 - 0.693145751953125);

MOE_DEV float pow2i(int n) { return __int_as_float((n + 127) << 23); }

MOE_DEV float exp32(float x) {
#pragma clang fp contract(off)
  if (x != x) return x;
  if (x > 89.0f) return __int_as_float(0x7f800000);
  if (x < -104.0f) return 0.0f;
  const float n = __builtin_rintf(x * kLog2e);
  const float r = (x - n * kC1) - n * kC2;
  float p = (float)(1.0 / 5040.0);
  p = p * r + (float)(1.0 / 720.0);
  p = p * r + (float)(1.0 / 120.0);
  p = p * r + (float)(1.0 / 24.0);
  p = p * r + (float)(1.0 / 6.0);
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const int ni = (int)n;
  const int n1 = ni >> 1;  // floor(n / 2)
  const int n2 = ni - n1;
  return (p * pow2i(n1)) * pow2i(n2);
}

MOE_DEV float log1p32(float y) {
#pragma clang fp contract(off)
  const float s = y / (2.0f + y);
  const float z = s * s;
  float q = (float)(1.0 / 17.0);
  q = q * z + (float)(1.0 / 15.0);
  q = q * z + (float)(1.0 / 13.0);
  q = q * z + (float)(1.0 / 11.0);
  q = q * z + (float)(1.0 / 9.0);
  q = q * z + (float)(1.0 / 7.0);
  q = q * z + (float)(1.0 / 5.0);
  q = q * z + (float)(1.0 / 3.0);
  q = q * z + 1.0f;
  return (2.0f * s) * q;
}

MOE_DEV float sigmoid32(float l) {
#pragma clang fp contract(off)
  return 1.0f / (1.0f + exp32(-l));
}

MOE_DEV float sqrtsoftplus32(float l) {
#pragma clang fp contract(off)
  const float sp = fmaxf(l, 0.0f) + log1p32(exp32(-fabsf(l)));
  return __builtin_sqrtf(sp);
}

}  // namespace score32
}  // namespace moe
