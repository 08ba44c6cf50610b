// The YaRN rotation of one pair of head dimensions, shared by every kernel
// that applies it, so that all of them round the same fp64 expressions in
// the same way ([P1] "YaRN, and matching what vLLM actually does": mscale
// multiplies cos and sin inside the rope, on the rotary dimensions only).
#pragma once

#include "device_common.h"

namespace yrk {

// mscale * cos and mscale * sin of the angle pos * inv_freq (fp64: at
// positions near 2^20 an fp32 angle is off by up to ~0.06 rad).
__device__ __forceinline__ void rope_cos_sin(int32_t pos, double inv_freq, double mscale,
                                             double* c, double* s) {
  double sn, cs;
  sincos((double)pos * inv_freq, &sn, &cs);
  *c = mscale * cs;
  *s = mscale * sn;
}

// Rotated pair (x1 = element i, x2 = element i + rotary_dim / 2), each
// rounded once to bf16.  Contraction into fused multiply-adds is off so that
// the products are rounded the same way wherever this is inlined.
__device__ __forceinline__ uint16_t rope_first(double x1, double x2, double c, double s) {
#pragma clang fp contract(off)
  return f64_to_bf16(x1 * c - x2 * s);
}
__device__ __forceinline__ uint16_t rope_second(double x1, double x2, double c, double s) {
#pragma clang fp contract(off)
  return f64_to_bf16(x2 * c + x1 * s);
}

}  // namespace yrk
