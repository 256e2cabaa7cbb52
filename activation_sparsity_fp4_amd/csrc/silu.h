// SiLU-gated product of a gate and an up projection (glue between a fused
// gate|up projection and the down projection; not part of the method), shared
// by the standalone kernel and the fused gate|up epilogue so that both round
// identically: h = bf16_rne(silu(g) * u).
#pragma once

#include "sharq_device.h"

namespace sharq {

// bf16 bits of f, rounded to nearest even (the hardware converter).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// silu(g) * u without overflow: with h = exp(-|g| / 2) (in (0, 1]),
//   g >= 0: g * u / (1 + h^2)           (h^2 = exp(-g))
//   g <  0: ((g * u) * h) * h / (1 + h^2)  (= g u e^g / (1 + e^g))
// The negative branch multiplies by the two half-exponentials one at a time so
// results down to the fp32 normal range survive even when e^g alone is subnormal.
// 1 / den (den in [1, 2]) is the hardware reciprocal (1 ulp): with the fast
// exponential the fp32 result is a few ulp from silu(g) * u, far inside the
// bf16 rounding that follows.
__device__ __forceinline__ float silu_times(float g, float u) {
  const float h = __expf(-0.5f * fabsf(g));
  const float r = __builtin_amdgcn_rcpf(1.0f + h * h);
  const float gu = g * u;
  return (g >= 0.0f ? gu : (gu * h) * h) * r;
}

}  // namespace sharq
