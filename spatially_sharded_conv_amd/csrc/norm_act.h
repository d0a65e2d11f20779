// GroupNorm apply on one value, shared by the standalone apply pass and the convolution
// operand path that folds the apply in, so that both produce the same bits.
#pragma once

#include <hip/hip_runtime.h>

namespace vaep {

// SiLU(v) = v / (1 + e^-v), with the hardware reciprocal (1 ulp) instead of an IEEE
// division: the result is rounded to the bf16 operand format (or feeds an fp32 conv
// operand) and the division's ten-instruction sequence made the norm passes VALU-bound.
// v -> -inf: e^-v = inf, rcp(inf) = 0, result -0 as with the division.
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// y = x * scale_c + shift_c (scale_c = rstd * gamma_c, shift_c = beta_c - mean * scale_c),
// then SiLU when act.
__device__ __forceinline__ float gn_affine_act(float x, float scale, float shift, bool act) {
  const float y = x * scale + shift;
  return act ? silu(y) : y;
}

}  // namespace vaep
