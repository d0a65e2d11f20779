// The fp8 encoding of the sub-pixel upsample conv's operand and weights.
//
// The sub-pixel conv multiplies an fp32 operand x (the residual stream) by phase-folded
// weights w (fp32 sums of bf16 weights).  Written as x = x_hi + x_lo, w = w_hi + w_lo
// (hi = bf16 rounding, lo = the exact remainder, |lo| <= 2^-9 |hi|), the product is
// x_hi w_hi + x_lo w + x w_lo - x_lo w_lo; the last term is below 2^-18 of the product.
// The first runs in bf16 on the matrix cores.  The two correction terms are 2^-9 of the
// product, so 2-3 significand bits suffice for them: they run as one fp8 matrix product
// with K = 2 x 64 per 64-channel block,
//     A = [e4m3(w 2^s) | e4m3(w_lo 2^(s+9))],  B = [e5m2(x_lo 2^9) | e5m2(x)],
// whose products all carry the factor 2^(s+9); the MFMA's E8M0 scale on A removes it.
// s is chosen per layer from the largest folded weight so that w 2^s stays below 224
// (e4m3 holds 448).  The relative error of the whole product is then below about 2^-11
// of sum |w| |x| (e5m2 rounding 2^-3 and e4m3 rounding 2^-4 of terms that are 2^-9 of
// the product), against 2^-9 for bf16 operands.
//
// Layouts (C a multiple of 64; per pixel of the operand, per output row and tap of the
// weights; 4 bytes per channel, as the bf16 [hi | lo] form they replace):
//   bytes [0, 2C)                    bf16 hi parts (x_hi, or w_hi unscaled)
//   bytes 2C + 128 b + [0, 64)       block b (channels 64 b ..): e5m2(x_lo 2^9) / e4m3(w 2^s)
//   bytes 2C + 128 b + [64, 128)     e5m2(x) / e4m3(w_lo 2^(s+9))
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

namespace vaep {
namespace split8 {

constexpr float kLoScale = 512.f;     // 2^9: x_lo and w_lo are stored scaled by it
constexpr int kLoShift = 9;
constexpr float kWeightTop = 224.f;   // largest scaled folded weight |w| 2^s

// OCP e5m2 / e4m3 of v, round to nearest even (gfx950 conversions).
__device__ __forceinline__ unsigned to_e5m2(float v) {
  return (unsigned)__builtin_amdgcn_cvt_pk_bf8_f32(v, 0.f, 0, false) & 0xffu;
}
__device__ __forceinline__ unsigned to_e4m3(float v) {
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xffu;
}
// Four e5m2 bytes of x_lo 2^9 (lo) and of x (xs) for four channels, packed little-endian.
__device__ __forceinline__ void operand_bytes4(const float* v, unsigned* lo, unsigned* xs) {
  unsigned l = 0, x = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float hi = __bfloat162float(__float2bfloat16(v[e]));
    l |= to_e5m2((v[e] - hi) * kLoScale) << (8 * e);
    x |= to_e5m2(v[e]) << (8 * e);
  }
  *lo = l;
  *xs = x;
}
// Byte offset, within a pixel's 4C bytes, of the fp8 lo byte of channel ch (the x byte
// follows 64 bytes later).
__device__ __forceinline__ long long lo_byte(int C, int ch) {
  return 2LL * C + 128LL * (ch >> 6) + (ch & 63);
}
// Weight scale exponent s for a folded-weight bound m (largest |w|): w 2^s <= kWeightTop.
__device__ __forceinline__ int weight_shift(float m) {
  if (!(m > 0.f)) return 0;
  int s = (int)floorf(log2f(kWeightTop / m));
  return s < -100 ? -100 : (s > 100 ? 100 : s);
}

}  // namespace split8
}  // namespace vaep
