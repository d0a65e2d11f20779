// Narrow-output convolution: the decoder's last conv (a few image channels out of 96-512
// normalised channels), written straight into the NC[T]HW output tensor.
//
// Same operation and band rules as conv.hip (ChituDiffusion "VAEP" feature page, conv
// section; "Static Layer-Wise VAE Decode", operator table, "Spatial convolution" row):
// the band reads its own rows and the neighbours' halo rows, zero padding only outside
// the image (and before frame 0 for causal 3x3x3 kernels).
//
// Layout of the work: D[pixel][co] = X[pixel][k] W[k][co] with
// v_mfma_f32_16x16x32_bf16, pixels as the 16 rows and the output channels (zero-padded
// to 16) as the columns, so the matrix cores spend their width on pixels rather than on
// a mostly empty output-channel tile.  One 256-thread workgroup covers 256 pixels of one
// band (4 waves x 4 blocks of 16); operand fragments load from global memory directly
// (each input pixel is re-read by the kernel taps from L1/L2).
#include "vaep_internal.h"

namespace vaep {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

namespace {

constexpr int kNarrowPix = 256;
constexpr unsigned kPadOffset = 0x80000000u;   // past the buffer resource: loads return 0

__device__ __forceinline__ int band_of_tile(const ConvArgs& a, int mt) {
  int b = 0;
  while (b + 1 < a.in.nb && mt >= a.tile_start[b + 1]) ++b;
  return b;
}

template <int KT, int KS, int NC>
__global__ void __launch_bounds__(256) conv_narrow(const ConvArgs a) {
  constexpr int TAPS = KT * KS * KS;   // NC: 32-channel chunks of the input
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int mt = blockIdx.x;
  const int band = band_of_tile(a, mt);
  const int tile = mt - a.tile_start[band];
  const int rows_in = a.in.rows[band];
  const int W = a.in.W;
  const int plane = rows_in * W;
  const long long m_band = (long long)a.in.n_img * plane;
  const int C = a.in.C;

  // input resource: the band rows this tile can read (see conv_wide)
  long long first_slot, last_slot;
  {
    const long long p0 = (long long)tile * kNarrowPix;
    long long p1 = p0 + kNarrowPix - 1;
    if (p1 >= m_band) p1 = m_band - 1;
    const int n0 = (int)(p0 / plane), r0 = (int)((p0 - (long long)n0 * plane) / W);
    const int n1 = (int)(p1 / plane), r1 = (int)((p1 - (long long)n1 * plane) / W);
    first_slot = (long long)(n0 - (KT - 1)) * (rows_in + 2) + r0;
    if (first_slot < 0) first_slot = 0;
    last_slot = (long long)n1 * (rows_in + 2) + r1 + 2;
  }
  const long long row_elems = (long long)W * C;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(a.x) + a.in.off[band] + first_slot * row_elems),
      0, (int)((last_slot - first_slot + 1) * row_elems * 2), 0x00020000);

  // A fragments: pixel tile*256 + 64*wave + 16*rb + lane%16, channels 8*(lane/16) of a chunk
  const int kc = 8 * (lane >> 4);
  unsigned pbase[4];
  int pmask[4];
  const int H = a.in.H, g0 = a.in.row0[band];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const long long p = (long long)tile * kNarrowPix + 64 * wave + 16 * rb + (lane & 15);
    const bool ok = p < m_band;
    const long long q = ok ? p : 0;
    const int n = (int)(q / plane);
    const int rem = (int)(q - (long long)n * plane);
    const int r = rem / W, c = rem - (rem / W) * W;
    const long long slot = (long long)n * (rows_in + 2) + r + 1;
    pbase[rb] = (unsigned)(((slot - first_slot) * W + c) * C * 2 + kc * 2);
    const int g = g0 + r;
    int m = 2 | 16;
    m |= (g - 1 >= 0) ? 1 : 0;
    m |= (g + 1 < H) ? 4 : 0;
    m |= (c - 1 >= 0) ? 8 : 0;
    m |= (c + 1 < W) ? 32 : 0;
    const int t = n % a.in.frames;
#pragma unroll
    for (int dt = 0; dt < KT; ++dt) m |= (t + dt - (KT - 1) >= 0) ? (64 << dt) : 0;
    pmask[rb] = ok ? m : 0;
  }
  // B fragments: W[co = lane%16][tap][c0 + 8*(lane/16) ..] (rows past cout are zero)
  const long long ktot = (long long)TAPS * C;
  const unsigned short* wrow = reinterpret_cast<const unsigned short*>(a.w) + (long long)(lane & 15) * ktot + kc;

  f32x4_t acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // all fragments of one tap are loaded together, one tap ahead of the MFMAs
  bf16x8_t ax[2][NC][4], bw[2][NC];
#define VAEP_LOAD_TAP(buf, tap)                                                                 \
  {                                                                                             \
    const int dt = (tap) / (KS * KS), sy = ((tap) / KS) % KS - KS / 2, sx = (tap) % KS - KS / 2; \
    const int need = (1 << (sy + 1)) | (8 << (sx + 1)) | (64 << dt);                             \
    const int delta = (int)((((long long)(dt - (KT - 1)) * (rows_in + 2) + sy) * W + sx) * C * 2); \
    _Pragma("unroll") for (int rb = 0; rb < 4; ++rb) {                                          \
      const unsigned off = ((pmask[rb] & need) == need) ? (unsigned)((int)pbase[rb] + delta) : kPadOffset; \
      _Pragma("unroll") for (int ch = 0; ch < NC; ++ch)                                         \
        ax[buf][ch][rb] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)off, ch * 64, 0)); \
    }                                                                                           \
    _Pragma("unroll") for (int ch = 0; ch < NC; ++ch)                                           \
      bw[buf][ch] = *reinterpret_cast<const bf16x8_t*>(wrow + (long long)(tap) * C + 32 * ch);   \
  }
#define VAEP_MFMA_TAP(buf)                                                                      \
  _Pragma("unroll") for (int ch = 0; ch < NC; ++ch)                                             \
    _Pragma("unroll") for (int rb = 0; rb < 4; ++rb)                                            \
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[buf][ch][rb], bw[buf][ch], acc[rb], 0, 0, 0);
  VAEP_LOAD_TAP(0, 0);
  for (int tap = 0; tap < TAPS; tap += 2) {
    if (tap + 1 < TAPS) VAEP_LOAD_TAP(1, tap + 1);
    VAEP_MFMA_TAP(0);
    if (tap + 1 >= TAPS) break;
    if (tap + 2 < TAPS) VAEP_LOAD_TAP(0, tap + 2);
    VAEP_MFMA_TAP(1);
  }
#undef VAEP_LOAD_TAP
#undef VAEP_MFMA_TAP

  // lane holds output channel lane%16 for pixels 16*rb + 4*(lane/16) + v of the wave
  const int co = lane & 15;
  if (co >= a.cout) return;
  const float bias = a.bias[co];
  const int T = a.final_frames;
  const long long hw = (long long)a.in.H * W;
  float* out = reinterpret_cast<float*>(a.y);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const long long p = (long long)tile * kNarrowPix + 64 * wave + 16 * rb + 4 * (lane >> 4) + v;
      if (p >= m_band) continue;
      const int n = (int)(p / plane);
      const int rem = (int)(p - (long long)n * plane);
      const int r = rem / W, c = rem - (rem / W) * W;
      const int bs = n / T, t = n - bs * T;
      const long long pix = a.out_transposed ? (long long)c * a.in.H + (g0 + r) : (long long)(g0 + r) * W + c;
      out[(((long long)bs * a.cout + co) * T + t) * hw + pix] = acc[rb][v] + bias;
    }
}

}  // namespace

bool conv_narrow_fits(const ConvArgs& a) {
  return a.mode == kModeFinal && a.cout <= 16 && a.cout_pad >= 16 && (a.in.C == 96 || a.in.C == 128) && !a.x_f32 &&
         !a.x_split && !a.ups && a.ks == 3 && (a.kt == 1 || a.kt == 3);
}

hipError_t launch_conv_narrow(ConvArgs& a, hipStream_t s) {
  for (int b = 0; b < a.in.nb; ++b)
    if ((long long)a.kt * (a.in.rows[b] + 2) * a.in.W * a.in.C * 2 + 2LL * kNarrowPix * a.in.C * 2 >= (1LL << 31) - 4096)
      return hipErrorInvalidValue;
  int t = 0;
  for (int b = 0; b < a.in.nb; ++b) {
    a.tile_start[b] = t;
    const long long m = (long long)a.in.n_img * a.in.rows[b] * a.in.W;
    t += (int)((m + kNarrowPix - 1) / kNarrowPix);
  }
  a.tile_start[a.in.nb] = t;
  a.tiles_total = t;
  a.kernel_used = VAEP_KERNEL_CONV_NARROW;
  if (t == 0) return hipSuccess;
  const bool c128 = a.in.C == 128;
  if (a.kt == 3 && c128)
    hipLaunchKernelGGL((conv_narrow<3, 3, 4>), dim3(t), dim3(256), 0, s, a);
  else if (a.kt == 3)
    hipLaunchKernelGGL((conv_narrow<3, 3, 3>), dim3(t), dim3(256), 0, s, a);
  else if (c128)
    hipLaunchKernelGGL((conv_narrow<1, 3, 4>), dim3(t), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((conv_narrow<1, 3, 3>), dim3(t), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace vaep
