// Halo-reading convolutions on per-band buffers.
//
// A band's conv reads its own rows plus the kernel-radius halo rows its neighbours
// pushed into the band's halo slots; rows outside the image and columns outside the
// width read as zero, and a band writes only its own output rows (ChituDiffusion
// "VAEP" feature page, conv section; "Static Layer-Wise VAE Decode", operator table,
// "Spatial convolution" row).  Nearest-2x upsampling, which stays local on the pages,
// is fused into the operand load: output pixel (y, x) reads source (floor(y/2),
// floor(x/2)), and the band's upsampled halo row maps to its source halo row.
//
// bf16 path: implicit GEMM on the gfx950 matrix cores, D[co][pixel] = W[co][k] *
// X[k][pixel] with k = (tap, input channel), v_mfma_f32_32x32x16_bf16, fp32
// accumulation.  Operands read from the fp32 residual stream (shortcut, upsample and
// time convs) are split into bf16 hi and lo parts and both are multiplied, so these
// convs see their input to about 16 significand bits.  One 256-thread workgroup computes 128 output channels x 128 pixels of
// one band; 4 waves each own 64 x 64 (2 x 2 MFMA blocks).  K advances 32 channels of one
// tap per step through a double-buffered LDS tile (global -> registers -> LDS while the
// previous tile feeds the MFMAs).
#include "vaep_internal.h"

namespace vaep {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

namespace {

// Input element offset (channel 0) of tap (dt, dy, dx) for compute pixel (n, r, c) of
// band b; *ok is false when the tap reads padding (outside the image or before frame 0).
__device__ __forceinline__ long long tap_source(const BandLayout& in, int b, int n, int r, int c,
                                                int dt, int dy, int dx, int kt, int ks, bool ups,
                                                bool* ok) {
  bool valid = true;
  int sn = n;
  if (kt > 1) {
    const int shift = dt - (kt - 1);         // causal: frames t-2 .. t
    const int t = n % in.frames;
    valid = valid && (t + shift >= 0);
    sn = n + shift;
  }
  const int h = ks >> 1;
  int sr, sc;
  if (ups) {
    const int ur = r + dy - h, uc = c + dx - h;          // coordinates in the upsampled band
    const int gr = 2 * in.row0[b] + ur;
    valid = valid && gr >= 0 && gr < 2 * in.H && uc >= 0 && uc < 2 * in.W;
    sr = ur >> 1;                                        // floor division, -1 -> -1 (halo)
    sc = uc >> 1;
  } else {
    sr = r + dy - h;
    sc = c + dx - h;
    const int gr = in.row0[b] + sr;
    valid = valid && gr >= 0 && gr < in.H && sc >= 0 && sc < in.W;
  }
  *ok = valid;
  return in.off[b] + (((long long)sn * (in.rows[b] + 2) + sr + 1) * in.W + sc) * (long long)in.C;
}

__device__ __forceinline__ long long band_offset(const BandLayout& L, int b, int n, int r, int c) {
  return L.off[b] + (((long long)n * (L.rows[b] + 2) + r + 1) * L.W + c) * (long long)L.C;
}

__device__ __forceinline__ int band_of_tile(const ConvArgs& a, int mt) {
  int b = 0;
  while (b + 1 < a.in.nb && mt >= a.tile_start[b + 1]) ++b;
  return b;
}

__device__ __forceinline__ unsigned short f2bf(float v) {
  __hip_bfloat16 h = __float2bfloat16(v);
  return *reinterpret_cast<unsigned short*>(&h);
}
__device__ __forceinline__ float bf2f(unsigned short u) {
  return __uint_as_float(((unsigned)u) << 16);
}

// Store 4 consecutive channels at element offset `off`: bf16 (8 bytes) or fp32 (16 bytes).
__device__ __forceinline__ void st4(void* base, long long off, const float* v) {
  uint2 p;
  p.x = (unsigned)f2bf(v[0]) | ((unsigned)f2bf(v[1]) << 16);
  p.y = (unsigned)f2bf(v[2]) | ((unsigned)f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(reinterpret_cast<unsigned short*>(base) + off) = p;
}
__device__ __forceinline__ void st4f(void* base, long long off, const float* v) {
  *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
}

// Band-layout fp32 store of 4 channels at (band b, image n, row r, col c) plus the halo
// push into the neighbours' halo slots when r is a boundary row of the band.
__device__ __forceinline__ void store_band4(const BandLayout& L, void* y, int b, int n, int r, int c,
                                            int ch, const float* v) {
  st4f(y, band_offset(L, b, n, r, c) + ch, v);
  if (r == 0 && b > 0) st4f(y, band_offset(L, b - 1, n, L.rows[b - 1], c) + ch, v);
  if (r == L.rows[b] - 1 && b + 1 < L.nb) st4f(y, band_offset(L, b + 1, n, -1, c) + ch, v);
}

// bf16 part of an fp32 value: hi = bf16(v); lo = bf16(v - hi).  hi + lo carries 16
// significand bits, so a product pass over each part recovers the fp32 operand to
// about 2^-17 relative.
__device__ __forceinline__ unsigned short split_part(float v, bool lo) {
  const unsigned short h = f2bf(v);
  return lo ? f2bf(v - bf2f(h)) : h;
}

// 8 channels of the operand source as packed bf16.  bf16 sources load as they are; fp32
// sources (the residual stream) give their hi part, or their lo part when `lo` is set.
template <bool XF32>
__device__ __forceinline__ uint4 load8(const void* base, long long off, bool lo) {
  if (XF32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    uint4 u;
    u.x = (unsigned)split_part(a.x, lo) | ((unsigned)split_part(a.y, lo) << 16);
    u.y = (unsigned)split_part(a.z, lo) | ((unsigned)split_part(a.w, lo) << 16);
    u.z = (unsigned)split_part(b.x, lo) | ((unsigned)split_part(b.y, lo) << 16);
    u.w = (unsigned)split_part(b.z, lo) | ((unsigned)split_part(b.w, lo) << 16);
    return u;
  }
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned short*>(base) + off);
}

template <int KT, int KS, bool UPS, int MODE, bool XF32>
__global__ void __launch_bounds__(256) conv_mfma_bf16(const ConvArgs a) {
  constexpr int BM = kConvTileN;   // output channels per workgroup
  constexpr int BN = kConvTileM;   // pixels per workgroup
  constexpr int BK = 32;
  constexpr int LDK = BK + 8;      // padded LDS row (80 bytes)
  __shared__ __attribute__((aligned(16))) unsigned short sW[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) unsigned short sX[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int mt = blockIdx.x;
  const int band = band_of_tile(a, mt);
  const int tile = mt - a.tile_start[band];
  const int co0 = blockIdx.y * BM;

  const int rows_in = a.in.rows[band];
  const int rows_c = UPS ? 2 * rows_in : rows_in;
  const int wc = UPS ? 2 * a.in.W : a.in.W;
  const int plane = rows_c * wc;
  const long long m_band = (long long)a.in.n_img * plane;
  const int cin = a.cin;
  const int csteps = cin / BK;
  constexpr int TAPS = KT * KS * KS;
  // fp32 sources run the K loop twice: the hi parts, then the lo parts (same weights)
  const int nsteps = TAPS * csteps * (XF32 ? 2 : 1);
  const long long ktot = (long long)TAPS * cin;
  const unsigned short* wg = reinterpret_cast<const unsigned short*>(a.w);

  // Operand-load roles: thread -> (row slots tid/4 and tid/4+64, 8-channel chunk tid%4).
  const int q8 = (tid & 3) * 8;
  int pn0, pr0, pc0, pn1, pr1, pc1;
  bool pv0, pv1;
  {
    const long long p0 = (long long)tile * BN + (tid >> 2);
    const long long p1 = p0 + 64;
    pv0 = p0 < m_band;
    pv1 = p1 < m_band;
    const long long q0 = pv0 ? p0 : 0, q1 = pv1 ? p1 : 0;
    pn0 = (int)(q0 / plane);
    int rem = (int)(q0 - (long long)pn0 * plane);
    pr0 = rem / wc;
    pc0 = rem - pr0 * wc;
    pn1 = (int)(q1 / plane);
    rem = (int)(q1 - (long long)pn1 * plane);
    pr1 = rem / wc;
    pc1 = rem - pr1 * wc;
  }
  const unsigned short* wrow0 = wg + (long long)(co0 + (tid >> 2)) * ktot + q8;
  const unsigned short* wrow1 = wrow0 + 64 * ktot;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int wco = (wave >> 1) * 64;
  const int wpx = (wave & 1) * 64;
  const int frag = (lane & 31) * LDK + (lane >> 5) * 8;
  const int srow = (tid >> 2) * LDK + q8;

  uint4 w0, w1, x0, x1;
  long long xo0 = 0, xo1 = 0;
  bool xk0 = false, xk1 = false;
  int tap = 0, c0 = 0;
  bool lo = false;

#define VAEP_CONV_LOAD()                                                                        \
  {                                                                                             \
    if (c0 == 0) {                                                                              \
      const int dt = tap / (KS * KS), dy = (tap / KS) % KS, dx = tap % KS;                      \
      bool ok;                                                                                  \
      xo0 = tap_source(a.in, band, pn0, pr0, pc0, dt, dy, dx, KT, KS, UPS, &ok) + q8;           \
      xk0 = ok && pv0;                                                                          \
      xo1 = tap_source(a.in, band, pn1, pr1, pc1, dt, dy, dx, KT, KS, UPS, &ok) + q8;           \
      xk1 = ok && pv1;                                                                          \
    }                                                                                           \
    w0 = *reinterpret_cast<const uint4*>(wrow0 + (long long)tap * cin + c0);                    \
    w1 = *reinterpret_cast<const uint4*>(wrow1 + (long long)tap * cin + c0);                    \
    x0 = xk0 ? load8<XF32>(a.x, xo0 + c0, lo) : make_uint4(0, 0, 0, 0);                         \
    x1 = xk1 ? load8<XF32>(a.x, xo1 + c0, lo) : make_uint4(0, 0, 0, 0);                         \
    c0 += BK;                                                                                   \
    if (c0 == cin) {                                                                            \
      c0 = 0;                                                                                   \
      if (++tap == TAPS) {                                                                      \
        tap = 0;                                                                                \
        lo = true;                                                                              \
      }                                                                                         \
    }                                                                                           \
  }
#define VAEP_CONV_STASH(buf)                                                                    \
  {                                                                                             \
    *reinterpret_cast<uint4*>(&sW[buf][srow]) = w0;                                             \
    *reinterpret_cast<uint4*>(&sW[buf][srow + 64 * LDK]) = w1;                                  \
    *reinterpret_cast<uint4*>(&sX[buf][srow]) = x0;                                             \
    *reinterpret_cast<uint4*>(&sX[buf][srow + 64 * LDK]) = x1;                                  \
  }

  VAEP_CONV_LOAD();
  VAEP_CONV_STASH(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) VAEP_CONV_LOAD();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&sW[buf][(wco + 32 * i) * LDK + frag + kk * 16]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sX[buf][(wpx + 32 * j) * LDK + frag + kk * 16]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nsteps) VAEP_CONV_STASH(buf ^ 1);
    __syncthreads();
  }
#undef VAEP_CONV_LOAD
#undef VAEP_CONV_STASH

  // Epilogue.  acc[i][j][v]: channel co0+wco+32i+8(v/4)+4(lane/32)+(v%4), pixel
  // tile*BN+wpx+32j+(lane%32).
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long long p = (long long)tile * BN + wpx + 32 * j + (lane & 31);
    if (p >= m_band) continue;
    const int n = (int)(p / plane);
    const int rem = (int)(p - (long long)n * plane);
    const int r = rem / wc;
    const int c = rem - r * wc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int co = co0 + wco + 32 * i + 8 * g + 4 * (lane >> 5);
        if (co >= a.cout) continue;
        float v[4];
        const float4 bb = *reinterpret_cast<const float4*>(a.bias + co);
        v[0] = acc[i][j][4 * g + 0] + bb.x;
        v[1] = acc[i][j][4 * g + 1] + bb.y;
        v[2] = acc[i][j][4 * g + 2] + bb.z;
        v[3] = acc[i][j][4 * g + 3] + bb.w;
        if (MODE == kModeBand) {
          if (a.res) {
            const float4 rr = *reinterpret_cast<const float4*>(
                reinterpret_cast<const float*>(a.res) + band_offset(a.out, band, n, r, c) + co);
            v[0] += rr.x;
            v[1] += rr.y;
            v[2] += rr.z;
            v[3] += rr.w;
          }
          store_band4(a.out, a.y, band, n, r, c, co, v);
        } else if (MODE == kModeTimeInterleave) {
          const int T = a.in.frames;
          const int t = n % T;
          if (t == 0) continue;                     // z[0] is not used by the layout
          const int bsm = n / T;
          const int half = a.cout >> 1;
          const int on = bsm * (2 * T - 1) + (co < half ? 2 * t - 1 : 2 * t);
          store_band4(a.out, a.y, band, on, r, c, co < half ? co : co - half, v);
        } else if (MODE == kModeQKV) {
          const int cc = a.cout / 3;
          const int tokens = a.in.H * a.in.W;
          const long long tok = (long long)(a.in.row0[band] + r) * a.in.W + c;
          if (co < cc) {
            st4(a.q, ((long long)n * tokens + tok) * cc + co, v);
          } else if (co < 2 * cc) {
            st4(a.k, ((long long)n * tokens + tok) * cc + (co - cc), v);
          } else {
            unsigned short* vt = reinterpret_cast<unsigned short*>(a.vt);
            const long long base = ((long long)n * cc + (co - 2 * cc)) * tokens + tok;
#pragma unroll
            for (int e = 0; e < 4; ++e) vt[base + (long long)e * tokens] = f2bf(v[e]);
          }
        } else {  // kModeFinal: NC[T]HW fp32 output
          const int T = a.final_frames;
          const int bsm = n / T, t = n - bsm * T;
          const long long hw = (long long)a.in.H * a.in.W;
          const long long pix = (long long)(a.in.row0[band] + r) * a.in.W + c;
          float* o = reinterpret_cast<float*>(a.y);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ch = co + e;
            if (ch < a.cout) o[(((long long)bsm * a.cout + ch) * T + t) * hw + pix] = v[e];
          }
        }
      }
    }
  }
}

// fp32 path (small decoders): one thread per (pixel, output channel), same geometry and
// epilogues as the MFMA kernel, fp32 accumulation.
__global__ void __launch_bounds__(128) conv_f32(const ConvArgs a) {
  const int mt = blockIdx.x;
  const int band = band_of_tile(a, mt);
  const int tile = mt - a.tile_start[band];
  const int co = blockIdx.y;
  const int rows_in = a.in.rows[band];
  const bool ups = a.ups != 0;
  const int rows_c = ups ? 2 * rows_in : rows_in;
  const int wc = ups ? 2 * a.in.W : a.in.W;
  const int plane = rows_c * wc;
  const long long p = (long long)tile * kConvTileM + threadIdx.x;
  if (p >= (long long)a.in.n_img * plane || co >= a.cout) return;
  const int n = (int)(p / plane);
  const int rem = (int)(p - (long long)n * plane);
  const int r = rem / wc, c = rem - (rem / wc) * wc;
  const float* xg = reinterpret_cast<const float*>(a.x);
  const float* wg = reinterpret_cast<const float*>(a.w);
  const int taps = a.kt * a.ks * a.ks;
  const long long ktot = (long long)taps * a.cin;
  float acc = 0.f;
  for (int tap = 0; tap < taps; ++tap) {
    const int dt = tap / (a.ks * a.ks), dy = (tap / a.ks) % a.ks, dx = tap % a.ks;
    bool ok;
    const long long off = tap_source(a.in, band, n, r, c, dt, dy, dx, a.kt, a.ks, ups, &ok);
    if (!ok) continue;
    const float* wr = wg + (long long)co * ktot + (long long)tap * a.cin;
    for (int ci = 0; ci < a.cin; ++ci) acc = fmaf(wr[ci], xg[off + ci], acc);
  }
  float v = acc + a.bias[co];
  if (a.mode == kModeBand) {
    const long long o = band_offset(a.out, band, n, r, c) + co;
    if (a.res) v += reinterpret_cast<const float*>(a.res)[o];
    float* y = reinterpret_cast<float*>(a.y);
    y[o] = v;
    if (r == 0 && band > 0) y[band_offset(a.out, band - 1, n, a.out.rows[band - 1], c) + co] = v;
    if (r == a.out.rows[band] - 1 && band + 1 < a.out.nb) y[band_offset(a.out, band + 1, n, -1, c) + co] = v;
  } else if (a.mode == kModeTimeInterleave) {
    const int T = a.in.frames;
    const int t = n % T;
    if (t == 0) return;
    const int half = a.cout >> 1;
    const int on = (n / T) * (2 * T - 1) + (co < half ? 2 * t - 1 : 2 * t);
    const int ch = co < half ? co : co - half;
    float* y = reinterpret_cast<float*>(a.y);
    y[band_offset(a.out, band, on, r, c) + ch] = v;
    if (r == 0 && band > 0) y[band_offset(a.out, band - 1, on, a.out.rows[band - 1], c) + ch] = v;
    if (r == a.out.rows[band] - 1 && band + 1 < a.out.nb) y[band_offset(a.out, band + 1, on, -1, c) + ch] = v;
  } else if (a.mode == kModeQKV) {
    const int cc = a.cout / 3;
    const int tokens = a.in.H * a.in.W;
    const long long tok = (long long)(a.in.row0[band] + r) * a.in.W + c;
    if (co < cc) reinterpret_cast<float*>(a.q)[((long long)n * tokens + tok) * cc + co] = v;
    else if (co < 2 * cc) reinterpret_cast<float*>(a.k)[((long long)n * tokens + tok) * cc + co - cc] = v;
    else reinterpret_cast<float*>(a.vt)[((long long)n * cc + co - 2 * cc) * tokens + tok] = v;
  } else {
    const int T = a.final_frames;
    const int bsm = n / T, t = n - bsm * T;
    const long long hw = (long long)a.in.H * a.in.W;
    const long long pix = (long long)(a.in.row0[band] + r) * a.in.W + c;
    reinterpret_cast<float*>(a.y)[(((long long)bsm * a.cout + co) * T + t) * hw + pix] = v;
  }
}

template <int KT, int KS, bool UPS, int MODE>
hipError_t go(const ConvArgs& a, hipStream_t s) {
  dim3 grid(a.tiles_total, a.cout_pad / kConvTileN);
  if (a.x_f32)
    hipLaunchKernelGGL((conv_mfma_bf16<KT, KS, UPS, MODE, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((conv_mfma_bf16<KT, KS, UPS, MODE, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(ConvArgs& a, int dtype, hipStream_t s) {
  const bool ups = a.ups != 0;
  int t = 0;
  for (int b = 0; b < a.in.nb; ++b) {
    a.tile_start[b] = t;
    const long long m = (long long)a.in.n_img * (ups ? 2 : 1) * a.in.rows[b] * (ups ? 2 : 1) * a.in.W;
    t += (int)((m + kConvTileM - 1) / kConvTileM);
  }
  a.tile_start[a.in.nb] = t;
  a.tiles_total = t;
  if (t == 0) return hipSuccess;
  if (dtype == VAEP_DTYPE_F32) {
    dim3 grid(t, a.cout);
    hipLaunchKernelGGL(conv_f32, grid, dim3(kConvTileM), 0, s, a);
    return hipGetLastError();
  }
  const int kt = a.kt, ks = a.ks, m = a.mode;
  if (kt == 1 && ks == 3 && !ups && m == kModeBand) return go<1, 3, false, kModeBand>(a, s);
  if (kt == 1 && ks == 3 && ups && m == kModeBand) return go<1, 3, true, kModeBand>(a, s);
  if (kt == 1 && ks == 1 && !ups && m == kModeBand) return go<1, 1, false, kModeBand>(a, s);
  if (kt == 1 && ks == 1 && !ups && m == kModeQKV) return go<1, 1, false, kModeQKV>(a, s);
  if (kt == 1 && ks == 3 && !ups && m == kModeFinal) return go<1, 3, false, kModeFinal>(a, s);
  if (kt == 3 && ks == 3 && !ups && m == kModeBand) return go<3, 3, false, kModeBand>(a, s);
  if (kt == 3 && ks == 3 && !ups && m == kModeFinal) return go<3, 3, false, kModeFinal>(a, s);
  if (kt == 3 && ks == 1 && !ups && m == kModeTimeInterleave)
    return go<3, 1, false, kModeTimeInterleave>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace vaep
