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
#include "conv_gn_stats.h"
#include "conv_epilogue.h"
#include "split8.h"
#include "norm_act.h"

#include <type_traits>

namespace vaep {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;   // 16 bytes, native vector

namespace {

// Input element offset (channel 0) of tap (dt, dy, dx) for compute pixel (n, r, c) of
// band b; *ok is false when the tap reads padding (outside the image or before frame 0).
__device__ __forceinline__ long long tap_source(const BandLayout& in, int b, int n, int r, int c,
                                                int dt, int dy, int dx, int kt, int ks, bool ups,
                                                bool* ok, bool down = false) {
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
  if (down) {
    // stride 2, no padding above or left of the image, one zero row / column below / right
    sr = 2 * r + dy;
    sc = 2 * c + dx;
    const int gr = in.row0[b] + sr;
    valid = valid && gr < in.H && sc < in.W;
  } else if (ups) {
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
// 4 channels as bf16 hi parts at `off` and lo parts `half` channels later.
__device__ __forceinline__ void st4split(void* base, long long off, int half, const float* v) {
  unsigned short h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = f2bf(v[e]);
    l[e] = f2bf(v[e] - bf2f(h[e]));
  }
  unsigned short* p = reinterpret_cast<unsigned short*>(base) + off;
  *reinterpret_cast<uint2*>(p) = make_uint2((unsigned)h[0] | ((unsigned)h[1] << 16), (unsigned)h[2] | ((unsigned)h[3] << 16));
  *reinterpret_cast<uint2*>(p + half) = make_uint2((unsigned)l[0] | ((unsigned)l[1] << 16), (unsigned)l[2] | ((unsigned)l[3] << 16));
}

// Band-layout fp32 store of 4 channels at (band b, image n, row r, col c) plus the halo
// push into the neighbours' halo slots when r is a boundary row of the band.
__device__ __forceinline__ void store_band4(const BandLayout& L, void* y, int b, int n, int r, int c,
                                            int ch, const float* v) {
  st4f(y, band_offset(L, b, n, r, c) + ch, v);
  if (r == 0 && b > 0) st4f(y, band_offset(L, b - 1, n, L.rows[b - 1], c) + ch, v);
  if (r == L.rows[b] - 1 && b + 1 < L.nb) st4f(y, band_offset(L, b + 1, n, -1, c) + ch, v);
}
// 4 channels in the sub-pixel operand encoding (split8.h) of a pixel starting at element
// `pix` of a layout of 2 x `half` bf16 elements per pixel.
__device__ __forceinline__ void st4split8(void* base, long long pix, int half, int ch, const float* v) {
  uint2 p;
  p.x = (unsigned)f2bf(v[0]) | ((unsigned)f2bf(v[1]) << 16);
  p.y = (unsigned)f2bf(v[2]) | ((unsigned)f2bf(v[3]) << 16);
  unsigned short* px = reinterpret_cast<unsigned short*>(base) + pix;
  *reinterpret_cast<uint2*>(px + ch) = p;
  unsigned lo, xs;
  split8::operand_bytes4(v, &lo, &xs);
  unsigned char* f = reinterpret_cast<unsigned char*>(px) + split8::lo_byte(half, ch);
  *reinterpret_cast<unsigned*>(f) = lo;
  *reinterpret_cast<unsigned*>(f + 64) = xs;
}

// bf16 part of an fp32 value: hi = bf16(v); lo = bf16(v - hi).  hi + lo carries 16
// significand bits, so a product pass over each part recovers the fp32 operand to
// about 2^-17 relative.
__device__ __forceinline__ unsigned short split_part(float v, bool lo) {
  const unsigned short h = f2bf(v);
  return lo ? f2bf(v - bf2f(h)) : h;
}

// Buffer resource over [base, base + bytes): loads outside the range return zeros, which
// is how padding taps read (their offset is set past the end).  dword3 = raw buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
constexpr unsigned kPadOffset = 0x80000000u;   // past every band buffer (< 2 GiB, host-checked)

// 8 channels of the operand source as packed bf16 at byte offset voff + soff.  bf16
// sources load as they are; fp32 sources (the residual stream) give their hi part, or
// their lo part when `lo` is set.
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
template <bool XF32>
__device__ __forceinline__ u32x4_t load8(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff, bool lo) {
  if (XF32) {
    const f32x4_t a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
    const f32x4_t b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff + 16, soff, 0));
    u32x4_t u;
    u.x = (unsigned)split_part(a.x, lo) | ((unsigned)split_part(a.y, lo) << 16);
    u.y = (unsigned)split_part(a.z, lo) | ((unsigned)split_part(a.w, lo) << 16);
    u.z = (unsigned)split_part(b.x, lo) | ((unsigned)split_part(b.y, lo) << 16);
    u.w = (unsigned)split_part(b.z, lo) | ((unsigned)split_part(b.w, lo) << 16);
    return u;
  }
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}

// Workgroup id -> tile id so that the 8 XCDs (which receive workgroups round-robin)
// each work on a contiguous run of tiles: neighbouring pixel tiles share halo rows in
// that XCD's L2.  A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int lin, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = lin & 7, i = lin >> 3;
  return x * q + (x < r ? x : r) + i;
}

// Expand a statement for j = 0 .. NP-1 (NP = 2 or 4) with j a compile-time constant, so
// that every array index below is static and the arrays live in registers.
#define VAEP_FOR_J(...)                                                       \
  {                                                                           \
    { constexpr int j = 0; __VA_ARGS__ }                                      \
    { constexpr int j = 1; __VA_ARGS__ }                                      \
    if constexpr (NP > 2) {                                                   \
      { constexpr int j = 2; __VA_ARGS__ }                                    \
      { constexpr int j = 3; __VA_ARGS__ }                                    \
    }                                                                         \
  }

template <int KT, int KS, bool UPS, int MODE, bool XF32, int BK, bool XN = false, bool DS = false>
__global__ void __launch_bounds__(256, 2) conv_mfma_bf16(const ConvArgs a) {
  static_assert(!(DS && (UPS || KS != 3 || KT != 1 || XN)), "stride 2 for plain 3x3 2-D convs");
  constexpr int BM = kConvTileN;   // output channels per workgroup
  constexpr int BN = kConvTileM;   // pixels per workgroup
  // BK: K per pipeline step (64, or 32 when Cin is not a multiple of 64), one tap
  constexpr int LDK = BK + 8;      // LDS row stride (144 bytes for BK 64): conflict-free reads
  constexpr int CH = BK / 8;       // 16-byte chunks per tile row
  constexpr int RP = 256 / CH;     // tile rows covered by one pass of the 256 threads
  constexpr int NP = BN / RP;      // passes per tile
  __shared__ __attribute__((aligned(16))) unsigned short sW[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) unsigned short sX[2][BN * LDK];
  // XN (folded GroupNorm apply): the tile's image's (scale, shift) per input channel
  __shared__ __attribute__((aligned(16))) float sN[XN ? 2 * 512 : 4];
  static_assert(!(XN && XF32), "the folded apply reads the raw fp32 input in one pass");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int mt = lin % gridDim.x;
  const int band = band_of_tile(a, mt);
  const int tile = mt - a.tile_start[band];
  const int co0 = (lin / gridDim.x) * BM;

  const int rows_in = a.in.rows[band];
  const int rows_c = UPS ? 2 * rows_in : (DS ? rows_in / 2 : rows_in);
  const int wc = UPS ? 2 * a.in.W : (DS ? a.in.W / 2 : a.in.W);
  const int plane = rows_c * wc;
  const long long m_band = (long long)a.in.n_img * plane;
  const int cin = a.cin;
  constexpr int TAPS = KT * KS * KS;
  // fp32 sources run the K loop twice: the hi parts, then the lo parts (same weights)
  const int nsteps = TAPS * (cin / BK) * (XF32 ? 2 : 1);
  const long long ktot = (long long)TAPS * cin;

  // Load roles: thread -> rows tid/CH + RP*j (j < NP) of both tiles, 8-channel chunk tid%CH.
  const int rs = tid / CH;
  const int q8 = (tid % CH) * 8;
  int pn[NP], pr[NP], pc[NP];
  bool pv[NP];
  VAEP_FOR_J({
    const long long p = (long long)tile * BN + rs + RP * j;
    pv[j] = p < m_band;
    const long long q = pv[j] ? p : 0;
    pn[j] = (int)(q / plane);
    const int rem = (int)(q - (long long)pn[j] * plane);
    pr[j] = rem / wc;
    pc[j] = rem - pr[j] * wc;
  });
  constexpr int XB = (XF32 || XN) ? 4 : 2;   // bytes per input element
  // weights: [cout_pad][taps][cin] bf16; thread rows co0 + rs + RP*j, chunk q8
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(a.w, (unsigned)((long long)a.cout_pad * ktot * 2));
  unsigned wvo[NP];
  VAEP_FOR_J({ wvo[j] = (unsigned)(((long long)(co0 + rs + RP * j) * ktot + q8) * 2); });
  // input: the rows of this band's buffer the tile can read.  Row slot of (image n, row
  // r in [-1, rows]) is n*(rows+2) + r + 1; the tile reads from the slot of its first
  // pixel's top neighbour (KT-1 frames back for causal convs) to its last pixel's bottom
  // neighbour.  The span stays far below 2 GiB, so the padding offset reads out of range.
  long long first_slot, last_slot;
  {
    const long long p0 = (long long)tile * BN;
    long long p1 = p0 + BN - 1;
    if (p1 >= m_band) p1 = m_band - 1;
    const int n0 = (int)(p0 / plane), r0 = (int)((p0 - (long long)n0 * plane) / wc);
    const int n1 = (int)(p1 / plane), r1 = (int)((p1 - (long long)n1 * plane) / wc);
    const int top = UPS ? ((r0 - 1) >> 1) : (DS ? 2 * r0 : r0 - 1);     // lowest source row (-1 = halo)
    const int bot = UPS ? ((r1 + 1) >> 1) : (DS ? 2 * r1 + 2 : r1 + 1);  // highest source row
    first_slot = (long long)(n0 - (KT - 1)) * (rows_in + 2) + top + 1;
    if (first_slot < 0) first_slot = 0;
    last_slot = (long long)n1 * (rows_in + 2) + bot + 1;
  }
  const long long row_elems = (long long)a.in.W * a.in.C;
  const long long x_base = a.in.off[band] + first_slot * row_elems;   // element offset
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(reinterpret_cast<const char*>(a.x) + x_base * XB,
                (unsigned)((last_slot - first_slot + 1) * row_elems * XB));
  const int wco = (wave >> 1) * 64;
  const int wpx = (wave & 1) * 64;
  // Accumulators acc<i><j>: channel co0+wco+32i+8(v/4)+4(lane/32)+(v%4), pixel
  // tile*BN+wpx+32j+(lane%32).  They start at bias + residual (band modes: fp32 with `cout`
  // channels in the output's band geometry, split outputs at half their offset), so the
  // epilogue only stores; the residual's latency overlaps the first operand loads.  (An
  // opaque copy of the lane index keeps the compiler from carrying these addresses through
  // the K loop for the epilogue.)
  f32x16_t acc00, acc01, acc10, acc11;
  {
    int ilane = lane;
    asm volatile("" : "+v"(ilane));
    auto init = [&](f32x16_t& acc, int i, int j) {
      const long long p = (long long)tile * BN + wpx + 32 * j + (ilane & 31);
      long long ro = -1;
      if ((MODE == kModeBand || MODE == kModeBandSplit) && a.res && p < m_band) {
        const int n = (int)(p / plane);
        const int rem = (int)(p - (long long)n * plane);
        const int r = rem / wc;
        const int c = rem - r * wc;
        ro = band_offset(a.out, band, n, r, c);
        if (MODE == kModeBandSplit) ro >>= 1;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int co = co0 + wco + 32 * i + 8 * g + 4 * (ilane >> 5);
        float4 v = *reinterpret_cast<const float4*>(a.bias + co);   // cout_pad entries
        if (ro >= 0 && co < a.cout) {
          const float4 rr = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.res) + ro + co);
          v.x += rr.x;
          v.y += rr.y;
          v.z += rr.z;
          v.w += rr.w;
        }
        acc[4 * g + 0] = v.x;
        acc[4 * g + 1] = v.y;
        acc[4 * g + 2] = v.z;
        acc[4 * g + 3] = v.w;
      }
    };
    init(acc00, 0, 0);
    init(acc01, 0, 1);
    init(acc10, 1, 0);
    init(acc11, 1, 1);
  }
  const int frag = (lane & 31) * LDK + (lane >> 5) * 8;
  const int srow = rs * LDK + q8;

  // XN stages hold the raw fp32 chunk (8 channels); the apply runs when it goes to LDS,
  // with the stage's first channel and padding chunks (bit j) recorded at its load
  struct F8 {
    f32x4_t lo, hi;
  };
  using XR = typename std::conditional<XN, F8, u32x4_t>::type;
  u32x4_t wa[NP], wb[NP];
  XR xa[NP], xb[NP];
  unsigned pma = 0, pmb = 0;
  int csa = 0, csb = 0;
  if constexpr (XN) {
    const int n_t = (int)(((long long)tile * BN) / plane);   // every band's plane is a multiple of BN
    const float* src = a.x_norm + (long long)n_t * cin * 2;
    for (int i = tid; i < 2 * cin; i += 256) sN[i] = src[i];
    __syncthreads();
  }
  unsigned xo[NP];   // byte offset of this thread's chunk at the current tap, or kPadOffset
  VAEP_FOR_J({ xo[j] = kPadOffset; });
  int tap = 0, c0 = 0, loaded = 0;
  bool lo = false;

// Loads: per step, weights at wvo[j] + (tap*cin + c0)*2 and inputs at xo[j] + c0*XB, both
// with the step part as a scalar offset.  Padding taps read past the end of the band
// buffer and get zeros; loads past the last step repeat the last step.
#define VAEP_CONV_LOAD(W, X, PM, CS)                                                            \
  {                                                                                             \
    if (c0 == 0) {                                                                              \
      const int dt = tap / (KS * KS), dy = (tap / KS) % KS, dx = tap % KS;                      \
      VAEP_FOR_J({                                                                              \
        bool ok;                                                                                \
        const long long o = tap_source(a.in, band, pn[j], pr[j], pc[j], dt, dy, dx, KT, KS, UPS, &ok, DS); \
        xo[j] = (ok && pv[j]) ? (unsigned)((o - x_base + q8) * XB) : kPadOffset;                \
      });                                                                                       \
    }                                                                                           \
    const int ws = (tap * cin + c0) * 2;                                                        \
    const int xs = c0 * XB;                                                                     \
    if constexpr (XN) {                                                                         \
      PM = 0u;                                                                                  \
      CS = c0;                                                                                  \
    }                                                                                           \
    VAEP_FOR_J({                                                                                \
      W[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wvo[j], ws, 0)); \
      if constexpr (XN) {                                                                       \
        X[j].lo = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)xo[j], xs, 0)); \
        X[j].hi = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)xo[j] + 16, xs, 0)); \
        if (xo[j] == kPadOffset) PM |= 1u << j;                                                 \
      } else {                                                                                  \
        X[j] = load8<XF32>(xrs, xo[j], xs, lo);                                                 \
      }                                                                                         \
    });                                                                                         \
    if (++loaded < nsteps) {                                                                    \
      c0 += BK;                                                                                 \
      if (c0 == cin) {                                                                          \
        c0 = 0;                                                                                 \
        if (++tap == TAPS) {                                                                    \
          tap = 0;                                                                              \
          lo = true;                                                                            \
        }                                                                                       \
      }                                                                                         \
    }                                                                                           \
  }
#define VAEP_CONV_STASH(W, X, buf, PM, CS)                                                      \
  {                                                                                             \
    if constexpr (XN) {                                                                         \
      const f32x4_t* nt = reinterpret_cast<const f32x4_t*>(&sN[2 * ((CS) + q8)]);               \
      const f32x4_t n0 = nt[0], n1 = nt[1], n2 = nt[2], n3 = nt[3];                             \
      const bool act = a.x_norm_act != 0;                                                       \
      VAEP_FOR_J({                                                                              \
        *reinterpret_cast<u32x4_t*>(&sW[buf][srow + RP * j * LDK]) = W[j];                      \
        u32x4_t u = u32x4_t{0u, 0u, 0u, 0u};                                                    \
        if (!(((PM) >> j) & 1u)) {                                                              \
          const F8 v = X[j];                                                                    \
          u.x = (unsigned)f2bf(gn_affine_act(v.lo.x, n0.x, n0.y, act)) |                        \
                ((unsigned)f2bf(gn_affine_act(v.lo.y, n0.z, n0.w, act)) << 16);                 \
          u.y = (unsigned)f2bf(gn_affine_act(v.lo.z, n1.x, n1.y, act)) |                        \
                ((unsigned)f2bf(gn_affine_act(v.lo.w, n1.z, n1.w, act)) << 16);                 \
          u.z = (unsigned)f2bf(gn_affine_act(v.hi.x, n2.x, n2.y, act)) |                        \
                ((unsigned)f2bf(gn_affine_act(v.hi.y, n2.z, n2.w, act)) << 16);                 \
          u.w = (unsigned)f2bf(gn_affine_act(v.hi.z, n3.x, n3.y, act)) |                        \
                ((unsigned)f2bf(gn_affine_act(v.hi.w, n3.z, n3.w, act)) << 16);                 \
        }                                                                                       \
        *reinterpret_cast<u32x4_t*>(&sX[buf][srow + RP * j * LDK]) = u;                         \
      });                                                                                       \
    } else {                                                                                    \
      VAEP_FOR_J({                                                                              \
        *reinterpret_cast<u32x4_t*>(&sW[buf][srow + RP * j * LDK]) = W[j];                      \
        *reinterpret_cast<u32x4_t*>(&sX[buf][srow + RP * j * LDK]) = X[j];                      \
      });                                                                                       \
    }                                                                                           \
  }
#define VAEP_MFMA_K(buf, kk)                                                                    \
  {                                                                                             \
    const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(&sW[buf][wco * LDK + frag + kk * 16]); \
    const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(&sW[buf][(wco + 32) * LDK + frag + kk * 16]); \
    const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&sX[buf][wpx * LDK + frag + kk * 16]); \
    const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&sX[buf][(wpx + 32) * LDK + frag + kk * 16]); \
    acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc00, 0, 0, 0);                    \
    acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc01, 0, 0, 0);                    \
    acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc10, 0, 0, 0);                    \
    acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc11, 0, 0, 0);                    \
  }
#define VAEP_CONV_COMPUTE(buf)                                                                  \
  {                                                                                             \
    VAEP_MFMA_K(buf, 0);                                                                        \
    VAEP_MFMA_K(buf, 1);                                                                        \
    if constexpr (BK == 64) {                                                                   \
      VAEP_MFMA_K(buf, 2);                                                                      \
      VAEP_MFMA_K(buf, 3);                                                                      \
    }                                                                                           \
  }

  // Two register stages (a, b) and two LDS buffers: the loads of step s+2 are issued
  // before the MFMAs of step s and land in LDS at the end of step s+1.
  // (stashes past the last step write a buffer no step reads)
  VAEP_CONV_LOAD(wa, xa, pma, csa);
  VAEP_CONV_LOAD(wb, xb, pmb, csb);
  VAEP_CONV_STASH(wa, xa, 0, pma, csa);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    VAEP_CONV_LOAD(wa, xa, pma, csa);
    VAEP_CONV_COMPUTE(0);
    VAEP_CONV_STASH(wb, xb, 1, pmb, csb);
    __syncthreads();
    if (s + 1 == nsteps) break;
    VAEP_CONV_LOAD(wb, xb, pmb, csb);
    VAEP_CONV_COMPUTE(1);
    VAEP_CONV_STASH(wa, xa, 0, pma, csa);
    __syncthreads();
  }
#undef VAEP_CONV_LOAD
#undef VAEP_CONV_STASH
#undef VAEP_CONV_COMPUTE
#undef VAEP_MFMA_K
  f32x16_t acc[2][2] = {{acc00, acc01}, {acc10, acc11}};

  // Epilogue: the accumulators hold the final values.  When a GroupNorm consumes the
  // output (a.gn_part set by the launch, whole-row tiles), the tile's moments are formed
  // before the values are stored.
  if constexpr (MODE == kModeBand) {
    if (a.gn_part) {
      const long long p0 = (long long)tile * BN;
      const int n0 = (int)(p0 / plane);
      const int rem0 = (int)(p0 - (long long)n0 * plane);
      const int cg = a.cout / a.gn_groups;
      const long long rec = gnstats::tile_record(a.out, band, n0, rem0 / wc, (rem0 % wc) / BN, wc / BN);
      const long long tiles = (long long)a.out.H * (wc / BN);
      gnstats::tile_stats<2, 2, 4, 2, BM, false>(acc, wave, lane, cg, BN,
                                                 gnstats::record(a.gn_part, rec, co0 / cg, a.gn_groups, tiles),
                                                 2 * tiles, reinterpret_cast<float*>(&sW[0][0]));
    }
  }
  // Band outputs leave in whole lines through the weight stages (free once every wave has
  // passed the LDS barrier after its last products or the statistics), 32 x 68 floats per
  // wave; with 32-channel steps the stages are too small and the stores below run instead.
  if constexpr ((MODE == kModeBand || MODE == kModeBandSplit) && sizeof(sW) >= 4 * 32 * 68 * sizeof(float)) {
    gnstats::lds_barrier();
    float* wl = reinterpret_cast<float*>(&sW[0][0]) + wave * (32 * 68);
    if (MODE == kModeBandSplit && a.split8)
      epi::split8_epilogue_lines<false, 2, 2, BN>(a, acc, band, tile, plane, m_band, wc, 0, 0, co0, wco, wpx, lane, wl);
    else if (MODE == kModeBandSplit)
      epi::split_epilogue_lines<false, 2, 2, BN>(a, acc, band, tile, plane, m_band, wc, 0, 0, co0, wco, wpx, lane, wl);
    else
      epi::band_epilogue_lines<false, 2, 2, BN>(a, acc, band, tile, plane, m_band, wc, 0, 0, co0, wco, wpx, lane, wl);
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long long p = (long long)tile * BN + wpx + 32 * j + (lane & 31);
    if (p >= m_band) continue;
    const int n = (int)(p / plane);
    const int rem = (int)(p - (long long)n * plane);
    const int r = rem / wc;
    const int c = rem - r * wc;
    // band modes: this pixel's own slot and its halo slots in the neighbours (boundary
    // rows; a one-row band has both), formed once per pixel block -- formed per store, the
    // band fields are re-read from the kernel arguments with a scalar-load wait each time
    long long own = 0, hu = -1, hd = -1;
    if (MODE == kModeBand || MODE == kModeBandSplit) {
      const BandLayout& L = a.out;
      const long long OC = L.C;
      const int rows_b = L.rows[band];
      own = L.off[band] + (((long long)n * (rows_b + 2) + r + 1) * L.W + c) * OC;
      if (band > 0 && r == 0)
        hu = L.off[band - 1] + (((long long)n * (L.rows[band - 1] + 2) + L.rows[band - 1] + 1) * L.W + c) * OC;
      if (band + 1 < L.nb && r == rows_b - 1)
        hd = L.off[band + 1] + ((long long)n * (L.rows[band + 1] + 2) * L.W + c) * OC;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int co = co0 + wco + 32 * i + 8 * g + 4 * (lane >> 5);
        if (co >= a.cout) continue;
        const float v[4] = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (MODE == kModeBandSplit) {
          auto put = [&](long long q) {
            if (a.split8)
              st4split8(a.y, q, a.cout, co, v);
            else
              st4split(a.y, q + co, a.cout, v);
          };
          put(own);
          if (hu >= 0) put(hu);
          if (hd >= 0) put(hd);
        } else if (MODE == kModeBand) {
          st4f(a.y, own + co, v);
          if (hu >= 0) st4f(a.y, hu + co, v);
          if (hd >= 0) st4f(a.y, hd + co, v);
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
          const long long pix = a.out_transposed ? (long long)c * a.in.H + (a.in.row0[band] + r)
                                                : (long long)(a.in.row0[band] + r) * a.in.W + c;
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
  const bool ups = a.ups != 0, down = a.down != 0;
  const int rows_c = ups ? 2 * rows_in : (down ? rows_in / 2 : rows_in);
  const int wc = ups ? 2 * a.in.W : (down ? a.in.W / 2 : a.in.W);
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
    const long long off = tap_source(a.in, band, n, r, c, dt, dy, dx, a.kt, a.ks, ups, &ok, down);
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
    const long long pix = a.out_transposed ? (long long)c * a.in.H + (a.in.row0[band] + r)
                                                : (long long)(a.in.row0[band] + r) * a.in.W + c;
    reinterpret_cast<float*>(a.y)[(((long long)bsm * a.cout + co) * T + t) * hw + pix] = v;
  }
}

template <int KT, int KS, bool UPS, int MODE, bool DS = false>
hipError_t go(const ConvArgs& a, hipStream_t s) {
  const int ny = a.cout_pad / kConvTileN;
  dim3 grid(a.tiles_total, ny);
  const bool k64 = a.cin % 64 == 0;
  if (a.x_norm) {
    if constexpr (KT == 1 && KS == 3 && !UPS && MODE == kModeBand) {
      hipLaunchKernelGGL((conv_mfma_bf16<KT, KS, UPS, MODE, false, 64, true>), grid, dim3(256), 0, s, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (a.x_f32 && k64)
    hipLaunchKernelGGL((conv_mfma_bf16<KT, KS, UPS, MODE, true, 64, false, DS>), grid, dim3(256), 0, s, a);
  else if (a.x_f32)
    hipLaunchKernelGGL((conv_mfma_bf16<KT, KS, UPS, MODE, true, 32, false, DS>), grid, dim3(256), 0, s, a);
  else if (k64)
    hipLaunchKernelGGL((conv_mfma_bf16<KT, KS, UPS, MODE, false, 64, false, DS>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((conv_mfma_bf16<KT, KS, UPS, MODE, false, 32, false, DS>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool conv_norm_fold_ok(const ConvArgs& a) {
  if (a.kt != 1 || a.ks != 3 || a.ups || a.down || a.mode != kModeBand || a.x_f32 || a.x_split || a.sub || a.x2 ||
      a.cin2)
    return false;
  if (a.cin % 64 != 0 || a.cin > 512 || a.in.C != a.cin) return false;
  ConvArgs u = a;   // the same conv unfolded runs on the tile128 kernel too
  u.x_norm = nullptr;
  if (conv_halo_fits(u) || conv_wide_fits(u) || conv_narrow_fits(u)) return false;
  for (int b = 0; b < a.in.nb; ++b)   // pixel tiles never straddle two images
    if (((long long)a.in.rows[b] * a.in.W) % kConvTileM != 0) return false;
  return true;
}

hipError_t launch_conv(ConvArgs& a, int dtype, hipStream_t s) {
  const bool ups = a.ups != 0, down = a.down != 0;
  a.gn_chunk = 0;
  if (down) {
    // stride 2: plain 3x3 2-D band convs, even band rows and width, on the tile kernels
    if (ups || a.kt != 1 || a.ks != 3 || a.mode != kModeBand || a.x_split || a.sub || a.x2 || a.cin2 || a.x_norm ||
        a.in.W % 2 != 0 || a.out.W != a.in.W / 2 || a.out.nb != a.in.nb)
      return hipErrorInvalidValue;
    for (int b = 0; b < a.in.nb; ++b)
      if (a.in.rows[b] % 2 != 0 || a.out.rows[b] != a.in.rows[b] / 2) return hipErrorInvalidValue;
    a.gn_part = nullptr;   // the next norm forms its own statistics
  }
  if (a.x_norm && (dtype != VAEP_DTYPE_BF16 || !conv_norm_fold_ok(a))) return hipErrorInvalidValue;
  if (!a.x_norm && dtype != VAEP_DTYPE_F32 && conv_halo_fits(a)) return launch_conv_halo(a, s);
  if (!a.x_norm && dtype != VAEP_DTYPE_F32 && conv_wide_fits(a)) return launch_conv_wide(a, s);
  if (!a.x_norm && dtype != VAEP_DTYPE_F32 && conv_narrow_fits(a)) {
    a.gn_part = nullptr;
    return launch_conv_narrow(a, s);
  }
  // split operands and sub-pixel weights exist only on the wide kernel; the fp8 split
  // output needs 64-channel blocks
  if (a.x_split || a.sub || (a.mode == kModeBandSplit && dtype == VAEP_DTYPE_F32)) return hipErrorInvalidValue;
  if (a.split8 && (a.mode != kModeBandSplit || a.cout % 64 != 0)) return hipErrorInvalidValue;
  if (a.x2 || a.cin2) return hipErrorInvalidValue;   // a folded second operand needs the wide kernel
  if (dtype != VAEP_DTYPE_F32) {
    // buffer-resource addressing: the rows one tile can read and the weights stay below
    // 2 GiB, so the padding offset reads out of range
    const long long xb = (a.x_f32 || a.x_norm) ? 4 : 2;
    for (int b = 0; b < a.in.nb; ++b)
      if ((tile_read_slots(a.in, b, a.kt, kConvTileM, ups, down) * a.in.W + 2LL * kConvTileM) * a.in.C * xb >=
          (1LL << 31) - 4096)
        return hipErrorInvalidValue;
    if ((long long)a.cout_pad * a.kt * a.ks * a.ks * a.cin * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  }
  int t = 0;
  for (int b = 0; b < a.in.nb; ++b) {
    a.tile_start[b] = t;
    const long long m = down ? (long long)a.in.n_img * (a.in.rows[b] / 2) * (a.in.W / 2)
                             : (long long)a.in.n_img * (ups ? 2 : 1) * a.in.rows[b] * (ups ? 2 : 1) * a.in.W;
    t += (int)((m + kConvTileM - 1) / kConvTileM);
  }
  a.tile_start[a.in.nb] = t;
  a.tiles_total = t;
  a.kernel_used = dtype == VAEP_DTYPE_F32 ? VAEP_KERNEL_CONV_F32 : VAEP_KERNEL_CONV_TILE128;
  // GroupNorm tile statistics in the epilogue: whole-row pixel tiles, every group inside
  // one channel tile
  const int wout = (ups ? 2 : 1) * a.in.W;
  a.gn_chunk = 0;
  if (a.gn_part && dtype != VAEP_DTYPE_F32 && a.mode == kModeBand && !a.x_f32 && wout % kConvTileM == 0 &&
      a.cout == a.cout_pad && a.gn_groups > 0 && a.cout % a.gn_groups == 0 && (a.cout / a.gn_groups) % 4 == 0 &&
      kConvTileN % (a.cout / a.gn_groups) == 0)
    a.gn_chunk = kConvTileM;
  if (!a.gn_chunk) a.gn_part = nullptr;
  if (t == 0) return hipSuccess;
  if (dtype == VAEP_DTYPE_F32) {
    dim3 grid(t, a.cout);
    hipLaunchKernelGGL(conv_f32, grid, dim3(kConvTileM), 0, s, a);
    return hipGetLastError();
  }
  const int kt = a.kt, ks = a.ks, m = a.mode;
  if (down) return go<1, 3, false, kModeBand, true>(a, s);
  if (kt == 1 && ks == 3 && !ups && m == kModeBand) return go<1, 3, false, kModeBand>(a, s);
  if (kt == 1 && ks == 3 && !ups && m == kModeBandSplit) return go<1, 3, false, kModeBandSplit>(a, s);
  if (kt == 3 && ks == 3 && !ups && m == kModeBandSplit) return go<3, 3, false, kModeBandSplit>(a, s);
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
