// Wide-tile halo convolution on the gfx950 matrix cores, for the large layers.
//
// The operation is the one of conv.hip: a band's conv reads its own rows plus the
// kernel-radius halo rows its neighbours pushed into the band's halo slots, rows outside
// the image and columns outside the width read as zero, and a band writes only its own
// output rows (ChituDiffusion "VAEP" feature page, conv section; "Static Layer-Wise VAE
// Decode", operator table, "Spatial convolution" row).
//
// Layout of the work: one workgroup of NW waves computes BM output channels x BN pixels
// of one band (256 x 256 and 128 x 512 with 8 waves, 128 x 256 with 4) as an implicit
// GEMM D[co][pixel] = W[co][k] X[k][pixel] with v_mfma_f32_32x32x16_bf16; the waves own
// (BM/2) x (2 BN/NW) each.  K advances one tap and 64 channels per step, taps fastest.
// Both operand tiles go global -> LDS directly (buffer loads with the LDS destination),
// through S stages (3 for 128 x 256, else 2), with one barrier per step and no staging
// registers.  A lane's 16-byte chunk lands at a fixed
// LDS slot, so the XOR swizzle that keeps the matrix-core reads free of bank conflicts is
// applied on the global side: LDS slot (row, p) holds logical chunk p ^ f(row),
// f(row) = (row & 7) ^ ((row >> 3) & 1).
//
// Nearest-2x upsample + 3x3 conv runs in sub-pixel form.  Output pixel (2i+py, 2j+px)
// reads, through the upsample, only source pixels (i+a-1+py, j+b-1+px), a, b in {0, 1};
// summing the 3x3 weights that fall on the same source pixel gives four 2x2 convs on the
// source grid (one per phase), 2.25x fewer products.  A tap outside the upsampled image
// is exactly a tap outside the source image, so zero padding carries over unchanged.  The
// summed weights are no longer bf16 values and are applied as bf16 hi + lo parts.
//
// The operand of the sub-pixel form is the fp32 residual stream in the encoding of
// split8.h (kModeBandSplit output with split8 set, or launch_split): bf16 hi parts, then
// per 64-channel block fp8 bytes of x_lo and of x.  K runs over two parts per tap: x_hi *
// w_hi as bf16 products, then the correction terms x_lo * w + x * w_lo as one fp8 step of
// K = 128 per 64 channels (v_mfma_scale_f32_32x32x64_f8f6f4, A e4m3 weights, B e5m2
// operand, A's E8M0 scale removing the power of two both were stored with).  That fp8
// step reads LDS exactly like a bf16 step: its 32-byte operands are the fragments of two
// consecutive 16-wide bf16 slices, taken in the same order for A and B, so every weight
// byte meets the operand byte of its channel.  Other convs have one part: x * w.
#include "vaep_internal.h"
#include "conv_dma.h"
#include "conv_gn_stats.h"
#include "split8.h"
#include "conv_epilogue.h"

namespace vaep {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) unsigned short lds_u16;

namespace {

using dma::kPadOffset;
using dma::make_rsrc;
using dma::dma16;
using dma::lds_addr;
using dma::xcd_remap;

__device__ __forceinline__ long long band_offset(const BandLayout& L, int b, int n, int r, int c) {
  return L.off[b] + (((long long)n * (L.rows[b] + 2) + r + 1) * L.W + c) * (long long)L.C;
}

__device__ __forceinline__ int band_of_tile(const ConvArgs& a, int mt) {
  int b = 0;
  while (b + 1 < a.in.nb && mt >= a.tile_start[b + 1]) ++b;
  return b;
}


// Part p of a tap selects the weight and operand halves of its packed rows: 0 = the bf16
// values (w or w_hi; x or x_hi), 1 = the fp8 correction block of split8.h.
__device__ __forceinline__ constexpr int wpart(int, int p) { return p; }
__device__ __forceinline__ constexpr int xpart(int p) { return p; }

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
// Two 16-byte fragments as one 32-byte fp8 operand.
__device__ __forceinline__ i32x8_t cat32(bf16x8_t a, bf16x8_t b) {
  const i32x4_t x = __builtin_bit_cast(i32x4_t, a), y = __builtin_bit_cast(i32x4_t, b);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Load g (0 .. NL-1) of a step is an A (weight) chunk load for g < NA, else a B (pixel)
// chunk load; the loads go out in four quarters, quarter q issuing loads QB(q) .. QB(q+1)-1.
// When both counts divide by four each quarter interleaves NA/4 A and NB/4 B loads.
template <int NA, int NB>
struct LoadOrder {
  static constexpr int NL = NA + NB;
  static constexpr bool even = NA % 4 == 0 && NB % 4 == 0;
  static constexpr int QB(int q) { return q * NL / 4; }
  static constexpr int count(int q) { return QB(q + 1) - QB(q); }
  // flat index of the t-th load of quarter q
  static constexpr int at(int q, int t) {
    return !even ? QB(q) + t : (t < NA / 4 ? q * (NA / 4) + t : NA + q * (NB / 4) + t - NA / 4);
  }
  // the load starts a run that shares one scalar offset (A loads, or B loads, of a quarter)
  static constexpr bool first(int q, int t) {
    return even ? (t == 0 || t == NA / 4) : (at(q, t) == QB(q) || at(q, t) == (QB(q) > NA ? QB(q) : NA));
  }
};

// X2: the conv reads a second operand (a.x2, a folded 1x1 shortcut) after its taps.
// H32: C = 32 mod 64, each tap's last 64-channel step half empty (not the sub-pixel form).
template <int KT, int KS, bool SUB, int PARTS, int MODE, int BM, int BN, int NW, bool X2, bool H32 = false>
__global__ void __launch_bounds__(NW * 64, 1) conv_wide(const ConvArgs a) {
  static_assert(!X2 || (!SUB && MODE == kModeBand), "a second operand folds into plain band convs only");
  // NW waves: 2 along the output channels x NW/2 along the pixels.  With 8 waves two
  // share each SIMD, so one wave's loads, LDS reads and barrier waits hide behind the
  // other's MFMAs.
  constexpr int S = (BM == 128 && BN == 256) ? 3 : 2;   // LDS stages
  constexpr int TAPS = SUB ? 4 : KT * KS * KS;
  static_assert(SUB ? PARTS == 2 : PARTS == 1, "sub-pixel convs run a bf16 and an fp8 part");
  constexpr int WP = PARTS;                   // weight parts per tap in the packed rows
  constexpr int WPX = NW / 2;                 // waves along the pixels
  constexpr int NA = BM / (8 * NW);           // A (weight) chunk loads per thread per step
  constexpr int NB = BN / (8 * NW);           // B (pixel) chunk loads per thread per step
  constexpr int MI = BM / 64;                 // 32-row channel blocks per wave
  constexpr int NJ = BN / (32 * WPX);         // 32-pixel blocks per wave
  typedef LoadOrder<NA, NB> LO;
  static_assert(LO::NL >= 4 && LO::count(0) >= 1 && MI * NJ >= 3, "loads per quarter step");
  constexpr int PH = SUB ? 4 : 1;
  // S operand stages: A (BM x 64) then B (BN x 64) per stage; the epilogue reuses the space
  constexpr int kStageElems = S * (BM + BN) * 64;
  __shared__ __attribute__((aligned(1024))) unsigned short smem[kStageElems];
  static_assert(NW * 32 * 68 * 4 <= kStageElems * 2, "epilogue transpose rows");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned wrow = wave * 8 * 64 * 2;   // LDS byte offset of this wave's first row block
  constexpr unsigned kRowStep = NW * 8 * 64 * 2;   // LDS bytes between a wave's row blocks
  // work id -> (output-channel tile, pixel tile, phase); the phases of a pixel tile are adjacent
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int phase = lin % PH;
  const int rest = lin / PH;
  const int mt = rest % a.tiles_total;
  const int co0 = (rest / a.tiles_total) * BM;
  const int band = band_of_tile(a, mt);
  const int tile = mt - a.tile_start[band];
  const int py = phase >> 1, px = phase & 1;

  const int rows_in = a.in.rows[band];
  const int W = a.in.W;
  const int plane = rows_in * W;                       // compute pixels per image (source grid)
  const long long m_band = (long long)a.in.n_img * plane;
  const int C = a.cin;                                 // input channels
  const int XC = a.in.C;                               // channel stride of the input buffer
  // 64-channel steps per tap; with C = 32 mod 64 (H32) the last step of a tap is half empty:
  // its pixel chunks past C read zeros (the padding offset), so whatever weights meet them add 0
  static_assert(!H32 || !SUB, "half-empty channel steps: not the sub-pixel form");
  const int csteps = H32 ? (C + 63) >> 6 : C >> 6;
  // K: the taps of the operand, then (a.x2) the channels of a second operand read at the
  // pixel itself -- a 1x1 conv folded into this one (a resnet's shortcut): its weights
  // follow the taps' in every packed row
  const int nsteps1 = TAPS * PARTS * csteps;
  const int cin2 = X2 ? a.cin2 : 0;
  const int nsteps = nsteps1 + (cin2 >> 6);
  const int kw = TAPS * WP * C + cin2;                 // packed weight row length (elements)

  // Input rows the tile can read: from its first pixel's row - 1 (KT - 1 frames back) to
  // its last pixel's row + 1; halo slots cover the rows beyond the band.
  long long first_slot, last_slot;
  {
    const long long p0 = (long long)tile * BN;
    long long p1 = p0 + BN - 1;
    if (p1 >= m_band) p1 = m_band - 1;
    const int n0 = (int)(p0 / plane), r0 = (int)((p0 - (long long)n0 * plane) / W);
    const int n1 = (int)(p1 / plane), r1 = (int)((p1 - (long long)n1 * plane) / W);
    first_slot = (long long)(n0 - (KT - 1)) * (rows_in + 2) + r0;
    if (first_slot < 0) first_slot = 0;
    last_slot = (long long)n1 * (rows_in + 2) + r1 + 2;
  }
  const long long row_elems = (long long)W * XC;
  const u32x4_t xrs = make_rsrc(
      reinterpret_cast<const unsigned short*>(a.x) + a.in.off[band] + first_slot * row_elems,
      (unsigned)((last_slot - first_slot + 1) * row_elems * 2));
  const u32x4_t wrs = make_rsrc(
      reinterpret_cast<const unsigned short*>(a.w) + (long long)phase * a.cout_pad * kw,
      (unsigned)((long long)a.cout_pad * kw * 2));

  // This thread's chunk: LDS rows (j*NW + wave)*8 + lane/8, slot lane%8, logical chunk ck.
  const int ck = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  unsigned avo[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j)
    avo[j] = (unsigned)(((long long)(co0 + (j * NW + wave) * 8 + (lane >> 3)) * kw + ck * 8) * 2);
  // Pixel rows: byte offset of the pixel's own position and validity bits
  // (0..2: row shift -1..1 inside the image, 3..5: column shift -1..1, 6..8: frame shift
  // -(KT-1)+dt not before frame 0).
  unsigned pbase[NB];
  int pmask[NB];
  // second operand (a.x2): cin2 channels per pixel in the input's band geometry (band
  // offsets scale with the channel count), over the same rows as the first
  unsigned pbase2[NB];
  const u32x4_t x2rs = make_rsrc(
      a.x2 ? reinterpret_cast<const unsigned short*>(a.x2) + a.in.off[band] / XC * a.cin2 + first_slot * W * a.cin2
           : nullptr,
      a.x2 ? (unsigned)((last_slot - first_slot + 1) * W * a.cin2 * 2) : 0u);
  const int H = a.in.H;
  const int g0 = a.in.row0[band];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const long long p = (long long)tile * BN + (j * NW + wave) * 8 + (lane >> 3);
    const bool ok = p < m_band;
    const long long q = ok ? p : 0;
    const int n = (int)(q / plane);
    const int rem = (int)(q - (long long)n * plane);
    const int r = rem / W;
    const int c = rem - r * W;
    const long long slot = (long long)n * (rows_in + 2) + r + 1;
    pbase[j] = (unsigned)(((slot - first_slot) * W + c) * XC * 2 + ck * 16);
    pbase2[j] = (unsigned)(((slot - first_slot) * W + c) * a.cin2 * 2 + ck * 16);
    const int g = g0 + r;
    int m = 0;
    m |= (g - 1 >= 0) ? 1 : 0;
    m |= 2;
    m |= (g + 1 < H) ? 4 : 0;
    m |= (c - 1 >= 0) ? 8 : 0;
    m |= 16;
    m |= (c + 1 < W) ? 32 : 0;
    const int t = n % a.in.frames;
#pragma unroll
    for (int dt = 0; dt < KT; ++dt) m |= (t + dt - (KT - 1) >= 0) ? (64 << dt) : 0;
    pmask[j] = ok ? m : 0;
  }
  unsigned bvo[NB];
  // acc[i][j][v]: channel co0 + wco + 32i + 8(v/4) + 4(lane/32) + v%4, pixel
  // tile*BN + wpx + 32j + lane%32 (source grid for sub-pixel convs).
  // fp8 step scales (E8M0 in every byte): A's removes the weights' and the operand's
  // power-of-two factors; B's is 1
  const int f8_scale_a = SUB ? *a.sub_scale : 0;
  constexpr int f8_scale_b = 127 * 0x01010101;
  const int wco = (wave / WPX) * (BM / 2);
  const int wpx = (wave % WPX) * (BN / WPX);
  // The accumulators start at bias + residual (fp32 with `cout` channels in the output's
  // band geometry; split outputs address it at half their offset), so the epilogue only
  // stores: the residual's HBM latency overlaps the first operand loads instead of
  // stalling the stores.
  // (an opaque copy of the lane index keeps the compiler from carrying these addresses
  // through the K loop for the epilogue, which forms them again)
  f32x16_t acc[MI][NJ];
  int ilane = lane;
  asm volatile("" : "+v"(ilane));
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const long long p = (long long)tile * BN + wpx + 32 * j + (ilane & 31);
    long long ro = -1;
    if (a.res && p < m_band) {
      const int n = (int)(p / plane);
      const int rem = (int)(p - (long long)n * plane);
      int r = rem / W;
      int c = rem - r * W;
      if (SUB) {
        r = 2 * r + py;
        c = 2 * c + px;
      }
      ro = band_offset(a.out, band, n, r, c);
      if (MODE == kModeBandSplit) ro >>= 1;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
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
        acc[i][j][4 * g + 0] = v.x;
        acc[i][j][4 * g + 1] = v.y;
        acc[i][j][4 * g + 2] = v.z;
        acc[i][j][4 * g + 3] = v.w;
      }
  }

  // Issue the loads of step (c0, part, tap) into LDS stage st; taps vary fastest, so
  // consecutive steps read shifted windows of the same rows and channels (L2 and the
  // neighbouring tiles' reads then serve most of them).  bvo holds the tap's offsets.
  int itap = 0, ipart = 0, ic = 0, issued = 0;
  // validity bits a tap needs (see pmask) and its byte displacement in the input buffer
#define VAEP_TAP_GEO(tp, need, delta)                                                          \
  int need, delta;                                                                             \
  {                                                                                            \
    int dt, sy, sx;                                                                            \
    if (SUB) {                                                                                 \
      dt = KT - 1;                                                                             \
      sy = ((tp) >> 1) - 1 + py;                                                               \
      sx = ((tp) & 1) - 1 + px;                                                                \
    } else {                                                                                   \
      dt = (tp) / (KS * KS);                                                                   \
      sy = ((tp) / KS) % KS - KS / 2;                                                          \
      sx = (tp) % KS - KS / 2;                                                                 \
    }                                                                                          \
    need = (1 << (sy + 1)) | (8 << (sx + 1)) | (64 << dt);                                     \
    delta = (int)((((long long)(dt - (KT - 1)) * (rows_in + 2) + sy) * W + sx) * XC * 2);      \
  }
#define VAEP_ADVANCE(tp, pt, cc)                                                               \
  if (++tp == TAPS) {                                                                          \
    tp = 0;                                                                                    \
    if (++pt == PARTS) {                                                                       \
      pt = 0;                                                                                  \
      cc += 64;                                                                                \
    }                                                                                          \
  }
#define VAEP_SA(st) (smem + (st) * (BM * 64))
#define VAEP_SB(st) (smem + S * (BM * 64) + (st) * (BN * 64))
// The loads of one step go out in four parts, one before each group of MFMAs of the
// current step, so that the wave never waits on a full load queue with the matrix cores
// idle.  One load of a step: quarter q (0..3), index t within the quarter (LoadOrder).
// Quarter 0's first load also forms the tap's offsets; quarter 3's last load advances the
// step counters.
#define VAEP_ISSUE_ONE(st, q, t)                                                               \
  {                                                                                            \
    const bool ext_ = X2 && issued >= nsteps1;     /* a step of the second operand */         \
    if ((q) == 0 && (t) == 0) {                                                                \
      if (ext_) {                                                                              \
        _Pragma("unroll") for (int j = 0; j < NB; ++j) bvo[j] = pmask[j] ? pbase2[j] : kPadOffset; \
      } else {                                                                                 \
        VAEP_TAP_GEO(itap, need, delta);                                                       \
        _Pragma("unroll") for (int j = 0; j < NB; ++j)                                         \
          bvo[j] = ((pmask[j] & need) == need) ? (unsigned)((int)pbase[j] + delta) : kPadOffset; \
        /* a half-empty last channel step: this lane's 8 channels past C read zeros */         \
        if (H32 && ic + 64 > C && ic + ck * 8 >= C) {                                          \
          _Pragma("unroll") for (int j = 0; j < NB; ++j) bvo[j] = kPadOffset;                  \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
    const int lg_ = LO::at((q), (t));                                                          \
    if (lg_ < NA) {                                                                            \
      const int j = lg_;                                                                       \
      const int aso = ext_ ? (TAPS * WP * C + (issued - nsteps1) * 64) * 2                     \
                           : ((itap * WP + wpart(PARTS, ipart)) * C + ic) * 2;                 \
      dma16(LO::first((q), (t)), wrs, lds_addr(VAEP_SA(st)) + wrow + j * kRowStep, avo[j], aso); \
    } else {                                                                                   \
      const int j = lg_ - NA;                                                                  \
      const int bso = ext_ ? (issued - nsteps1) * 128 : (xpart(ipart) * C + ic) * 2;           \
      dma16(LO::first((q), (t)), ext_ ? x2rs : xrs, lds_addr(VAEP_SB(st)) + wrow + j * kRowStep, bvo[j], bso); \
    }                                                                                          \
    if ((q) == 3 && (t) == LO::count(3) - 1) {                                                 \
      ++issued;                                                                                \
      VAEP_ADVANCE(itap, ipart, ic);                                                           \
    }                                                                                          \
  }
#define VAEP_ISSUE_PART(st, q)                                                                 \
  {                                                                                            \
    _Pragma("unroll") for (int t = 0; t < LO::count(q); ++t) VAEP_ISSUE_ONE(st, q, t);         \
  }
#define VAEP_ISSUE(st)                                                                         \
  {                                                                                            \
    VAEP_ISSUE_PART(st, 0);                                                                    \
    VAEP_ISSUE_PART(st, 1);                                                                    \
    VAEP_ISSUE_PART(st, 2);                                                                    \
    VAEP_ISSUE_PART(st, 3);                                                                    \
  }

  // matrix-core operand reads: row (block base + lane%32), logical chunk 2*kk + lane/32
  const int fl = (lane & 7) ^ ((lane >> 3) & 1);
  const int lr = (lane & 31) * 64;
  int ko[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ko[kk] = lr + (((2 * kk + (lane >> 5)) ^ fl) << 3);

  // Step s computes from stage s % S and first issues step s + S - 1 into stage
  // (s + S - 1) % S, which every wave finished reading before the barrier.  Loads complete
  // in issue order; this thread's loads of step s have landed once at most the loads
  // issued after them (the next step's group when S is 3) are outstanding.  The barrier
  // then publishes every thread's chunks.  (An L2 prefetch of later steps' lines was
  // measured here: it slowed the 256 x 256 convs by 10 %.)  The last S - 1 steps issue
  // loads for steps past the end too, into stages no step reads, so the issue slots need
  // no branch: their offsets run past the operand rows, and a buffer load past a
  // resource's end returns zeros; the wait after the loop drains them.
#define VAEP_STEP_K(cs, ns, si, F8)                                                              \
  {                                                                                            \
    if (S == 3 && (si) + 2 <= nsteps)                                                          \
      __builtin_amdgcn_s_waitcnt((LO::NL & 15) | ((LO::NL >> 4) << 14) | (7 << 4) | (15 << 8)); \
    else                                                                                       \
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));                                        \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                            \
    const unsigned short* A = VAEP_SA(cs);                                                     \
    const unsigned short* B = VAEP_SB(cs);                                                     \
    if (F8) {                                                                                  \
      /* fp8 correction step: slices 2g and 2g+1 form the 32-byte operands of group g */      \
      _Pragma("unroll") for (int grp = 0; grp < 2; ++grp) {                                    \
        /* one A operand at a time keeps the operand registers at (1 + NJ) x 8; the two */    \
        /* 16-byte reads land in the halves of the 32-byte operand */                          \
        const int k0 = ko[2 * grp], k1 = ko[2 * grp + 1];                                      \
        i32x8_t fb[NJ];                                                                        \
        _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                       \
          fb[j].lo = *reinterpret_cast<const i32x4_t*>(B + (wpx + 32 * j) * 64 + k0);          \
          fb[j].hi = *reinterpret_cast<const i32x4_t*>(B + (wpx + 32 * j) * 64 + k1);          \
        }                                                                                      \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                       \
          i32x8_t fa;                                                                          \
          fa.lo = *reinterpret_cast<const i32x4_t*>(A + (wco + 32 * i) * 64 + k0);             \
          fa.hi = *reinterpret_cast<const i32x4_t*>(A + (wco + 32 * i) * 64 + k1);             \
          _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                     \
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                       \
                fa, fb[j], acc[i][j], 0, 1, 0, f8_scale_a, 0, f8_scale_b);                     \
          }                                                                                    \
        }                                                                                      \
        /* the group's MFMAs (64 cycles each) run while quarters 2g, 2g+1 issue */            \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        VAEP_ISSUE_PART(ns, 2 * grp);                                                          \
        VAEP_ISSUE_PART(ns, 2 * grp + 1);                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                     \
      }                                                                                        \
    } else {                                                                                   \
      /* operand fragments double-buffered across the four 16-wide K slices: the reads of */  \
      /* slice kk+1 are in flight while slice kk's MFMAs run */                               \
      bf16x8_t af[2][MI], bfr[2][NJ];                                                          \
      _Pragma("unroll") for (int i = 0; i < MI; ++i)                                           \
        af[0][i] = *reinterpret_cast<const bf16x8_t*>(A + (wco + 32 * i) * 64 + ko[0]);        \
      _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                           \
        bfr[0][j] = *reinterpret_cast<const bf16x8_t*>(B + (wpx + 32 * j) * 64 + ko[0]);       \
      _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                       \
        const int cur = kk & 1;                                                                \
        if (kk < 3) {                                                                          \
          _Pragma("unroll") for (int i = 0; i < MI; ++i)                                       \
            af[cur ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(A + (wco + 32 * i) * 64 + ko[kk + 1]); \
          _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                       \
            bfr[cur ^ 1][j] = *reinterpret_cast<const bf16x8_t*>(B + (wpx + 32 * j) * 64 + ko[kk + 1]); \
        }                                                                                      \
        /* the quarter step's loads go out one at a time between groups of MFMAs */           \
        _Pragma("unroll") for (int i = 0; i < MI; ++i)                                         \
          _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                     \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0); \
            const int per = (MI * NJ) / LO::count(kk);                                         \
            const int idx = i * NJ + j;                                                        \
            if (idx % per == per - 1 && idx / per < LO::count(kk)) {                           \
              __builtin_amdgcn_sched_barrier(0);                                               \
              VAEP_ISSUE_ONE(ns, kk, idx / per);                                               \
              __builtin_amdgcn_sched_barrier(0);                                               \
            }                                                                                  \
          }                                                                                    \
      }                                                                                        \
    }                                                                                          \
  }

  // step si of a sub-pixel conv is an fp8 step when its part is 1
#define VAEP_STEP(cs, ns, si) VAEP_STEP_K(cs, ns, si, SUB && ((si) / TAPS) % PARTS == 1)
  // prologue: steps 0 .. S-2 into stages 0 .. S-2
  VAEP_ISSUE(0);
  if (S == 3 && issued < nsteps) VAEP_ISSUE(1);
  // whole rounds of S steps, then the remainder (stage numbering restarts at 0).  A
  // two-stage sub-pixel conv runs rounds of 8 steps (4 taps of the bf16 part, then 4 of the
  // fp8 part) whose kinds are known at compile time: with both kinds behind a run-time
  // branch in every step the register allocation does not fit 2 waves per SIMD.
  const int nmain = nsteps - nsteps % S;
  int s = 0;
  if constexpr (SUB && S == 2) {
    for (; s < nsteps; s += 8) {
      VAEP_STEP_K(0, 1, s, false);
      VAEP_STEP_K(1, 0, s + 1, false);
      VAEP_STEP_K(0, 1, s + 2, false);
      VAEP_STEP_K(1, 0, s + 3, false);
      VAEP_STEP_K(0, 1, s + 4, true);
      VAEP_STEP_K(1, 0, s + 5, true);
      VAEP_STEP_K(0, 1, s + 6, true);
      VAEP_STEP_K(1, 0, s + 7, true);
    }
  } else {
    for (; s < nmain; s += S) {
      if (S == 2) {
        VAEP_STEP(0, 1, s);
        VAEP_STEP(1, 0, s + 1);
      } else {
        VAEP_STEP(0, 2, s);
        VAEP_STEP(1, 0, s + 1);
        VAEP_STEP(2, 1, s + 2);
      }
    }
    if (s < nsteps) VAEP_STEP(0, S - 1, s);
    if (S == 3 && s + 1 < nsteps) VAEP_STEP(1, 0, s + 1);
  }
#undef VAEP_STEP
#undef VAEP_STEP_K
#undef VAEP_SA
#undef VAEP_SB
#undef VAEP_TAP_GEO
#undef VAEP_ADVANCE
#undef VAEP_ISSUE_PART
#undef VAEP_ISSUE_ONE
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // every operand load has landed
#undef VAEP_ISSUE
#undef VAEP_SET_TAP

  // Epilogue: the accumulators hold the final values.
  const int half = a.cout;   // kModeBandSplit: lo parts start `cout` channels after the hi parts
  // When a GroupNorm consumes the output (a.gn_part set by the launch: whole-row tiles),
  // the tile's moments are formed from the values the norm reads (hi + lo for split
  // outputs); plain outputs are stored first and the statistics formed afterwards.
  const bool gn = a.gn_part != nullptr;
  auto gn_stats = [&](auto splitv) {
    gnstats::lds_barrier();   // every wave is done with the operand stages: the LDS is scratch now
    const long long p0 = (long long)tile * BN;
    const int n0 = (int)(p0 / plane);
    const int rem0 = (int)(p0 - (long long)n0 * plane);
    const int r0 = rem0 / W, c0 = rem0 - (rem0 / W) * W;
    const int chunks = (SUB ? 2 : 1) * (W / BN);
    const long long rec = gnstats::tile_record(a.out, band, n0, SUB ? 2 * r0 + py : r0,
                                               (SUB ? px * (W / BN) : 0) + c0 / BN, chunks);
    const int cg = a.cout / a.gn_groups;
    const long long tiles = (long long)a.out.H * chunks;
    gnstats::tile_stats<MI, NJ, NW, WPX, BM, decltype(splitv)::value>(
        acc, wave, lane, cg, BN, gnstats::record(a.gn_part, rec, co0 / cg, a.gn_groups, tiles), 2 * tiles,
        reinterpret_cast<float*>(smem));
  };
  if (MODE == kModeBandSplit && gn) gn_stats(std::true_type{});
  // The operand stages are free (the LDS barrier below, after the last products, or inside
  // the statistics); each wave transposes through its own 32 x 68 floats.
  gnstats::lds_barrier();
  float* wl = reinterpret_cast<float*>(smem) + wave * (32 * 68);
  if (MODE == kModeBandSplit) {
    if (a.split8)
      epi::split8_epilogue_lines<SUB, MI, NJ, BN>(a, acc, band, tile, plane, m_band, W, py, px, co0, wco, wpx, lane, wl);
    else
      epi::split_epilogue_lines<SUB, MI, NJ, BN>(a, acc, band, tile, plane, m_band, W, py, px, co0, wco, wpx, lane, wl);
    return;
  }
  epi::band_epilogue_lines<SUB, MI, NJ, BN>(a, acc, band, tile, plane, m_band, W, py, px, co0, wco, wpx, lane, wl);
  if (gn) gn_stats(std::false_type{});
}

template <int KT, int KS, bool SUB, int PARTS, int MODE, bool X2, bool H32 = false>
hipError_t go_tile(const ConvArgs& a, WideTile t, hipStream_t s) {
  const int ph = SUB ? 4 : 1;
  const long long wgs = (long long)a.tiles_total * (a.cout_pad / t.bm) * ph;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  if (t.bm == 256) {
    hipLaunchKernelGGL((conv_wide<KT, KS, SUB, PARTS, MODE, 256, 256, 8, X2, H32>), dim3((unsigned)wgs), dim3(512), 0, s, a);
  } else if constexpr (SUB) {
    // 128 x 256 tiles: sub-pixel convs only (plain convs of that size run on the 128 x 128
    // kernel); 8 waves, whose second wave per SIMD hides the fp8 step's extra issue slots
    if (t.bn != 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((conv_wide<KT, KS, SUB, PARTS, MODE, 128, 256, 8, X2, H32>), dim3((unsigned)wgs), dim3(512), 0, s, a);
  } else {
    if (t.bn != 512) return hipErrorInvalidValue;
    hipLaunchKernelGGL((conv_wide<KT, KS, SUB, PARTS, MODE, 128, 512, 8, X2, H32>), dim3((unsigned)wgs), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

template <int KT, int KS, bool SUB, int PARTS>
hipError_t go_mode(const ConvArgs& a, WideTile t, hipStream_t s) {
  if constexpr (!SUB) {
    if (a.cin % 64 == 32) {   // half-empty last channel step per tap
      if (a.mode == kModeBandSplit) return go_tile<KT, KS, SUB, PARTS, kModeBandSplit, false, true>(a, t, s);
      if constexpr (KS == 3)
        if (a.x2) return go_tile<KT, KS, SUB, PARTS, kModeBand, true, true>(a, t, s);
      if (a.x2) return hipErrorInvalidValue;
      return go_tile<KT, KS, SUB, PARTS, kModeBand, false, true>(a, t, s);
    }
  }
  if (a.mode == kModeBandSplit) return go_tile<KT, KS, SUB, PARTS, kModeBandSplit, false>(a, t, s);
  if constexpr (!SUB && KS == 3)
    if (a.x2) return go_tile<KT, KS, SUB, PARTS, kModeBand, true>(a, t, s);
  if (a.x2) return hipErrorInvalidValue;
  return go_tile<KT, KS, SUB, PARTS, kModeBand, false>(a, t, s);
}

}  // namespace

// Workgroup tile (output channels x pixels) of the wide kernel: 256 x 256 when a layer
// still fills the 256 CUs with two workgroups each (sub-pixel convs count their four
// phases); else, for plain convs, 128 x 512 with 8 waves when that does; else 128 x 256
// (the launch runs it for sub-pixel convs only; conv_wide_fits sends such plain convs to
// the 128 x 128 kernel).  Decided on the whole image, so every band table of an image runs
// the same kernel.
WideTile wide_tile(const ConvArgs& a) {
  const int ph = a.sub ? 4 : 1;
  const long long px = (long long)a.in.n_img * a.in.H * a.in.W;
  if (a.cout_pad % 256 == 0 && (px + 255) / 256 * (a.cout_pad / 256) * ph >= 512) return {256, 256};
  if (!a.sub && a.cout_pad % 128 == 0 && (px + 511) / 512 * (a.cout_pad / 128) >= 512) return {128, 512};
  return {128, 256};
}

bool conv_wide_fits(const ConvArgs& a) {
  if (a.sub) return true;
  if (a.x_f32 || a.x_split || a.ups || a.down) return false;
  if (a.mode != kModeBand && a.mode != kModeBandSplit) return false;
  if (a.cin % 32 != 0 || (a.sub && a.cin % 64 != 0) || a.cout_pad % 128 != 0) return false;
  const bool geo = (a.kt == 1 && (a.ks == 3 || a.ks == 1)) || (a.kt == 3 && a.ks == 3);
  // With 128 x 256 tiles the 1-workgroup-per-CU kernel cannot hide its fp32 epilogue
  // behind another workgroup's K loop; those layers stay on the 2-per-CU kernel.
  const WideTile t = wide_tile(a);
  return geo && !(t.bm == 128 && t.bn == 256);
}

hipError_t launch_conv_wide(ConvArgs& a, hipStream_t s) {
  a.gn_chunk = 0;
  if (a.cin % 32 != 0 || a.cout_pad % 128 != 0) return hipErrorInvalidValue;
  // split operands feed the sub-pixel form only, whose fp8 part needs 64-channel blocks and
  // its scale; the fp8 split output likewise needs 64-channel blocks
  if (a.sub != a.x_split || (a.sub && (a.kt != 1 || a.ks != 3 || a.cin % 64 != 0 || !a.sub_scale)))
    return hipErrorInvalidValue;
  if (a.split8 && (a.mode != kModeBandSplit || a.cout % 64 != 0)) return hipErrorInvalidValue;
  // a second operand: plain band output, 64-channel steps (and, below, the rows one tile
  // reads below 2 GiB)
  if (a.x2 && (a.sub || a.mode != kModeBand || a.cin2 <= 0 || a.cin2 % 64 != 0)) return hipErrorInvalidValue;
  if (!a.x2 && a.cin2 != 0) return hipErrorInvalidValue;
  if (a.in.C != (a.x_split ? 2 * a.cin : a.cin)) return hipErrorInvalidValue;
  const WideTile wt = wide_tile(a);
  const int bn = wt.bn;
  // buffer-resource addressing: the rows one tile reads (of the operand and of a second
  // operand) and the weights stay below 2 GiB, the padding offset beyond them
  for (int b = 0; b < a.in.nb; ++b) {
    const long long slot_px = tile_read_slots(a.in, b, a.kt, bn, false) * a.in.W;
    if (a.x2 && (slot_px + 2LL * bn) * a.cin2 * 2 >= (1LL << 31) - 4096) return hipErrorInvalidValue;
    if ((slot_px + 2LL * bn) * a.in.C * 2 >= (1LL << 31) - 4096) return hipErrorInvalidValue;
  }
  const long long kw = (long long)a.kt * (a.sub ? 4 * 2 : a.ks * a.ks) * a.cin + a.cin2;
  if ((long long)a.cout_pad * kw * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  // tiles over the compute pixels (the source grid for sub-pixel convs)
  int t = 0;
  for (int b = 0; b < a.in.nb; ++b) {
    a.tile_start[b] = t;
    const long long m = (long long)a.in.n_img * a.in.rows[b] * a.in.W;
    t += (int)((m + bn - 1) / bn);
  }
  a.tile_start[a.in.nb] = t;
  a.tiles_total = t;
  if (t == 0) return hipSuccess;
  const int bm = wt.bm;
  a.kernel_used = bm == 256 ? VAEP_KERNEL_CONV_WIDE256
                            : (bn == 512 ? VAEP_KERNEL_CONV_WIDE128X512 : VAEP_KERNEL_CONV_WIDE128);
  // GroupNorm tile statistics in the epilogue: whole-row pixel tiles, every group inside
  // one channel tile
  a.gn_chunk = 0;
  if (a.gn_part && (a.mode == kModeBand || (a.mode == kModeBandSplit && !a.res)) && a.in.W % bn == 0 &&
      a.cout == a.cout_pad && a.gn_groups > 0 && a.cout % a.gn_groups == 0 && (a.cout / a.gn_groups) % 4 == 0 &&
      bm % (a.cout / a.gn_groups) == 0)
    a.gn_chunk = bn;
  if (!a.gn_chunk) a.gn_part = nullptr;
  if (a.sub) return go_mode<1, 3, true, 2>(a, wt, s);
  if (a.kt == 1 && a.ks == 3) return go_mode<1, 3, false, 1>(a, wt, s);
  if (a.kt == 1 && a.ks == 1) return go_mode<1, 1, false, 1>(a, wt, s);
  if (a.kt == 3 && a.ks == 3) return go_mode<3, 3, false, 1>(a, wt, s);
  return hipErrorInvalidValue;
}

}  // namespace vaep
