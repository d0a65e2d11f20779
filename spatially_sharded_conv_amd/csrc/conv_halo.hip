// 3x3 halo convolution with the pixel operand staged once per channel block.
//
// The operation is the band conv of conv.hip and conv_wide.hip: a band's conv reads its own
// rows plus the kernel-radius halo rows its neighbours pushed into the band's halo slots,
// rows outside the image and columns outside the width read as zero, and a band writes
// only its own output rows (ChituDiffusion "VAEP" feature page, conv section; "Static
// Layer-Wise VAE Decode", operator table, "Spatial convolution" row).
//
// Layout of the work: a workgroup of 8 waves computes BM output channels x a tile of
// 4 x TW pixels as an implicit GEMM D[co][pixel] = W[co][tap, ci] X[tap, ci][pixel] on
// v_mfma_f32_32x32x16_bf16.  Tiles start at global rows that are multiples of 4 and are
// clipped at band edges (a band's first or last tile may hold fewer rows), so every pixel
// is computed by the same code on every band table.  Per 32-channel block the pixel
// operand is loaded once into LDS as the (4 + 2) x (TW + 2) halo tile, and each of the
// nine taps reads its shifted window from there; the weights of one kernel row (three
// taps) go to LDS per step.  Operand tiles travel global -> LDS by DMA; the halo tile is
// double-buffered across channel blocks and the weights across steps.  A pixel row of the
// halo tile is 32 channels (64 bytes, four 16-byte chunks); chunk c of halo pixel q sits in
// slot c ^ ((q >> 2) & 3), so 16 consecutive pixels of a fragment read hit 16 distinct
// bank groups for any window offset.  The same rule orders the weight rows.
//
// Wave w covers output channels (w / 4) * BM / 2 .. + BM / 2 and tile row w % 4: its
// GroupNorm tile statistics (one row by TW columns, per group) need no other wave.
//
// The K order of every output element is (channel block, kernel row, kernel column, 16
// channels), independent of the tile shape and the band table.
//
// X2: a second operand read at the pixel itself (a resnet's 1x1 shortcut folded into its
// conv2, a.x2 with a.cin2 channels in the input's band geometry; its weights follow the
// nine taps in every packed weight row) adds one K step per 32 of its channels after the
// taps.  Such a step stages the operand's 4 x TW tile in the centre of a halo stage and its
// weights in the centre-tap slot of a weight stage, and runs the centre tap's products.
#include "vaep_internal.h"
#include "conv_dma.h"
#include "conv_gn_stats.h"

namespace vaep {

namespace {

using dma::kPadOffset;
using dma::make_rsrc;
using dma::dma16;
using dma::lds_addr;
using dma::xcd_remap;
using dma::u32x4_t;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float nt_f32x4_t;

// Whole-line output store with the nontemporal hint: the kernel never re-reads its output,
// and lines written whole need no merging in L2 (measured: the 1024^2 decode's 128-channel
// layers 2 % faster than with plain stores).
__device__ __forceinline__ void store_line16(float* p, float4 v) {
  __builtin_nontemporal_store(nt_f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f32x4_t*>(p));
}

constexpr int kTH = 4;   // tile rows (one per pixel-wave)

__device__ __forceinline__ long long band_offset(const BandLayout& L, int b, int n, int r, int c) {
  return L.off[b] + (((long long)n * (L.rows[b] + 2) + r + 1) * L.W + c) * (long long)L.C;
}

// First tile row (in units of kTH global rows) and tile-row count of band b.
__device__ __host__ __forceinline__ int first_tile_row(const BandLayout& L, int b) { return L.row0[b] / kTH; }
__device__ __host__ __forceinline__ int tile_rows(const BandLayout& L, int b) {
  return (L.row0[b] + L.rows[b] - 1) / kTH - L.row0[b] / kTH + 1;
}

// Sum over the 32 lanes of each half-wave (DPP row butterflies and v_permlane16_swap).
__device__ __forceinline__ float half_sum(float v) { return gnstats::half_sum(v); }

template <int BM, int TW, bool X2>
__global__ void __launch_bounds__(512, 1) conv_halo(const ConvArgs a) {
  constexpr int NW = 8;
  constexpr int MI = BM / 64;                   // 32-channel blocks per wave
  constexpr int NJ = TW / 32;                   // 32-pixel blocks per wave (one tile row)
  constexpr int HW = TW + 2;                    // halo tile width
  constexpr int HPX = (kTH + 2) * HW;           // halo pixels
  constexpr int HCH = HPX * 4;                  // 16-byte chunks of a halo tile
  constexpr int HWL = (HCH + 63) / 64;          // wave-loads per halo tile
  constexpr int HROUNDS = (HWL + NW - 1) / NW;  // halo loads per thread per channel block
  constexpr int HST = HWL * 1024;               // bytes per halo stage
  constexpr int AST = 3 * BM * 64;              // bytes per weight stage (3 taps x BM rows)
  constexpr int AL = 3 * BM * 4 / (NW * 64);    // weight loads per thread per step
  static_assert(AL * NW * 64 == 3 * BM * 4, "weight chunks per thread");
  static_assert(2 * HST + 2 * AST <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * HST + 2 * AST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int wq = wave & 3;                      // tile row of this wave
  const int wco = (wave >> 2) * (BM / 2);       // first local output channel of this wave

  // work id -> (output-channel tile, pixel tile); pixel tiles of a band: image-major, then
  // tile row, then tile column
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = lin % a.tiles_total;
  const int co0 = (lin / a.tiles_total) * BM;
  const BandLayout& L = a.in;
  int band = 0;
  while (band + 1 < L.nb && mt >= a.tile_start[band + 1]) ++band;
  const int W = L.W, H = L.H, XC = L.C, C = a.cin;
  const int ctiles = W / TW;
  const int per_img = tile_rows(L, band) * ctiles;
  const int local = mt - a.tile_start[band];
  const int n = local / per_img;
  const int rem = local - n * per_img;
  const int tr = rem / ctiles;
  const int c0 = (rem - tr * ctiles) * TW;
  const int g0 = (first_tile_row(L, band) + tr) * kTH;   // global row of tile row 0
  const int rb0 = L.row0[band], rbn = L.rows[band];
  const int gw = g0 + wq;                                  // this wave's output row
  const bool row_ok = gw >= rb0 && gw < rb0 + rbn;         // wave-uniform

  // Rows the tile reads: global rows g0 - 1 .. g0 + 4, kept to the band's slots (its rows
  // and one halo row either side); rows beyond the image read as zero.
  int s_first = g0 - 1 - rb0 + 1, s_last = g0 + kTH - rb0 + 1;   // band slot indices
  if (s_first < 0) s_first = 0;
  if (s_last > rbn + 1) s_last = rbn + 1;
  const long long row_elems = (long long)W * XC;
  const long long slot0 = (long long)n * (rbn + 2) + s_first;
  const u32x4_t xrs = make_rsrc(reinterpret_cast<const unsigned short*>(a.x) + L.off[band] + slot0 * row_elems,
                                (unsigned)((long long)(s_last - s_first + 1) * row_elems * 2));
  const int cin2 = X2 ? a.cin2 : 0;
  const int kw = 9 * C + cin2;                             // packed weight row (elements)
  const u32x4_t wrs = make_rsrc(a.w, (unsigned)((long long)a.cout_pad * kw * 2));
  // second operand: the same slots of its band buffer, cin2 channels per pixel
  const u32x4_t x2rs =
      X2 ? make_rsrc(reinterpret_cast<const unsigned short*>(a.x2) + L.off[band] / XC * cin2 + slot0 * W * cin2,
                     (unsigned)((long long)(s_last - s_first + 1) * W * cin2 * 2))
         : u32x4_t{0u, 0u, 0u, 0u};

  // Halo loads of this thread: round k loads chunk (k * NW + wave) * 64 + lane of the tile.
  unsigned hoff[HROUNDS];
#pragma unroll
  for (int k = 0; k < HROUNDS; ++k) {
    const int hc = (k * NW + wave) * 64 + lane;
    const int q = hc >> 2, slot = hc & 3;
    const int hr = q / HW, hx = q - hr * HW;
    const int gr = g0 - 1 + hr, col = c0 - 1 + hx;
    const int sl = gr - rb0 + 1;                           // band slot of that row
    const bool in = hc < HCH && gr >= 0 && gr < H && col >= 0 && col < W && sl >= s_first && sl <= s_last;
    const int logical = slot ^ ((q >> 2) & 3);
    hoff[k] = in ? (unsigned)((((long long)(sl - s_first) * W + col) * XC + logical * 8) * 2) : kPadOffset;
  }
  // Second-operand loads: the same chunks of the halo stage, filled only at the tile's own
  // pixels (halo rows 1 .. 4, columns 1 .. TW) of rows inside the band; only the wave-loads
  // [X2L0, X2L1) hold such chunks.
  constexpr int X2L0 = HW * 4 / 64, X2L1 = (5 * HW * 4 + 63) / 64;
  unsigned hoff2[X2 ? HROUNDS : 1];
#pragma unroll
  for (int k = 0; k < (X2 ? HROUNDS : 1); ++k) {
    const int hc = (k * NW + wave) * 64 + lane;
    const int q = hc >> 2, slot = hc & 3;
    const int hr = q / HW, hx = q - hr * HW;
    const int gr = g0 - 1 + hr, col = c0 - 1 + hx;
    const int sl = gr - rb0 + 1;
    const bool in = X2 && hc < HCH && hr >= 1 && hr <= kTH && hx >= 1 && hx <= TW && gr >= rb0 && gr < rb0 + rbn;
    const int logical = slot ^ ((q >> 2) & 3);
    hoff2[k] = in ? (unsigned)((((long long)(sl - s_first) * W + col) * cin2 + logical * 8) * 2) : kPadOffset;
  }
  // Weight loads: chunk u * 512 + tid of a step = tap t3 (of the kernel row), row, slot.
  unsigned aoff[AL];
#pragma unroll
  for (int u = 0; u < AL; ++u) {
    const int idx = u * NW * 64 + tid;
    const int t3 = idx / (BM * 4), r2 = idx - t3 * (BM * 4);
    const int row = r2 >> 2, slot = r2 & 3;
    const int logical = slot ^ ((row >> 2) & 3);
    aoff[u] = (unsigned)((((long long)(co0 + row) * kw + t3 * C) + logical * 8) * 2);
  }
  const int ncb = C >> 5;
  const int nsteps = 3 * ncb;                              // the taps' steps
  const int ncb2 = cin2 >> 5;                              // second-operand steps after them
#define VAEP_HALO_ISSUE(st, cb, k)                                                             \
  {                                                                                            \
    if ((k) * NW + wave < HWL)                                                                 \
      dma16((k) == 0, xrs, lds_addr(smem + (st) * HST) + ((k) * NW + wave) * 1024, hoff[k], (cb) * 64); \
  }
// second-operand block e (32 channels) into halo stage st: the wave-loads holding the
// tile's own pixels
#define VAEP_X2_ISSUE(st, e, k)                                                                \
  {                                                                                            \
    if ((k) * NW + wave >= X2L0 && (k) * NW + wave < X2L1)                                     \
      dma16(true, x2rs, lds_addr(smem + (st) * HST) + ((k) * NW + wave) * 1024, hoff2[k], (e) * 64); \
  }
// weights of second-operand block e into the centre-tap slot of weight stage st
#define VAEP_A2_ISSUE(st, e)                                                                   \
  {                                                                                            \
    _Pragma("unroll") for (int u = AL / 3; u < 2 * AL / 3; ++u)                                \
      dma16(u == AL / 3, wrs, lds_addr(smem + 2 * HST + (st) * AST) + (u * NW + wave) * 1024,   \
            aoff[u], (8 * C + (e) * 32) * 2);                                                  \
  }
// weight loads of tap t3 (0..2) of step s: loads u with u * 512 / (4 BM) == t3
#define VAEP_A_ISSUE(st, s, t3)                                                                \
  {                                                                                            \
    const int cb_ = (s) / 3, dy_ = (s) - 3 * ((s) / 3);                                        \
    _Pragma("unroll") for (int u = (t3) * AL / 3; u < ((t3) + 1) * AL / 3; ++u)                \
      dma16(u == (t3) * AL / 3, wrs, lds_addr(smem + 2 * HST + (st) * AST) + (u * NW + wave) * 1024, \
            aoff[u], (3 * dy_ * C + cb_ * 32) * 2);                                            \
  }

  // Accumulators start at bias + residual (fp32, the output's band geometry).
  f32x16_t acc[MI][NJ];
  int ilane = lane;
  asm volatile("" : "+v"(ilane));
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int col = c0 + 32 * j + (ilane & 31);
    const long long ro = (a.res && row_ok) ? band_offset(a.out, band, n, gw - rb0, col) : -1;
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

  // halo pixel of the centre tap for each pixel block of this wave
  int pq[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) pq[j] = (wq + 1) * HW + 32 * j + (lane & 31) + 1;

  // prologue: the halo tile of block 0 and the weights of step 0
#pragma unroll
  for (int k = 0; k < HROUNDS; ++k) VAEP_HALO_ISSUE(0, 0, k);
  VAEP_A_ISSUE(0, 0, 0);
  VAEP_A_ISSUE(0, 0, 1);
  VAEP_A_ISSUE(0, 0, 2);

  // Step s = (channel block s / 3, kernel row s % 3) computes from halo stage (s / 3) & 1 and
  // weight stage s & 1.  Before each tap's products it issues a third of the weights of
  // step s + 1 into the other weight stage (read last in step s - 1) and a share of the next
  // block's halo tile into the other halo stage (read last in the previous block), so the
  // loads go out between groups of matrix products.  Every load issued during a step has
  // landed by the next step's barrier.
  // Fragments of sub-step u = 2 dx + kk (tap dx, 16-channel half kk) of a step; the reads
  // of sub-step u + 1 go out before the products of u (two fragment sets), so LDS latency
  // hides behind matrix work within the wave.
  auto read_frags = [&](const unsigned char* AB, const unsigned char* HB, int dy, int u, bf16x8_t(&af)[MI],
                        bf16x8_t(&bfr)[NJ]) {
    const int dx = u >> 1, c = 2 * (u & 1) + h;
    const int dq = (dy - 1) * HW + (dx - 1);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wco + 32 * i + (lane & 31);
      af[i] = *reinterpret_cast<const bf16x8_t*>(AB + (dx * BM + r) * 64 + ((c ^ ((r >> 2) & 3)) << 4));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int q = pq[j] + dq;
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(HB + q * 64 + ((c ^ ((q >> 2) & 3)) << 4));
    }
  };
  for (int s = 0; s < nsteps; ++s) {
    const int cb = s / 3, dy = s - 3 * cb;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const unsigned char* HB = smem + (cb & 1) * HST;
    const unsigned char* AB = smem + 2 * HST + (s & 1) * AST;
    bf16x8_t af[2][MI], bfr[2][NJ];
    read_frags(AB, HB, dy, 0, af[0], bfr[0]);
#pragma unroll
    for (int dx = 0; dx < 3; ++dx) {
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < nsteps) VAEP_A_ISSUE((s + 1) & 1, s + 1, dx);
      if (X2 && s + 1 == nsteps && ncb2 > 0 && dx == 1) VAEP_A2_ISSUE((s + 1) & 1, 0);
      if (cb + 1 < ncb) {
        // halo round k goes out in step dy = k * 3 / HROUNDS of the block, tap k % 3
#pragma unroll
        for (int k = 0; k < HROUNDS; ++k)
          if (k * 3 / HROUNDS == dy && k % 3 == dx) VAEP_HALO_ISSUE((cb + 1) & 1, cb + 1, k);
      } else if (X2 && ncb2 > 0) {
        // the last block stages the first second-operand tile instead
#pragma unroll
        for (int k = 0; k < HROUNDS; ++k)
          if (k * 3 / HROUNDS == dy && k % 3 == dx) VAEP_X2_ISSUE((cb + 1) & 1, 0, k);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int u = 2 * dx + kk, cur = u & 1;
        if (u + 1 < 6) read_frags(AB, HB, dy, u + 1, af[cur ^ 1], bfr[cur ^ 1]);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
      }
      // issue order: each read of the next sub-step between two products of this one
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (2 * dx + kk + 1 < 6) {
#pragma unroll
          for (int t = 0; t < MI + NJ; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          }
          __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ - (MI + NJ), 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ, 0);
        }
      }
    }
  }
  // Second-operand steps: block e sits in halo stage (ncb + e) & 1 and weight stage
  // (nsteps + e) & 1; each step stages block e + 1 into the other stages.
  if constexpr (X2) {
    for (int e = 0; e < ncb2; ++e) {
      const int s = nsteps + e;
      asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const unsigned char* HB = smem + ((ncb + e) & 1) * HST;
      const unsigned char* AB = smem + 2 * HST + (s & 1) * AST;
      bf16x8_t af[2][MI], bfr[2][NJ];
      read_frags(AB, HB, 1, 2, af[0], bfr[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (e + 1 < ncb2) {
        VAEP_A2_ISSUE((s + 1) & 1, e + 1);
#pragma unroll
        for (int k = 0; k < HROUNDS; ++k) VAEP_X2_ISSUE((ncb + e + 1) & 1, e + 1, k);
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frags(AB, HB, 1, 3, af[1], bfr[1]);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
    }
  }
#undef VAEP_HALO_ISSUE
#undef VAEP_A_ISSUE
#undef VAEP_X2_ISSUE
#undef VAEP_A2_ISSUE
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // every operand load has landed

  // Epilogue 1: fp32 band output.  Each 32-channel x 32-pixel block passes through this
  // wave's own LDS rows (36 floats per pixel), then eight lanes write one pixel's 32
  // channels (128 contiguous bytes) to its slot and, for a band's first or last row, to
  // the neighbour's halo slot.  Whole-line stores take a quarter of the L2 write requests
  // of one 16-byte piece per lane and line.
  gnstats::lds_barrier();                              // the operand stages are free now
  if (row_ok) {
    float* wl = reinterpret_cast<float*>(smem) + wave * (32 * 36);
    const BandLayout& O = a.out;
    const int r = gw - rb0;
    const long long own_row = O.off[band] + ((long long)n * (rbn + 2) + r + 1) * (long long)O.W * O.C;
    const long long up_row =
        (r == 0 && band > 0) ? O.off[band - 1] + ((long long)n * (O.rows[band - 1] + 2) + O.rows[band - 1] + 1) *
                                                     (long long)O.W * O.C
                             : -1;
    const long long dn_row =
        (r == rbn - 1 && band + 1 < O.nb) ? O.off[band + 1] + (long long)n * (O.rows[band + 1] + 2) * O.W * O.C : -1;
    float* y = reinterpret_cast<float*>(a.y);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(wl + (lane & 31) * 36 + 8 * g + 4 * h) =
              make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int cb32 = co0 + wco + 32 * i;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int px = 8 * rr + (lane >> 3), c4 = (lane & 7) * 4;
          const float4 v = *reinterpret_cast<const float4*>(wl + px * 36 + c4);
          const long long col = c0 + 32 * j + px;
          if (cb32 + c4 < a.cout) {
            store_line16(y + own_row + col * O.C + cb32 + c4, v);
            if (up_row >= 0) store_line16(y + up_row + col * O.C + cb32 + c4, v);
            if (dn_row >= 0) store_line16(y + dn_row + col * O.C + cb32 + c4, v);
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
  }

  // Epilogue 2: GroupNorm statistics of the output row (when a GroupNorm reads it next):
  // per group, mean and M2 = sum (x - mean)^2 over the TW pixels of this row and tile and
  // the group's channels, two-pass; record (image * H + row) * (W / TW) + column / TW in
  // the group-major layout of gnstats::record.
  if (a.gn_part && row_ok) {
    const int cg = a.cout / a.gn_groups;               // 4, 8 or 16 (the launch checks)
    const double cnt = (double)TW * cg;
    const long long rec = ((long long)n * H + gw) * ctiles + c0 / TW;
    const long long tiles = (long long)H * ctiles;
    // quad sums: channels co0 + wco + 32 i + 8 g + 4 h + 0..3 over the wave's pixels
    float qs[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) t += acc[i][j][4 * g + e];
        qs[i][g] = half_sum(t);
      }
    // group sums in every lane: quads (i, g, h) of the group -- cg = 4: (i, g, h) itself;
    // 8: both halves of (i, g); 16: both halves of (i, 2 (g / 2)) and (i, 2 (g / 2) + 1)
    auto group_sum = [&](float (&q)[MI][4], float (&out)[MI][4]) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // halves added in the order (h = 0) + (h = 1) in both halves
          float t = q[i][g];
          if (cg >= 8) {
            const float o = __shfl_xor(t, 32);
            t = h ? o + t : t + o;
          }
          if (cg >= 16) {
            float u = q[i][g ^ 1];
            const float o = __shfl_xor(u, 32);
            u = h ? o + u : u + o;
            t = (g & 1) ? u + t : t + u;
          }
          out[i][g] = t;
        }
    };
    float gs[MI][4];
    group_sum(qs, gs);
    float mean[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) mean[i][g] = (float)((double)gs[i][g] / cnt);
    // pass 2: squared deviations from the group mean
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float m = mean[i][g];
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = acc[i][j][4 * g + e] - m;
            t = fmaf(d, d, t);
          }
        qs[i][g] = half_sum(t);
      }
    float gm2[MI][4];
    group_sum(qs, gm2);
    // one lane per group writes the record
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cfirst = wco + 32 * i + 8 * g + 4 * h;          // first channel of this quad
        const bool writer = (lane & 31) == 0 && (cfirst % cg) == 0;
        if (writer) {
          const int grp = (co0 + cfirst) / cg;
          // M2 about the fp32 mean m_f equals M2 about the exact mean + n (mean - m_f)^2
          const double mx = (double)gs[i][g] / cnt;
          const double d = mx - (double)mean[i][g];
          const double m2 = (double)gm2[i][g] - cnt * d * d;
          double* pr = gnstats::record(a.gn_part, rec, grp, a.gn_groups, tiles);
          pr[0] = mx;
          pr[1] = m2 > 0.0 ? m2 : 0.0;
        }
      }
  }
}

template <int BM, int TW>
hipError_t go(const ConvArgs& a, hipStream_t s) {
  const long long wgs = (long long)a.tiles_total * (a.cout_pad / BM);
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.x2)
    hipLaunchKernelGGL((conv_halo<BM, TW, true>), dim3((unsigned)wgs), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((conv_halo<BM, TW, false>), dim3((unsigned)wgs), dim3(512), 0, s, a);
  return hipGetLastError();
}

// Tile shape for a layer: 128 channels x (4 x 128) pixels for 128-channel outputs, 256 x
// (4 x 64) for multiples of 256.  0 = the layer does not fit this kernel.  The 256-channel
// tile runs only on images at least 512 pixels wide: on 256-pixel-wide 512-channel layers
// its 64-byte weight pieces (three taps of 32 channels per step) cost more than the halo
// tile saves, and the wide kernel is 20-30 % faster there (measured on the 1024^2 decode's
// 256^2 stage).
int halo_bm(const ConvArgs& a) {
  if (a.cout_pad % 256 == 0) return a.in.W >= 512 ? 256 : 0;
  if (a.cout_pad == 128) return 128;
  return 0;
}

}  // namespace

// The layer runs on the halo kernel when it is a plain 3x3 2-D conv into an fp32 band
// output, its width holds whole tiles, channels come in 32-channel blocks, and its tiles
// fill the GPU.  Decided on the layer's shape alone: every band table of a layer uses the
// same kernel.
bool conv_halo_fits(const ConvArgs& a) {
  if (a.kt != 1 || a.ks != 3 || a.ups || a.down || a.sub || a.x_split || a.x_f32) return false;
  // a folded 1x1 second operand in 32-channel steps
  if ((a.x2 != nullptr) != (a.cin2 > 0) || a.cin2 % 32 != 0) return false;
  if (a.mode != kModeBand || a.split8) return false;
  if (a.cin % 32 != 0 || a.in.C != a.cin || a.cout != a.cout_pad) return false;
  const int bm = halo_bm(a);
  if (!bm) return false;
  const int tw = bm == 128 ? 128 : 64;
  if (a.in.W % tw != 0) return false;
  const long long tiles = (long long)a.in.n_img * ((a.in.H + kTH - 1) / kTH) * (a.in.W / tw) * (a.cout_pad / bm);
  return tiles >= 512;
}

hipError_t launch_conv_halo(ConvArgs& a, hipStream_t s) {
  if (!conv_halo_fits(a)) return hipErrorInvalidValue;
  const int bm = halo_bm(a);
  const int tw = bm == 128 ? 128 : 64;
  // buffer-resource addressing: six rows of the input, and the weights, below 2 GiB
  if ((long long)(kTH + 2) * a.in.W * a.in.C * 2 >= (1LL << 31) - 4096) return hipErrorInvalidValue;
  if ((long long)a.cout_pad * (9 * a.cin + a.cin2) * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  if ((long long)(kTH + 2) * a.in.W * a.cin2 * 2 >= (1LL << 31) - 4096) return hipErrorInvalidValue;
  if (a.out.W != a.in.W || a.out.C < a.cout || a.out.nb != a.in.nb) return hipErrorInvalidValue;
  int t = 0;
  for (int b = 0; b < a.in.nb; ++b) {
    a.tile_start[b] = t;
    t += a.in.n_img * tile_rows(a.in, b) * (a.in.W / tw);
  }
  a.tile_start[a.in.nb] = t;
  a.tiles_total = t;
  a.kernel_used = a.x2 ? VAEP_KERNEL_CONV_HALO_X2 : VAEP_KERNEL_CONV_HALO;
  // GroupNorm records of the output: one-row slabs, chunks of the tile width; every group
  // inside one wave's channels
  a.gn_chunk = 0;
  if (a.gn_part && a.gn_groups > 0 && a.cout % a.gn_groups == 0) {
    const int cg = a.cout / a.gn_groups;
    if ((cg == 4 || cg == 8 || cg == 16) && (bm / 2) % cg == 0) a.gn_chunk = tw;
  }
  if (!a.gn_chunk) a.gn_part = nullptr;
  if (t == 0) return hipSuccess;
  if (bm == 128) return go<128, 128>(a, s);
  return go<256, 64>(a, s);
}

}  // namespace vaep
