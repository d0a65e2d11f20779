// GroupNorm tile statistics computed in a convolution's epilogue (the consumer of the
// conv output is a GroupNorm): the first half of the statistics pass moves into the
// producer, so the norm no longer re-reads its input to form local moments.
//
// The statistics are the same local central moments as the standalone pass (ChituDiffusion
// "VAEP" feature page, GroupNorm section): per tile and group, mean and M2 = sum (x -
// mean)^2, two-pass over the tile's values, later merged with element-count weights.  A
// tile is the conv workgroup's pixel tile -- BN consecutive pixels of one image row (the
// launch requires the row width to be a multiple of BN) -- so the tiling is a function of
// the image alone and band decodes stay bit-identical to the full decode.  Tile index:
// (image * rows + row) * (W / BN) + column / BN, the tiling gn_merge reads with one-row
// slabs and BN-pixel chunks; records are stored group-major (see record()).
#pragma once

#include "vaep_internal.h"

namespace vaep {
namespace gnstats {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// Workgroup barrier for LDS traffic only: every wave's LDS operations have completed, but
// its global stores (the epilogue's output) stay in flight.  __syncthreads would also wait
// for those, serialising the store latency of the whole tile.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over the 32 lanes of each half-wave (lanes 0-31 and 32-63 separately), in the VALU:
// DPP butterflies within each row of 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror), then rows 0+1 and 2+3 through v_permlane16_swap.
__device__ __forceinline__ float half_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// val[i][j][v] holds the final value (what the norm reads) of local channel
// wco + 32i + 8(v/4) + 4(lane/32) + v%4 and tile pixel wpx + 32j + lane%32.  Waves are laid
// out WPX along the pixels and NWAVES/WPX along the channels (wave w: channel half w/WPX).
// lds: at least NWAVES*MI*8 + BM floats + BM/4 doubles of workgroup scratch no other thread
// uses meanwhile.  cg: channels per group (multiple of 4, divides BM).  part: the tile's
// record of the workgroup's first group, (mean, M2) doubles; the next group's record is
// `gstride` doubles further (the group-major layout of record()).
// Contains LDS barriers (lds_barrier); every thread of the workgroup must call it, and
// the caller must have passed an lds_barrier since the last use of `lds` for anything else.
// SPLITV: the output is stored as bf16 hi / lo parts, which the norm reads back as
// hi + lo (exact in fp32); the moments are taken of that value.
__device__ __forceinline__ float bf16_round(float v) {
  return __bfloat162float(__float2bfloat16(v));
}
template <bool SPLITV>
__device__ __forceinline__ float seen(float v) {
  if (!SPLITV) return v;
  const float hi = bf16_round(v);
  return hi + bf16_round(v - hi);
}
template <int MI, int NJ, int NWAVES, int WPX, int BM, bool SPLITV>
__device__ __forceinline__ void tile_stats(const f32x16_t (&val)[MI][NJ], int wave, int lane, int cg,
                                           int tile_pixels, double* part, long long gstride, float* lds) {
  constexpr int NQ = MI * 8;                  // 4-channel quads per wave (both half-waves)
  float* qs = lds;                            // [NWAVES][NQ] quad sums
  float* gmean = lds + NWAVES * NQ;           // [BM / 4] group means (fp32), indexed by group
  double* gm64 = reinterpret_cast<double*>(gmean + BM);   // [BM / 4] group means (fp64)
  const int h = lane >> 5;
  const int ngroups = BM / cg;
  const double cnt = (double)tile_pixels * cg;
  const int wc = wave / WPX;                  // channel half of this wave
  constexpr int WAVE_CH = BM / (NWAVES / WPX);
  // group sums over quads of waves: quad q of wave w covers local channel
  // (w / WPX) * WAVE_CH + 32 (q / 8) + 8 ((q % 8) / 2) + 4 (q % 2)
  auto reduce_groups = [&](bool second) {
    lds_barrier();
    if ((int)threadIdx.x < ngroups) {
      const int gi = threadIdx.x;
      double s = 0.0;
      for (int c = gi * cg; c < (gi + 1) * cg; c += 4) {
        const int w_c = c / WAVE_CH, rem = c - w_c * WAVE_CH;
        const int q = (rem / 32) * 8 + ((rem % 32) / 8) * 2 + (rem % 8) / 4;
        for (int wp = 0; wp < WPX; ++wp) s += (double)qs[(w_c * WPX + wp) * NQ + q];
      }
      if (!second) {
        const double m = s / cnt;
        gm64[gi] = m;
        gmean[gi] = (float)m;
      } else {
        // sum (x - m_f)^2 = M2 + n (m - m_f)^2 with m_f the fp32 mean used by the lanes
        const double d = gm64[gi] - (double)gmean[gi];
        double m2 = s - cnt * d * d;
        part[gi * gstride] = gm64[gi];
        part[gi * gstride + 1] = m2 > 0.0 ? m2 : 0.0;
      }
    }
    if (!second) lds_barrier();   // the group means are read by every lane next
  };
  // pass 1: sums
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += seen<SPLITV>(val[i][j][4 * g + e]);
      s = half_sum(s);
      if ((lane & 31) == 0) qs[wave * NQ + (i * 4 + g) * 2 + h] = s;
    }
  reduce_groups(false);
  // pass 2: squared deviations from the group mean
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = wc * WAVE_CH + 32 * i + 8 * g + 4 * h;
      const float m = gmean[c / cg];
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = seen<SPLITV>(val[i][j][4 * g + e]) - m;
          s = fmaf(d, d, s);
        }
      s = half_sum(s);
      if ((lane & 31) == 0) qs[wave * NQ + (i * 4 + g) * 2 + h] = s;
    }
  reduce_groups(true);
}

// Records are stored [image][group][tile of the image][2] doubles (mean, M2), `tiles` per
// image and group, so that the merge reads each group's records contiguously.  rec: the
// tile's index image * tiles + tile; g: the group.
__device__ __forceinline__ double* record(double* gn_part, long long rec, int g, int groups, long long tiles) {
  const long long n = rec / tiles;
  return gn_part + ((n * groups + g) * tiles + (rec - n * tiles)) * 2;
}

// Record of the tile holding pixel p0 (first pixel of the workgroup tile) of band b in the
// layout `out` (one-row slabs, chunks of `bn` pixels), or of its sub-pixel phase tile:
// output row 2r + py, chunk px * (W / bn) + c / bn on the source grid of width W.
__device__ __forceinline__ long long tile_record(const BandLayout& out, int b, int n, int r_out, int chunk,
                                                 int chunks) {
  return ((long long)n * out.H + out.row0[b] + r_out) * chunks + chunk;
}

}  // namespace gnstats
}  // namespace vaep
