// Whole-line epilogues of the LDS-staged convolution kernels (gfx950).
//
// After its K loop a conv workgroup holds its output tile in the matrix-core accumulator
// layout: acc[i][j][v] is local channel wco + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4 of
// tile pixel wpx + 32 j + lane % 32, so one 16-byte store of a lane covers 4 channels of
// one pixel and a store instruction touches 32 pixels in 32-byte pieces.  The epilogues
// here pass each 32-channel x 32-pixel block through the wave's own LDS rows first; eight
// lanes then own one pixel and write whole 128-byte lines, with the nontemporal hint (the
// kernel never re-reads its output, and whole lines need no merging in L2).  Outputs are
// the band layout of ChituDiffusion "VAEP" feature page, conv section: a band's own rows,
// and a band's first / last row also into the neighbour's halo slot.
#pragma once

#include "vaep_internal.h"
#include "split8.h"

namespace vaep {
namespace epi {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ unsigned short f2bf(float v) {
  __hip_bfloat16 h = __float2bfloat16(v);
  return *reinterpret_cast<unsigned short*>(&h);
}
__device__ __forceinline__ float bf2f(unsigned short u) { return __uint_as_float(((unsigned)u) << 16); }

__device__ __forceinline__ long long band_offset(const BandLayout& L, int b, int n, int r, int c) {
  return L.off[b] + (((long long)n * (L.rows[b] + 2) + r + 1) * L.W + c) * (long long)L.C;
}

// 16-byte global store with the nontemporal hint, for epilogues that write whole 128-byte
// lines: the kernel never re-reads its output, and whole lines need no merging in L2.
typedef __attribute__((ext_vector_type(4))) unsigned nt_u32x4_t;
typedef __attribute__((ext_vector_type(4))) float nt_f32x4_t;
__device__ __forceinline__ void store_line16(void* p, uint4 v) {
  __builtin_nontemporal_store(nt_u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4_t*>(p));
}
__device__ __forceinline__ void store_line16(void* p, float4 v) {
  __builtin_nontemporal_store(nt_f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f32x4_t*>(p));
}

// Output slots of compute pixel p of the tile's band (own slot; halo slots in the bands
// above / below for a band's first / last row, -1 where there is none); own = -1 past the
// band's pixels.
template <bool SUB>
__device__ __forceinline__ void out_slots(const ConvArgs& a, int band, long long p, long long m_band, int plane,
                                          int W, int py, int px, long long& own, long long& hu, long long& hd) {
  own = hu = hd = -1;
  if (p >= m_band) return;
  const int n = (int)(p / plane);
  const int rem = (int)(p - (long long)n * plane);
  int r = rem / W;
  int c = rem - r * W;
  if (SUB) {
    r = 2 * r + py;
    c = 2 * c + px;
  }
  own = band_offset(a.out, band, n, r, c);
  if (r == 0 && band > 0) hu = band_offset(a.out, band - 1, n, a.out.rows[band - 1], c);
  if (r == a.out.rows[band] - 1 && band + 1 < a.out.nb) hd = band_offset(a.out, band + 1, n, -1, c);
}

// Split output (bf16 hi and lo planes, no fp8 bytes).  Per pixel block and pair of
// 32-channel blocks the wave passes its accumulators through its own LDS
// rows (68 floats per pixel); eight lanes then own one pixel's 64 channels, 8 each, and
// write its 128-byte hi line and 128-byte lo line.  wl: this wave's 32 x 68 floats, free.
template <bool SUB, int MI, int NJ, int BN>
__device__ __forceinline__ void split_epilogue_lines(const ConvArgs& a, const f32x16_t (&acc)[MI][NJ], int band,
                                                     int tile, int plane, long long m_band, int W, int py, int px,
                                                     int co0, int wco, int wpx, int lane, float* wl) {
  static_assert(MI % 2 == 0, "pairs of channel blocks");
  const int h = lane >> 5;
  const int half = a.cout;
  const int c8 = (lane & 7) * 8;
  unsigned short* y = reinterpret_cast<unsigned short*>(a.y);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    long long own[4], hu[4], hd[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      out_slots<SUB>(a, band, (long long)tile * BN + wpx + 32 * j + 8 * rr + (lane >> 3), m_band, plane, W, py, px,
                     own[rr], hu[rr], hd[rr]);
#pragma unroll
    for (int ip = 0; ip < MI / 2; ++ip) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(wl + (lane & 31) * 68 + 32 * t + 8 * g + 4 * h) =
              make_float4(acc[2 * ip + t][j][4 * g], acc[2 * ip + t][j][4 * g + 1], acc[2 * ip + t][j][4 * g + 2],
                          acc[2 * ip + t][j][4 * g + 3]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int co = co0 + wco + 64 * ip + c8;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float* src = wl + (8 * rr + (lane >> 3)) * 68 + c8;
        const float4 v0 = *reinterpret_cast<const float4*>(src);
        const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
        const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        unsigned hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned short h0 = f2bf(v[2 * e]), h1 = f2bf(v[2 * e + 1]);
          const unsigned short l0 = f2bf(v[2 * e] - bf2f(h0)), l1 = f2bf(v[2 * e + 1] - bf2f(h1));
          hw[e] = (unsigned)h0 | ((unsigned)h1 << 16);
          lw[e] = (unsigned)l0 | ((unsigned)l1 << 16);
        }
        if (own[rr] < 0 || co >= a.cout) continue;
        const uint4 hv = make_uint4(hw[0], hw[1], hw[2], hw[3]), lv = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        store_line16(y + own[rr] + co, hv);
        store_line16(y + own[rr] + half + co, lv);
        if (hu[rr] >= 0) {
          store_line16(y + hu[rr] + co, hv);
          store_line16(y + hu[rr] + half + co, lv);
        }
        if (hd[rr] >= 0) {
          store_line16(y + hd[rr] + co, hv);
          store_line16(y + hd[rr] + half + co, lv);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

// Split output in the fp8 encoding of split8.h.  After the same LDS transpose as
// split_epilogue_lines, lane k (of the eight on a pixel) owns channels
// 8k .. 8k+7 of a 64-channel block: it stores their bf16 hi parts (eight lanes, one
// 128-byte line).  The block's fp8 bytes are a second 128-byte line, 64 bytes of x_lo then
// 64 of x; lanes 2m and 2m+1 swap halves (one DPP move) so that lane 2m stores the x_lo
// bytes of channels 16m .. 16m+15 and lane 2m+1 their x bytes, 16 contiguous bytes each.
template <bool SUB, int MI, int NJ, int BN>
__device__ __forceinline__ void split8_epilogue_lines(const ConvArgs& a, const f32x16_t (&acc)[MI][NJ], int band,
                                                      int tile, int plane, long long m_band, int W, int py,
                                                      int px, int co0, int wco, int wpx, int lane, float* wl) {
  static_assert(MI % 2 == 0, "pairs of channel blocks");
  const int h = lane >> 5;
  const int half = a.cout;
  const int k8 = lane & 7;
  const bool odd = k8 & 1;
  unsigned short* y = reinterpret_cast<unsigned short*>(a.y);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    long long own[4], hu[4], hd[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      out_slots<SUB>(a, band, (long long)tile * BN + wpx + 32 * j + 8 * rr + (lane >> 3), m_band, plane, W, py, px,
                     own[rr], hu[rr], hd[rr]);
#pragma unroll
    for (int ip = 0; ip < MI / 2; ++ip) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(wl + (lane & 31) * 68 + 32 * t + 8 * g + 4 * h) =
              make_float4(acc[2 * ip + t][j][4 * g], acc[2 * ip + t][j][4 * g + 1], acc[2 * ip + t][j][4 * g + 2],
                          acc[2 * ip + t][j][4 * g + 3]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int cblk = co0 + wco + 64 * ip;   // first channel of the 64-channel block
      const int co = cblk + 8 * k8;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float* src = wl + (8 * rr + (lane >> 3)) * 68 + 8 * k8;
        const float4 v0 = *reinterpret_cast<const float4*>(src);
        const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
        const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint4 hv;
        hv.x = (unsigned)f2bf(v[0]) | ((unsigned)f2bf(v[1]) << 16);
        hv.y = (unsigned)f2bf(v[2]) | ((unsigned)f2bf(v[3]) << 16);
        hv.z = (unsigned)f2bf(v[4]) | ((unsigned)f2bf(v[5]) << 16);
        hv.w = (unsigned)f2bf(v[6]) | ((unsigned)f2bf(v[7]) << 16);
        uint2 lo, xs;
        split8::operand_bytes4(v, &lo.x, &xs.x);
        split8::operand_bytes4(v + 4, &lo.y, &xs.y);
        // even lanes send their x bytes and keep their x_lo bytes; odd lanes the reverse
        const uint2 send = odd ? lo : xs;
        uint2 recv;
        recv.x = (unsigned)__builtin_amdgcn_update_dpp(0, (int)send.x, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
        recv.y = (unsigned)__builtin_amdgcn_update_dpp(0, (int)send.y, 0xB1, 0xf, 0xf, false);
        const uint4 fv = odd ? make_uint4(recv.x, recv.y, xs.x, xs.y) : make_uint4(lo.x, lo.y, recv.x, recv.y);
        if (own[rr] < 0 || co >= a.cout) continue;
        // this lane's 16 fp8 bytes: x_lo (even) or x (odd) of channels cblk + 16 (k8 / 2) ..
        const long long fb = split8::lo_byte(half, cblk) + 16 * (k8 >> 1) + (odd ? 64 : 0);
        auto put = [&](long long q) {
          store_line16(y + q + co, hv);
          store_line16(reinterpret_cast<unsigned char*>(y + q) + fb, fv);
        };
        put(own[rr]);
        if (hu[rr] >= 0) put(hu[rr]);
        if (hd[rr] >= 0) put(hd[rr]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

// Plain fp32 output: each 32-channel x 32-pixel block passes through the wave's LDS rows
// (68 floats per pixel), then eight lanes write one pixel's 32 channels, a whole line.
// wl: this wave's 32 x 68 floats, free.
template <bool SUB, int MI, int NJ, int BN>
__device__ __forceinline__ void band_epilogue_lines(const ConvArgs& a, const f32x16_t (&acc)[MI][NJ], int band,
                                                    int tile, int plane, long long m_band, int W, int py, int px,
                                                    int co0, int wco, int wpx, int lane, float* wl) {
  float* y = reinterpret_cast<float*>(a.y);
  const int c4 = (lane & 7) * 4;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    long long own[4], hu[4], hd[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      out_slots<SUB>(a, band, (long long)tile * BN + wpx + 32 * j + 8 * rr + (lane >> 3), m_band, plane, W, py,
                     px, own[rr], hu[rr], hd[rr]);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(wl + (lane & 31) * 68 + 8 * g + 4 * (lane >> 5)) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int co = co0 + wco + 32 * i + c4;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 v = *reinterpret_cast<const float4*>(wl + (8 * rr + (lane >> 3)) * 68 + c4);
        if (own[rr] < 0 || co >= a.cout) continue;
        store_line16(y + own[rr] + co, v);
        if (hu[rr] >= 0) store_line16(y + hu[rr] + co, v);
        if (hd[rr] >= 0) store_line16(y + hd[rr] + co, v);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

}  // namespace epi
}  // namespace vaep
