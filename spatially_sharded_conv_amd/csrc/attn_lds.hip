// AGKV attention, bf16 operands, d = 384 and 512: K and V staged in LDS, whole query rows
// per wave.
//
// ChituDiffusion "VAEP" feature page, attention section, and "Static Layer-Wise VAE
// Decode", attention row: each band's queries attend over the global K/V (gathered once by
// the QKV projection, which writes them token-major and channel-major), and the band keeps
// its own output rows.  Single head, d = channels, scale 1/sqrt(d).
//
// A workgroup owns 128 queries of one band and image, 32 per wave, and each wave keeps
// whole rows of its queries: Q^T (bf16) and O^T (fp32, d x 32) in registers, so no product
// is split over waves and the softmax never leaves the wave.  Per 32-key tile the four
// waves load the K tile (token-major rows) and the V^T tile (d rows of 32 keys) into LDS
// once, with direct buffer-to-LDS loads spread between the S products; two stages, so
// tile t + 1 lands while tile t is computed, and one barrier per tile.  Each wave then
//   1. forms S^T = K Q^T (v_mfma_f32_32x32x16_bf16, K fragments read from LDS),
//   2. runs the online softmax of its 32 queries in fp32 (exp2 domain); the two 16-key
//      halves of a query's column meet through v_permlane32_swap,
//   3. accumulates O^T += V^T P^T, P^T taken straight from the S^T accumulators.
// The lane that supplies K row r of the S product reads key sigma(r), sigma swapping bits 2
// and 3 of r.  A lane's 16 accumulators then hold two runs of 8 consecutive keys, which is
// the P^T operand of the PV product's two 16-key steps, and the matching V^T fragments are
// plain 16-byte reads.  In LDS the 16-byte chunks of K row r are XOR-permuted by r & 15 and
// those of V^T row d by (d >> 2) & 3, so the fragment reads are free of bank conflicts.
// The running max moves only when a query's tile max passes it by more than 8 (P <= 256
// otherwise; numerator and denominator share the max, so the result is unchanged) and the
// O rescale runs only on tiles that move one.  With keys split in two halves (a.part set)
// workgroup 2 i + s takes query block i against half s of the key tiles and writes its
// unnormalised O and (max, sum) for attn_merge.  Every query's sums run over the same key
// tiles in the same order, whatever band or block holds it.
//
// Registers at d = 512: O^T takes all 256 accumulation registers and Q^T 128 of the 256
// VGPRs, so the S^T products are written in VGPR form (inline asm) and the PV products in
// the builtin's accumulation-register form.
#include "vaep_internal.h"
#include "conv_dma.h"

namespace vaep {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

namespace {

__device__ __forceinline__ unsigned short to_bf16(float v) {
  __hip_bfloat16 h = __float2bfloat16(v);
  return *reinterpret_cast<unsigned short*>(&h);
}

template <int D>
__global__ void __launch_bounds__(256, 1) attn_lds(const AttnArgs a) {
  using namespace dma;
  constexpr int KS = D / 16;          // 16-channel steps of S^T
  constexpr int CB = D / 32;          // 32-channel blocks of O^T
  constexpr int BK = 32;              // keys per tile
  constexpr int NQ = 128;             // queries per workgroup
  constexpr int RC = D / 8;           // 16-byte chunks of a K row
  constexpr int KT = BK * D * 2;      // bytes of a K tile, and of a V^T tile
  constexpr int ST = 2 * KT;          // bytes of a stage: K tile, then V^T tile
  constexpr int KP = KT / 1024;       // 1 KiB pieces of a K tile
  constexpr int NI = 2 * KP / 4;      // pieces per wave and tile
  constexpr int RD = 4;               // LDS fragment ring depth
  static_assert(RC % 16 == 0 && KT % 4096 == 0 && KS >= 2 * NI, "tile shape");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * ST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsplit = a.part ? 2 : 1;
  const int blk = blockIdx.x / nsplit, half = blockIdx.x - blk * nsplit;
  int b = 0;
  while (b + 1 < a.L.nb && blk >= a.tile_start[b + 1]) ++b;
  const int local = blk - a.tile_start[b];
  const int W = a.L.W;
  const int nq = a.L.rows[b] * W;
  const int qt_img = (nq + NQ - 1) / NQ;
  const int n = local / qt_img;
  const int q0 = (local - n * qt_img) * NQ + 32 * wave;   // this wave's first query
  const int tokens = a.tokens;
  const long long tok0 = (long long)a.L.row0[b] * W;
  const int l32 = lane & 31, h = lane >> 5;

  const unsigned tbytes = (unsigned)tokens * D * 2;   // < 2 GiB, host-checked
  const u32x4_t krs = make_rsrc(reinterpret_cast<const unsigned short*>(a.k) + (long long)n * tokens * D, tbytes);
  const u32x4_t vrs = make_rsrc(reinterpret_cast<const unsigned short*>(a.vt) + (long long)n * D * tokens, tbytes);

  // Piece u = 4 j + wave of a tile fills stage bytes [1024 u, 1024 u + 1024), lane chunk
  // p = 64 u + lane: pieces j < NI / 2 of every wave are K pieces (u < KP), the rest V^T
  // pieces.  K: tile row r = p / RC; stored chunk s of a row holds the row's source chunk
  // s ^ (r & 15).  V^T: row d = 16 (u - KP) + lane / 4; stored chunk s = lane % 4 holds keys
  // 8 c .. 8 c + 7 of the tile, c = s ^ ((d >> 2) & 3) = s ^ ((lane >> 4) & 3).  A piece past
  // the last key reads zeros.
  static_assert(4 * (NI / 2) == KP, "piece split");
  const int vc = (lane & 3) ^ ((lane >> 4) & 3);
  const unsigned vlane = (unsigned)((lane >> 2) * tokens + 8 * vc) * 2u;
#define VAEP_KV_PIECE(j, st, k0)                                                                \
  {                                                                                             \
    const int u = 4 * (j) + wave;                                                               \
    const unsigned lds = lds_addr(smem + (st) * ST) + u * 1024;                                 \
    if ((j) < NI / 2) {                                                                         \
      const int p = 64 * u + lane, r = p / RC, c = (p - r * RC) ^ (r & 15);                     \
      const unsigned off = (unsigned)(((k0) + r) * D + 8 * c) * 2u;                             \
      dma16(false, krs, lds, (k0) + r < tokens ? off : kPadOffset, 0);                          \
    } else {                                                                                    \
      const unsigned off = vlane + (unsigned)(16 * (u - KP) * tokens + (k0)) * 2u;              \
      dma16(false, vrs, lds, (k0) + 8 * vc < tokens ? off : kPadOffset, 0);                     \
    }                                                                                           \
  }

  // Q^T fragments (B operand of S^T): query q0 + lane % 32 (clamped), channels 16 ks + 8 h
  bf16x8_t qf[KS];
  {
    const int ql = q0 + l32 < nq ? q0 + l32 : nq - 1;
    const unsigned short* qr =
        reinterpret_cast<const unsigned short*>(a.q) + ((long long)n * tokens + tok0 + ql) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * ks);
    // wait for Q here: the loop's own loads are not counted by the compiler, so a wait for
    // Q placed inside the loop would also wait for them
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  f32x16_t oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[cb][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const int ntiles = (tokens + BK - 1) / BK;
  const int tper = (ntiles + nsplit - 1) / nsplit;
  const int tbeg = half * tper;
  const int tend = tbeg + tper < ntiles ? tbeg + tper : ntiles;
  // K row read by this lane: sigma(lane % 32)
  const int srow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const int kfo = srow * RC * 16, kx = srow & 15;
  // V^T row 32 cb + lane % 32: swizzle term ((lane % 32) >> 2) & 3
  const int vfo = l32 * 64, vx = (l32 >> 2) & 3;

  if (tbeg < tend) {
#pragma unroll
    for (int j = 0; j < NI; ++j) VAEP_KV_PIECE(j, 0, tbeg * BK);
  }
  for (int t = tbeg; t < tend; ++t) {
    const int st = (t - tbeg) & 1;
    const int k0 = t * BK;
    // tile t has landed (every wave's pieces); every wave is done with tile t - 1
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const unsigned char* KB = smem + st * ST;
    const unsigned char* VB = KB + KT;

    // S^T: the products in VGPR form (inline asm; the builtin form would put S^T in the
    // accumulation registers, which O^T fills), one chain accumulating in place (no wait
    // states between its products); 24 after the last one cover its VALU readers.  (Two
    // chains, even and odd channel steps, changed the decode beyond what the summation
    // order explains, so the single chain stays.)  K fragments
    // come through a ring of RD, read RD - 1 products ahead (LDS latency under load is
    // several products long), fenced so the scheduler keeps that depth.
    f32x16_t sacc;
    bf16x8_t kf[RD];
#pragma unroll
    for (int i = 0; i < RD - 1; ++i)
      kf[i] = *reinterpret_cast<const bf16x8_t*>(KB + kfo + (((2 * i + h) ^ kx) << 4));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + RD - 1 < KS)
        kf[(ks + RD - 1) % RD] =
            *reinterpret_cast<const bf16x8_t*>(KB + kfo + (((2 * (ks + RD - 1) + h) ^ kx) << 4));
      // tile t + 1 into the other stage (after the last tile: a tile nobody reads, past the
      // last key or in the other key half)
      if ((ks & 1) == 0 && ks / 2 < NI) VAEP_KV_PIECE(ks / 2, st ^ 1, k0 + BK);
      if (ks == 0)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                     : "=&v"(sacc) : "v"(kf[0]), "v"(qf[0]));
      else if (ks + 1 < KS)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+v"(sacc) : "v"(kf[ks % RD]), "v"(qf[ks]));
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(sacc) : "v"(kf[ks % RD]), "v"(qf[ks]));
      __builtin_amdgcn_sched_barrier(0);
    }

    // lane: query q0 + lane % 32; sacc[v] is key k0 + 16 (v >> 3) + 8 h + (v & 7)
    float sv[16];
    float rmax = -INFINITY;
    if (k0 + BK > tokens) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sv[v] = k0 + 16 * (v >> 3) + 8 * h + (v & 7) < tokens ? sacc[v] * sl2 : -INFINITY;
        rmax = fmaxf(rmax, sv[v]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sv[v] = sacc[v] * sl2;
        rmax = fmaxf(rmax, sv[v]);
      }
    }
    {
      const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
      rmax = fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
    }
    const bool need = rmax > m_run + 8.f;
    const float m_new = need ? rmax : m_run;
    const float alpha = need ? exp2f(m_run - m_new) : 1.f;
    // P = 2^(s - m) <= 256; v_exp_f32 flushes results below 2^-126 to zero
    float rs = 0.f;
    unsigned pk[8];
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sv[v] - m_new), p1 = __builtin_amdgcn_exp2f(sv[v + 1] - m_new);
      rs += p0 + p1;
      pk[v / 2] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t));
    }
    {
      // the two halves added in the same order in both lanes of a query
      const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
      rs = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // in place in the accumulation register (a VALU multiply there would make the
          // allocator move O^T out of those registers)
          float x = oacc[cb][v], tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\ts_nop 1\n\tv_mul_f32 %1, %1, %2\n\ts_nop 1\n\t"
                       "v_accvgpr_write_b32 %0, %1"
                       : "+a"(x), "=&v"(tmp) : "v"(alpha));
          oacc[cb][v] = x;
        }
      asm volatile("s_nop 4");   // accumulation-register writes before the next products read them
    }
    // O^T += V^T P^T, V^T fragments through a ring of RD
    const bf16x8_t pf[2] = {
        __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3])),
        __builtin_bit_cast(bf16x8_t, make_uint4(pk[4], pk[5], pk[6], pk[7]))};
#define VAEP_VFRAG(i) \
  (*reinterpret_cast<const bf16x8_t*>(VB + ((i) % CB) * 2048 + vfo + (((2 * ((i) / CB) + h) ^ vx) << 4)))
    bf16x8_t vf[RD];
#pragma unroll
    for (int i = 0; i < RD - 1; ++i) vf[i] = VAEP_VFRAG(i);
#pragma unroll
    for (int i = 0; i < 2 * CB; ++i) {
      if (i + RD - 1 < 2 * CB) vf[(i + RD - 1) % RD] = VAEP_VFRAG(i + RD - 1);
      oacc[i % CB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % RD], pf[i / CB], oacc[i % CB], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#undef VAEP_VFRAG
  }
#undef VAEP_KV_PIECE
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load into LDS outlives the workgroup

  // O^T block cb: lane holds query q0 + lane % 32, channels 32 cb + 8 g + 4 h + 0..3
  const int ql = q0 + l32;
  if (ql >= nq) return;
  if (a.part) {
    // this half's unnormalised O, and (m, l), at the query's global token
    const int n_img = a.L.n_img;
    const long long row = (long long)(half * n_img + n) * tokens + tok0 + ql;
    float* po = a.part + row * D;
    if (h == 0) {
      float* pml = a.part + (long long)2 * n_img * tokens * D + row * 2;
      pml[0] = m_run;
      pml[1] = l_run;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4_t*>(po + 32 * cb + 8 * g + 4 * h) =
            f32x4_t{oacc[cb][4 * g], oacc[cb][4 * g + 1], oacc[cb][4 * g + 2], oacc[cb][4 * g + 3]};
    return;
  }
  const float inv = 1.f / l_run;
  const int r = ql / W, c = ql - (ql / W) * W;
  const BandLayout& L = a.L;
  unsigned short* out = reinterpret_cast<unsigned short*>(a.o) + L.off[b] +
                        (((long long)n * (L.rows[b] + 2) + r + 1) * L.W + c) * (long long)L.C;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk2;
      pk2.x = (unsigned)to_bf16(oacc[cb][4 * g] * inv) | ((unsigned)to_bf16(oacc[cb][4 * g + 1] * inv) << 16);
      pk2.y = (unsigned)to_bf16(oacc[cb][4 * g + 2] * inv) | ((unsigned)to_bf16(oacc[cb][4 * g + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(out + 32 * cb + 8 * g + 4 * h) = pk2;
    }
}

}  // namespace

hipError_t launch_attn_lds(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if (a.tokens % 8 != 0 || (long long)a.tokens * a.c * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  switch (a.c) {
    case 384: hipLaunchKernelGGL(attn_lds<384>, dim3(grid), dim3(256), 0, s, a); break;
    case 512: hipLaunchKernelGGL(attn_lds<512>, dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vaep
