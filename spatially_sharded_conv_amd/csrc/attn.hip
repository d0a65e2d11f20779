// AGKV attention: each band's queries against the global K/V.
//
// ChituDiffusion "VAEP" feature page, attention section, and "Static Layer-Wise VAE
// Decode", attention row: Q, K and V are computed per band; K and V of all bands are
// gathered once; each band runs softmax attention of its local Q against the global
// K/V and keeps its own output rows.  On one device the gather is the QKV projection
// writing K and V straight into global token-major buffers at the band's token offset;
// this kernel then reads them.  Single head, d = channels, scale 1/sqrt(d).
//
// bf16 path (flash style): a workgroup owns 64 queries of one band and image (16 per
// wave).  Per 64-key tile, K (64 x d) and V^T (d x 64) are staged in LDS; each wave
// computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (Q held in registers), runs the
// online softmax in fp32 (exp2 domain) on its 16 query columns, casts P to bf16 and
// accumulates O^T += V^T P^T in registers.  The P^T operand comes straight from the
// S^T accumulators: the 32-key K index of the PV product is permuted identically in
// both operands, which leaves the sum unchanged.
#include "vaep_internal.h"

namespace vaep {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

namespace {

__device__ __forceinline__ long long band_offset(const BandLayout& L, int b, int n, int r, int c) {
  return L.off[b] + (((long long)n * (L.rows[b] + 2) + r + 1) * L.W + c) * (long long)L.C;
}

__device__ __forceinline__ unsigned short f2bf(float v) {
  __hip_bfloat16 h = __float2bfloat16(v);
  return *reinterpret_cast<unsigned short*>(&h);
}

__device__ __forceinline__ int band_of(const AttnArgs& a, int blk) {
  int b = 0;
  while (b + 1 < a.L.nb && blk >= a.tile_start[b + 1]) ++b;
  return b;
}

constexpr int kQ = 64;    // queries per workgroup
constexpr int kKeys = 64; // keys per tile

template <int D>
__global__ void __launch_bounds__(256) flash_bf16(const AttnArgs a) {
  constexpr int LDK = D + 8;
  constexpr int LDV = kKeys + 8;
  constexpr int NKK = D / 32;
  constexpr int NDB = D / 16;
  __shared__ __attribute__((aligned(16))) unsigned short sK[kKeys * LDK];
  __shared__ __attribute__((aligned(16))) unsigned short sV[D * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = band_of(a, blockIdx.x);
  const int local = blockIdx.x - a.tile_start[b];
  const int W = a.L.W;
  const int nq = a.L.rows[b] * W;
  const int qt_img = (nq + kQ - 1) / kQ;
  const int n = local / qt_img;
  const int qt = local - n * qt_img;
  const int tokens = a.tokens;
  const long long tok0 = (long long)a.L.row0[b] * W;
  const int ql = qt * kQ + wave * 16 + (lane & 15);
  const bool qvalid = ql < nq;
  const long long qtok = tok0 + (qvalid ? ql : nq - 1);

  const unsigned short* Q = reinterpret_cast<const unsigned short*>(a.q) + ((long long)n * tokens + qtok) * D;
  bf16x8_t qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8_t*>(Q + kk * 32 + (lane >> 4) * 8);

  f32x4_t o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const unsigned short* Kg = reinterpret_cast<const unsigned short*>(a.k) + (long long)n * tokens * D;
  const unsigned short* Vg = reinterpret_cast<const unsigned short*>(a.vt) + (long long)n * D * tokens;
  const bool vec_ok = (tokens & 7) == 0;

  for (int k0 = 0; k0 < tokens; k0 += kKeys) {
    __syncthreads();
    for (int idx = tid; idx < kKeys * D / 8; idx += 256) {
      const int row = idx / (D / 8), col = (idx - row * (D / 8)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k0 + row < tokens) v = *reinterpret_cast<const uint4*>(Kg + (long long)(k0 + row) * D + col);
      *reinterpret_cast<uint4*>(&sK[row * LDK + col]) = v;
    }
    for (int idx = tid; idx < D * kKeys / 8; idx += 256) {
      const int row = idx / (kKeys / 8), col = (idx - row * (kKeys / 8)) * 8;
      const unsigned short* src = Vg + (long long)row * tokens + k0 + col;
      uint4 v;
      if (vec_ok && k0 + col + 8 <= tokens) {
        v = *reinterpret_cast<const uint4*>(src);
      } else {
        unsigned short t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (k0 + col + e < tokens) ? src[e] : 0;
        v.x = t[0] | ((unsigned)t[1] << 16);
        v.y = t[2] | ((unsigned)t[3] << 16);
        v.z = t[4] | ((unsigned)t[5] << 16);
        v.w = t[6] | ((unsigned)t[7] << 16);
      }
      *reinterpret_cast<uint4*>(&sV[row * LDV + col]) = v;
    }
    __syncthreads();

    // S^T[key][query] for the 4 key blocks of the tile
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
            &sK[(kb * 16 + (lane & 15)) * LDK + kk * 32 + (lane >> 4) * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], s[kb], 0, 0, 0);
      }
    }
    // online softmax over the tile (column = this lane's query)
    float mt = -1e30f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + kb * 16 + (lane >> 4) * 4 + j;
        const float v = key < tokens ? s[kb][j] * sl2 : -1e30f;
        s[kb][j] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2f(s[kb][j] - m_new);
        s[kb][j] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] *= alpha;

    bf16x8_t pf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pf[h][j] = (__bf16)s[2 * h][j];
        pf[h][4 + j] = (__bf16)s[2 * h + 1][j];
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const unsigned short* vr = &sV[(db * 16 + (lane & 15)) * LDV + h * 32 + (lane >> 4) * 4];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(&u);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[h], o[db], 0, 0, 0);
      }
    }
  }

  if (!qvalid) return;
  const float inv = 1.f / l_run;
  const int r = ql / W, c = ql - (ql / W) * W;
  unsigned short* out = reinterpret_cast<unsigned short*>(a.o) + band_offset(a.L, b, n, r, c);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = db * 16 + (lane >> 4) * 4;
    uint2 p;
    p.x = (unsigned)f2bf(o[db][0] * inv) | ((unsigned)f2bf(o[db][1] * inv) << 16);
    p.y = (unsigned)f2bf(o[db][2] * inv) | ((unsigned)f2bf(o[db][3] * inv) << 16);
    *reinterpret_cast<uint2*>(out + d) = p;
  }
}

// bf16 path, split-channel form (tokens a multiple of 8).  A workgroup owns 32 * QB queries;
// wave w owns channels [w*DS, (w+1)*DS) of both products (DS = d/4), so no K or V
// element is read by two waves and both go straight from global memory into registers
// (V of a tile loads while its S is formed, K of the next tile while its softmax and
// P V run).  Per 32-key tile:
//   1. each wave forms its partial S^T[key][q] = K[key][slice] Q^T[slice][q]
//      (v_mfma_f32_32x32x16_bf16) and stores it to LDS;
//   2. wave w sums the four partials for queries 16w .. 16w+15 (waves 0 and 1 only when
//      QB = 1), runs the online softmax in fp32 (exp2 domain) and stores P (bf16) and the
//      rescale factors;
//   3. each wave accumulates O^T[slice][q] += V^T[slice][key] P^T[key][q].
// The running max moves only when a row's tile max exceeds it by more than 8 (factor 256
// in P); otherwise P is formed against the old max (still exact: numerator and
// denominator use the same max), so the O rescale runs only on the rare tiles that move
// a max.
// Split keys (a.part set): workgroup 2i + s takes query block i against the s-th half of
// the key tiles and writes its unnormalised O, running max and sum (fp32) to a.part;
// attn_merge combines the halves.  Two workgroups then share each CU, one's barrier and
// softmax phases overlapping the other's products.  Runs d = 128 and 256 (QB = 2); d = 384
// and 512 run the LDS-staged kernel, which holds whole query rows per wave.
template <int DS, int QB>
__global__ void __launch_bounds__(256, (DS <= 96 || QB == 1) ? 2 : 1) attn_split(const AttnArgs a) {
  constexpr int D = 4 * DS;
  constexpr int KS = DS / 16;   // 16-channel steps of the S product
  constexpr int CB = DS / 32;   // 32-channel blocks of O^T
  constexpr int BK = 32;        // keys per tile
  constexpr int NQ = 32 * QB;   // queries per workgroup
  __shared__ __attribute__((aligned(16))) float sS[4][64][36];
  __shared__ __attribute__((aligned(16))) unsigned short sP[64][40];
  __shared__ float sAlpha[64];
  __shared__ float sL[64];
  __shared__ int sFlag[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool kSplit = DS <= 96;   // the key-split form exists for d <= 384
  const int nsplit = kSplit && a.part ? 2 : 1;
  const int blk = blockIdx.x / nsplit, half = blockIdx.x - blk * nsplit;
  const int b = band_of(a, blk);
  const int local = blk - a.tile_start[b];
  const int W = a.L.W;
  const int nq = a.L.rows[b] * W;
  const int qt_img = (nq + NQ - 1) / NQ;
  const int n = local / qt_img;
  const int q0 = (local - n * qt_img) * NQ;
  const int tokens = a.tokens;
  const long long tok0 = (long long)a.L.row0[b] * W;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool smw = QB == 2 || wave < 2;   // this wave runs the softmax of 16 queries
  const int c0 = wave * DS;

  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.q), 0, 0x7fffffff, 0x00020000);
  const unsigned short* kbase = reinterpret_cast<const unsigned short*>(a.k) + (long long)n * tokens * D;
  const unsigned short* vbase = reinterpret_cast<const unsigned short*>(a.vt) + (long long)n * D * tokens;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(kbase), 0, tokens * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(vbase), 0, tokens * D * 2, 0x00020000);

  // Q^T fragments (B operand of S^T): query q0 + 32*qb + lane%32, channels c0 + 16*ks + 8*hi
  bf16x8_t qf[QB][KS];
  {
    const unsigned short* qbase = reinterpret_cast<const unsigned short*>(a.q) + (long long)n * tokens * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int ql = q0 + 32 * qb + l32;
      if (ql > nq - 1) ql = nq - 1;
      const unsigned short* qr = qbase + (tok0 + ql) * D + c0 + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * ks);
    }
  }
  (void)qrs;

  // K fragments (A operand of S^T): key k0 + lane%32 (clamped), channels c0 + 16*ks + 8*hi.
  // V^T fragments (A operand of O^T): channel c0 + 32*cb + lane%32, keys k0 + 16*kk + 8*hi
  // (clamped to the last 8 keys; those keys get P = 0).
  bf16x8_t kf[KS], vf[CB][2];
#define VAEP_LOAD_K(KF, k0)                                                                    \
  {                                                                                            \
    int kr = (k0) + l32;                                                                       \
    if (kr > tokens - 1) kr = tokens - 1;                                                      \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                                          \
      KF[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(             \
          krs, (kr * D + c0 + 16 * ks + 8 * hi) * 2, 0, 0));                                   \
  }
#define VAEP_LOAD_V(VF, k0)                                                                    \
  {                                                                                            \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                         \
      int kc = (k0) + 16 * kk + 8 * hi;                                                        \
      if (kc > tokens - 8) kc = tokens - 8;                                                    \
      _Pragma("unroll") for (int cb = 0; cb < CB; ++cb)                                        \
        VF[cb][kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(       \
            vrs, ((c0 + 32 * cb + l32) * tokens + kc) * 2, 0, 0));                             \
    }                                                                                          \
  }

  f32x16_t oacc[CB][QB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[cb][qb][v] = 0.f;
  // softmax rows of this lane: query 16*wave + lane/4, keys 8*(lane%4) .. +8 of a tile
  const int qs = 16 * wave + (lane >> 2);
  const int kq = (lane & 3) * 8;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const int ntiles = (tokens + BK - 1) / BK;
  const int tper = (ntiles + nsplit - 1) / nsplit;
  const int tbeg = half * tper;
  const int tend = tbeg + tper < ntiles ? tbeg + tper : ntiles;

#define VAEP_TILE(KF, VF, k0)                                                                  \
  {                                                                                            \
    VAEP_LOAD_V(VF, k0);                                                                       \
    f32x16_t sacc[QB];                                                                         \
    _Pragma("unroll") for (int qb = 0; qb < QB; ++qb) {                                         \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) sacc[qb][v] = 0.f;                        \
      _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                                        \
        sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KF[ks], qf[qb][ks], sacc[qb], 0, 0, 0); \
    }                                                                                          \
    if ((k0) + BK < tokens) VAEP_LOAD_K(KF, (k0) + BK);                                        \
    /* partial S^T: lane holds query 32qb + lane%32, keys 8g + 4hi + 0..3 */                   \
    _Pragma("unroll") for (int qb = 0; qb < QB; ++qb)                                           \
      _Pragma("unroll") for (int g = 0; g < 4; ++g)                                            \
        *reinterpret_cast<f32x4_t*>(&sS[wave][32 * qb + l32][8 * g + 4 * hi]) =                \
            f32x4_t{sacc[qb][4 * g], sacc[qb][4 * g + 1], sacc[qb][4 * g + 2], sacc[qb][4 * g + 3]}; \
    __syncthreads();                                                                           \
    if (smw) {                                                                                 \
      float sv[8];                                                                             \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) sv[e] = 0.f;                               \
      _Pragma("unroll") for (int w = 0; w < 4; ++w) {                                          \
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(&sS[w][qs][kq]);                  \
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(&sS[w][qs][kq + 4]);              \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                        \
          sv[e] += x0[e];                                                                      \
          sv[4 + e] += x1[e];                                                                  \
        }                                                                                      \
      }                                                                                        \
      float rmax = -INFINITY;                                                                  \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                          \
        sv[e] = ((k0) + kq + e < tokens) ? sv[e] * sl2 : -INFINITY;                            \
        rmax = fmaxf(rmax, sv[e]);                                                             \
      }                                                                                        \
      rmax = fmaxf(rmax, __shfl_xor(rmax, 1));                                                 \
      rmax = fmaxf(rmax, __shfl_xor(rmax, 2));                                                 \
      const bool need = rmax > m_run + 8.f;                                                    \
      const float m_new = need ? rmax : m_run;                                                 \
      const float alpha = need ? exp2f(m_run - m_new) : 1.f;                                   \
      float rs = 0.f;                                                                          \
      unsigned pk[4];                                                                          \
      _Pragma("unroll") for (int e = 0; e < 8; e += 2) {                                       \
        const float p0 = exp2f(sv[e] - m_new), p1 = exp2f(sv[e + 1] - m_new);                  \
        rs += p0 + p1;                                                                         \
        pk[e / 2] = (unsigned)f2bf(p0) | ((unsigned)f2bf(p1) << 16);                           \
      }                                                                                        \
      rs += __shfl_xor(rs, 1);                                                                 \
      rs += __shfl_xor(rs, 2);                                                                 \
      l_run = l_run * alpha + rs;                                                              \
      m_run = m_new;                                                                           \
      *reinterpret_cast<uint4*>(&sP[qs][kq]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);         \
      if ((lane & 3) == 0) sAlpha[qs] = alpha;                                                 \
      const bool anyw = __builtin_amdgcn_ballot_w64(need) != 0;                                \
      if (lane == 0) sFlag[wave] = anyw ? 1 : 0;                                               \
    }                                                                                          \
    __syncthreads();                                                                           \
    if (sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3]) {                                           \
      _Pragma("unroll") for (int qb = 0; qb < QB; ++qb) {                                       \
        const float al = sAlpha[32 * qb + l32];                                                \
        _Pragma("unroll") for (int cb = 0; cb < CB; ++cb) oacc[cb][qb] *= al;                  \
      }                                                                                        \
    }                                                                                          \
    _Pragma("unroll") for (int qb = 0; qb < QB; ++qb)                                           \
      _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                       \
        const bf16x8_t pf = *reinterpret_cast<const bf16x8_t*>(&sP[32 * qb + l32][16 * kk + 8 * hi]); \
        _Pragma("unroll") for (int cb = 0; cb < CB; ++cb)                                      \
          oacc[cb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VF[cb][kk], pf, oacc[cb][qb], 0, 0, 0); \
      }                                                                                        \
  }

  if (!smw && lane == 0) sFlag[wave] = 0;   // ordered before its reads by the tile's first barrier
  VAEP_LOAD_K(kf, tbeg * BK);
  for (int t = tbeg; t < tend; ++t) VAEP_TILE(kf, vf, t * BK);
#undef VAEP_TILE
#undef VAEP_LOAD_K
#undef VAEP_LOAD_V

  if (kSplit && a.part) {
    // this half's unnormalised O^T, and (m, l) per query, at the query's global token
    float* po = a.part + ((long long)(half * a.L.n_img + n) * tokens + tok0) * D;
    float* pml = a.part + (long long)2 * a.L.n_img * tokens * D + ((long long)(half * a.L.n_img + n) * tokens + tok0) * 2;
    if (smw && (lane & 3) == 0 && q0 + qs < nq) {
      pml[(long long)(q0 + qs) * 2] = m_run;
      pml[(long long)(q0 + qs) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int ql = q0 + 32 * qb + l32;
      if (ql >= nq) continue;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4_t*>(po + (long long)ql * D + c0 + 32 * cb + 8 * g + 4 * hi) =
              f32x4_t{oacc[cb][qb][4 * g], oacc[cb][qb][4 * g + 1], oacc[cb][qb][4 * g + 2], oacc[cb][qb][4 * g + 3]};
    }
    return;
  }
  if (smw && (lane & 3) == 0) sL[qs] = l_run;
  __syncthreads();
  // O^T block (cb, qb): lane holds query 32qb + lane%32, channels c0 + 32cb + 8g + 4hi + 0..3
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int ql = q0 + 32 * qb + l32;
    if (ql >= nq) continue;
    const float inv = 1.f / sL[32 * qb + l32];
    const int r = ql / W, c = ql - (ql / W) * W;
    unsigned short* out = reinterpret_cast<unsigned short*>(a.o) + band_offset(a.L, b, n, r, c);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = c0 + 32 * cb + 8 * g + 4 * hi;
        uint2 pk;
        pk.x = (unsigned)f2bf(oacc[cb][qb][4 * g] * inv) | ((unsigned)f2bf(oacc[cb][qb][4 * g + 1] * inv) << 16);
        pk.y = (unsigned)f2bf(oacc[cb][qb][4 * g + 2] * inv) | ((unsigned)f2bf(oacc[cb][qb][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + d) = pk;
      }
  }
}

// Combine the two key halves of attn_split: per query, m = max(m0, m1),
// O = (O0 2^(m0-m) + O1 2^(m1-m)) / (l0 2^(m0-m) + l1 2^(m1-m)), stored as bf16 in the band
// layout.  One workgroup per 64-query block, 4 channels per thread and step.
__global__ void __launch_bounds__(256) attn_merge(const AttnArgs a) {
  const int b = band_of(a, blockIdx.x);
  const int local = blockIdx.x - a.tile_start[b];
  const int W = a.L.W, D = a.c, tokens = a.tokens;
  const int nq = a.L.rows[b] * W;
  const int qt_img = (nq + 63) / 64;
  const int n = local / qt_img;
  const int q0 = (local - n * qt_img) * 64;
  const long long tok0 = (long long)a.L.row0[b] * W;
  const int n_img = a.L.n_img;
  const float* ml = a.part + (long long)2 * n_img * tokens * D;
  const int per_q = D / 4;                          // float4 steps per query
  for (int e = threadIdx.x; e < 64 * per_q; e += 256) {
    const int qi = e / per_q, d = (e - qi * per_q) * 4;
    const int ql = q0 + qi;
    if (ql >= nq) break;
    const long long t0 = (long long)n * tokens + tok0 + ql;               // half 0
    const long long t1 = (long long)(n_img + n) * tokens + tok0 + ql;     // half 1
    const float m0 = ml[t0 * 2], l0 = ml[t0 * 2 + 1], m1 = ml[t1 * 2], l1 = ml[t1 * 2 + 1];
    const float m = fmaxf(m0, m1);
    const float f0 = l0 > 0.f ? exp2f(m0 - m) : 0.f, f1 = l1 > 0.f ? exp2f(m1 - m) : 0.f;
    const float inv = 1.f / (l0 * f0 + l1 * f1);
    const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(a.part + t0 * D + d);
    const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(a.part + t1 * D + d);
    const int r = ql / W, c = ql - (ql / W) * W;
    unsigned short* out = reinterpret_cast<unsigned short*>(a.o) + band_offset(a.L, b, n, r, c) + d;
    uint2 pk;
    pk.x = (unsigned)f2bf((o0[0] * f0 + o1[0] * f1) * inv) | ((unsigned)f2bf((o0[1] * f0 + o1[1] * f1) * inv) << 16);
    pk.y = (unsigned)f2bf((o0[2] * f0 + o1[2] * f1) * inv) | ((unsigned)f2bf((o0[3] * f0 + o1[3] * f1) * inv) << 16);
    *reinterpret_cast<uint2*>(out) = pk;
  }
}

// fp32 path: one wave per query, keys in sequence with an online softmax; lanes split d.
__global__ void __launch_bounds__(256) attn_f32(const AttnArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = band_of(a, blockIdx.x);
  const int local = blockIdx.x - a.tile_start[b];
  const int W = a.L.W;
  const int nq = a.L.rows[b] * W;
  const int qt_img = (nq + 3) / 4;
  const int n = local / qt_img;
  const int ql = (local - n * qt_img) * 4 + wave;
  if (ql >= nq) return;
  const int D = a.c, tokens = a.tokens;
  const long long qtok = (long long)a.L.row0[b] * W + ql;
  const float* Q = reinterpret_cast<const float*>(a.q) + ((long long)n * tokens + qtok) * D;
  const float* K = reinterpret_cast<const float*>(a.k) + (long long)n * tokens * D;
  const float* Vt = reinterpret_cast<const float*>(a.vt) + (long long)n * D * tokens;
  constexpr int kMaxPer = 16;   // d <= 1024
  float q[kMaxPer], o[kMaxPer];
  const int per = (D + 63) / 64;
  for (int i = 0; i < kMaxPer; ++i) {
    const int d = lane + 64 * i;
    q[i] = (i < per && d < D) ? Q[d] : 0.f;
    o[i] = 0.f;
  }
  float m = -1e30f, l = 0.f;
  for (int key = 0; key < tokens; ++key) {
    float part = 0.f;
    for (int i = 0; i < per; ++i) {
      const int d = lane + 64 * i;
      if (d < D) part += q[i] * K[(long long)key * D + d];
    }
    for (int w = 32; w > 0; w >>= 1) part += __shfl_xor(part, w);
    const float sc = part * a.scale;
    const float mn = fmaxf(m, sc);
    const float al = __expf(m - mn);
    const float p = __expf(sc - mn);
    l = l * al + p;
    for (int i = 0; i < per; ++i) {
      const int d = lane + 64 * i;
      if (d < D) o[i] = o[i] * al + p * Vt[(long long)d * tokens + key];
    }
    m = mn;
  }
  const int r = ql / W, c = ql - (ql / W) * W;
  float* out = reinterpret_cast<float*>(a.o) + band_offset(a.L, b, n, r, c);
  for (int i = 0; i < per; ++i) {
    const int d = lane + 64 * i;
    if (d < D) out[d] = o[i] / l;
  }
}

}  // namespace

hipError_t launch_attention(AttnArgs& a, int dtype, hipStream_t s) {
  // bf16 with tokens % 8 == 0 (16-byte V^T rows): the LDS-staged kernel (attn_lds.hip) at
  // d = 384 and 512, the split-channel kernel at d = 128 and 256; flash_bf16 otherwise.
  const bool split = dtype != VAEP_DTYPE_F32 && a.tokens % 8 == 0 &&
                     (long long)a.tokens * a.c * 2 < (1LL << 31);
  auto block_starts = [&a](int per) {
    int t = 0;
    for (int b = 0; b < a.L.nb; ++b) {
      a.tile_start[b] = t;
      t += a.L.n_img * ((a.L.rows[b] * a.L.W + per - 1) / per);
    }
    a.tile_start[a.L.nb] = t;
    a.tiles_total = t;
    return t;
  };
  if (split && (a.c == 384 || a.c == 512)) {
    // 128 queries per workgroup.  Keys split in two (a.part: the caller's scratch of
    // attn_part_floats) when the whole image's 128-query blocks fill at most half of the
    // CUs (256) -- decided on the whole image, so every band table computes the same sums.
    const long long q128 = (long long)a.L.n_img * (((long long)a.L.H * a.L.W + 127) / 128);
    if (q128 > 128) a.part = nullptr;
    const int t = block_starts(128);
    if (t == 0) return hipSuccess;
    hipError_t e = launch_attn_lds(a, (unsigned)t * (a.part ? 2u : 1u), s);
    if (e != hipSuccess || !a.part) return e;
    hipLaunchKernelGGL(attn_merge, dim3(block_starts(64)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int t = block_starts(dtype == VAEP_DTYPE_F32 ? 4 : kQ);
  if (t == 0) return hipSuccess;
  if (dtype == VAEP_DTYPE_F32) {
    if (a.c > 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_f32, dim3(t), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (split && (a.c == 128 || a.c == 256)) {
    // keys in two halves when the 64-query blocks alone would not give every CU two
    // workgroups -- decided on the whole image
    const long long q64 = (long long)a.L.n_img * (((long long)a.L.H * a.L.W + 63) / 64);
    if (q64 >= 512) a.part = nullptr;
    const unsigned g = (unsigned)t * (a.part ? 2u : 1u);
    if (a.c == 128)
      hipLaunchKernelGGL((attn_split<32, 2>), dim3(g), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attn_split<64, 2>), dim3(g), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.part) return e;
    hipLaunchKernelGGL(attn_merge, dim3(t), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  switch (a.c) {
    case 128: hipLaunchKernelGGL(flash_bf16<128>, dim3(t), dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(flash_bf16<256>, dim3(t), dim3(256), 0, s, a); break;
    case 384: hipLaunchKernelGGL(flash_bf16<384>, dim3(t), dim3(256), 0, s, a); break;
    case 512: hipLaunchKernelGGL(flash_bf16<512>, dim3(t), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vaep
