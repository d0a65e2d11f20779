// GroupNorm with band-merged statistics, channel RMSNorm, and the moment merge.
//
// GroupNorm (ChituDiffusion "VAEP" feature page, GroupNorm section; "Static Layer-Wise
// VAE Decode", GroupNorm row and the formula below the table): every band computes
// FP32 central moments per (sample, group) of its own rows; the bands' moments are
// merged with actual-element-count weights,
//     mean = sum_i w_i mean_i,  var = sum_i w_i (var_i + (mean_i - mean)^2),
// and every band normalises with the merged statistics, then the channel affine and
// (in the decoder's norm -> SiLU pairs) SiLU.
//
// Local moments are formed per tile of a fixed tiling of the image (slabs of rows that
// no band boundary can split, cut into pixel chunks), in fp64 and two-pass.  The merged
// statistics are the count-weighted merge of all tiles in global row order, and each
// band's moments are the same merge over the tiles it owns.  Any band table therefore
// yields bit-identical statistics: a decoded image does not depend on its partition.
//
// Data movement: the stats pass reads the band's rows once (16-byte loads, each
// workgroup a contiguous slab of one band and image), two-pass in registers per tile;
// the apply pass streams the rows again and writes the result plus the boundary rows
// into the neighbours' halo slots.  Channel RMSNorm is local to a pixel and needs no
// merge.
#include <type_traits>

#include "vaep_internal.h"
#include "norm_act.h"

namespace vaep {
namespace {

constexpr int kThreads = 256;
constexpr int V = 4;               // channels per 16-byte load of the fp32 input

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Inputs larger than the last-level cache are read with nontemporal loads (NT): each
// element is read once per pass, and streaming loads keep the HBM read rate near ~90 %
// of peak instead of ~80 %.  Smaller inputs were just written by the producing conv and
// are still partly cached; there plain loads are faster.
constexpr long long kStreamBytes = 192ll << 20;

template <bool NT, typename T>
__device__ __forceinline__ T ld_x(const T* p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__device__ __forceinline__ void load4(const float* p, float* v) {
  const f32x4_t q = ld_x<NT>(reinterpret_cast<const f32x4_t*>(p));
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ float bf_at(unsigned w, int hi) { return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16)); }

// Input element access.  `pix` is the element offset of a pixel's channel 0 in the
// C-channel layout.  XS: the buffer holds bf16 hi / lo halves of the fp32 values (2C
// channels per pixel, written by a split-output conv); x = hi + lo is exact in fp32.
template <bool XS, bool NT>
__device__ __forceinline__ void loadx4(const void* x, long long pix, int C, int ch, float* v) {
  if (!XS) {
    load4<NT>(reinterpret_cast<const float*>(x) + pix + ch, v);
  } else {
    const unsigned short* s = reinterpret_cast<const unsigned short*>(x) + 2 * pix + ch;
    const u32x2_t h = ld_x<NT>(reinterpret_cast<const u32x2_t*>(s));
    const u32x2_t l = ld_x<NT>(reinterpret_cast<const u32x2_t*>(s + C));
    v[0] = bf_at(h.x, 0) + bf_at(l.x, 0);
    v[1] = bf_at(h.x, 1) + bf_at(l.x, 1);
    v[2] = bf_at(h.y, 0) + bf_at(l.y, 0);
    v[3] = bf_at(h.y, 1) + bf_at(l.y, 1);
  }
}
template <bool XS>
__device__ __forceinline__ float loadx1(const void* x, long long pix, int C, int ch) {
  if (!XS) return reinterpret_cast<const float*>(x)[pix + ch];
  const unsigned short* s = reinterpret_cast<const unsigned short*>(x) + 2 * pix + ch;
  return __uint_as_float((unsigned)s[0] << 16) + __uint_as_float((unsigned)s[C] << 16);
}

template <typename T> struct Out;
template <> struct Out<float> {
  __device__ static void store4(float* p, const float* v) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
  }
};
template <> struct Out<bf16> {
  __device__ static unsigned short rne(float f) {
    __hip_bfloat16 h = __float2bfloat16(f);
    return *reinterpret_cast<unsigned short*>(&h);
  }
  __device__ static void store4(bf16* p, const float* v) {
    u32x2_t q;
    q.x = rne(v[0]) | ((unsigned)rne(v[1]) << 16);
    q.y = rne(v[2]) | ((unsigned)rne(v[3]) << 16);
    *reinterpret_cast<u32x2_t*>(p) = q;
  }
};

__device__ __forceinline__ long long row_offset(const BandLayout& L, int b, int n, int r) {
  return L.off[b] + ((long long)n * (L.rows[b] + 2) + r + 1) * (long long)L.W * L.C;
}

__device__ __forceinline__ int band_of_block(const int* start, int nb, int blk) {
  int b = 0;
  while (b + 1 < nb && blk >= start[b + 1]) ++b;
  return b;
}

// Pass 1: central moments of one tile (a pixel chunk of one slab of one image):
// partials[tile][g] = (mean, M2) of group g.  Each thread streams its channel slot over
// the tile's pixels accumulating sums shifted by the tile's first pixel (fp32 over 4
// pixels, then fp64); the block then reduces per group in fp64.  The tiling is fixed,
// so the result does not depend on the band table.
template <bool XS, bool NT>
__global__ void __launch_bounds__(kThreads) gn_stats(const NormArgs a) {
  __shared__ double r1[kThreads * V];
  __shared__ double r2[kThreads * V];
  __shared__ float shift[1024];
  const BandLayout& L = a.L;
  const int C = L.C, S = C / V, PL = kThreads / S;
  const int G = a.groups, cpg = C / G;
  const int blk = blockIdx.x;
  const int per_img = a.slabs * a.chunks;
  const int n = blk / per_img;
  const int slab = (blk - n * per_img) / a.chunks;
  const int chunk = blk - n * per_img - slab * a.chunks;
  const int g0 = slab * a.slab_rows;                    // first global row of the slab
  int b = 0;
  while (b + 1 < L.nb && g0 >= L.row0[b + 1]) ++b;
  const long long slab_pix = (long long)a.slab_rows * L.W;
  const long long p0 = (long long)chunk * a.chunk_pix;
  long long tp = slab_pix - p0;
  if (tp > a.chunk_pix) tp = a.chunk_pix;
  const int tid = threadIdx.x;
  const int slot = tid % S, pl = tid / S;
  const bool active = pl < PL;
  const long long tile_x = row_offset(L, b, n, g0 - L.row0[b]) + p0 * C;   // pixel offset
  // per-channel shift: the tile's first pixel
  for (int c = tid; c < C; c += kThreads) shift[c] = loadx1<XS>(a.x, tile_x, C, c);
  __syncthreads();
  float k[V];
#pragma unroll
  for (int e = 0; e < V; ++e) k[e] = shift[slot * V + e];
  double s1[V], s2[V];
#pragma unroll
  for (int e = 0; e < V; ++e) s1[e] = s2[e] = 0.0;
  if (active) {
    for (long long p = pl; p < tp; p += 4LL * PL) {
      float f1[V], f2[V];
#pragma unroll
      for (int e = 0; e < V; ++e) f1[e] = f2[e] = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const long long q = p + (long long)u * PL;
        if (q < tp) {
          float x[V];
          loadx4<XS, NT>(a.x, tile_x + q * C, C, slot * V, x);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const float d = x[e] - k[e];
            f1[e] += d;
            f2[e] = fmaf(d, d, f2[e]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        s1[e] += (double)f1[e];
        s2[e] += (double)f2[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) {
    r1[tid * V + e] = active ? s1[e] : 0.0;
    r2[tid * V + e] = active ? s2[e] : 0.0;
  }
  __syncthreads();
  // per channel c: sum over the PL pixel lanes (slot c / V, element c % V)
  const double cnt = (double)tp;
  if (tid < G) {
    const int gc = tid * cpg;
    double sum = 0.0;          // sum over the group of x
    for (int j = 0; j < cpg; ++j) {
      const int c = gc + j, sl = c / V, e = c % V;
      double a1 = 0.0;
      for (int q = 0; q < PL; ++q) a1 += r1[(q * S + sl) * V + e];
      sum += cnt * (double)shift[c] + a1;
    }
    const double mean = sum / (cnt * cpg);
    double m2 = 0.0;           // sum over the group of (x - mean)^2
    for (int j = 0; j < cpg; ++j) {
      const int c = gc + j, sl = c / V, e = c % V;
      double a1 = 0.0, a2 = 0.0;
      for (int q = 0; q < PL; ++q) {
        a1 += r1[(q * S + sl) * V + e];
        a2 += r2[(q * S + sl) * V + e];
      }
      // sum (x - mean)^2 = sum (d - dm)^2 with d = x - k_c, dm = mean - k_c
      const double dm = mean - (double)shift[c];
      m2 += a2 - 2.0 * dm * a1 + cnt * dm * dm;
    }
    // group-major records: [image][group][tile of the image]
    double* out = a.partials + (((long long)n * G + tid) * per_img + (blk - n * per_img)) * 2;
    out[0] = mean;
    out[1] = m2 > 0.0 ? m2 : 0.0;
  }
}

// Sum of one fp64 value per thread of the workgroup, in a fixed order: a butterfly within
// each wave (every lane ends with the same sum), then the wave sums in wave order.  sh:
// kThreads / 64 doubles of LDS.
__device__ __forceinline__ double block_sum(double v, double* sh) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) r += sh[w];
  __syncthreads();
  return r;
}

// Count-weighted merge (feature page, GroupNorm section) of the tiles [t0, t1) of
// image n, group g: mean = sum w_t mean_t, var = sum w_t (var_t + (mean_t - mean)^2),
// w_t = n_t / sum n_t.  Fixed thread striding and a fixed reduction order: the result
// depends only on the tiles.  Every thread returns (count, mean, var).
__device__ void merge_tiles(const NormArgs& a, int n, int g, int t0, int t1, double* sh,
                            double* cnt, double* mean, double* var) {
  const int tid = threadIdx.x;
  const int G = a.groups, cpg = a.L.C / G;
  const long long slab_pix = (long long)a.slab_rows * a.L.W;
  // group g's records of image n, contiguous (group-major layout)
  const double* P = a.partials + ((long long)n * G + g) * ((long long)a.slabs * a.chunks) * 2;
  auto tile_n = [&](int t) {
    const int chunk = t % a.chunks;
    long long tp = slab_pix - (long long)chunk * a.chunk_pix;
    if (tp > a.chunk_pix) tp = a.chunk_pix;
    return (double)(tp * cpg);
  };
  // the tiles cover whole slabs: the element count is exact
  const double total = (double)((t1 - t0) / a.chunks) * (double)slab_pix * cpg;
  // Each thread takes tiles t0 + tid, t0 + tid + kThreads, ... in that order; the loads of a
  // batch of kBatch tiles are issued together (one memory latency per batch, not per tile),
  // the sums still run tile by tile.
  //
  // When the chunks divide the slab (the records of every conv epilogue) all tiles hold the
  // same count nt, so nt / total is one double formed once instead of per tile; when nt is
  // a power of two, M2_t / nt is exactly M2_t * (1 / nt).  Either way every term is the
  // same double as the per-tile form, and the merge result does not change.
  constexpr int kBatch = 8;
  const bool uniform = slab_pix % a.chunk_pix == 0;
  const long long nt_i = (long long)a.chunk_pix * cpg;
  const double nt_u = (double)nt_i, w_u = nt_u / total, inv_u = 1.0 / nt_u;
  const bool pow2 = (nt_i & (nt_i - 1)) == 0;
  auto pass1 = [&](auto U) {
    constexpr bool kU = decltype(U)::value;
    double s = 0.0;
    for (int t_b = t0 + tid; t_b < t1; t_b += kBatch * kThreads) {
      double mt[kBatch];
#pragma unroll
      for (int r = 0; r < kBatch; ++r) {
        const int t = t_b + r * kThreads;
        mt[r] = t < t1 ? P[(long long)t * 2] : 0.0;
      }
#pragma unroll
      for (int r = 0; r < kBatch; ++r) {
        const int t = t_b + r * kThreads;
        if (t < t1) s += (kU ? w_u : tile_n(t) / total) * mt[r];
      }
    }
    return s;
  };
  const double m = block_sum(uniform ? pass1(std::true_type{}) : pass1(std::false_type{}), sh);
  auto pass2 = [&](auto U, auto P2) {
    constexpr bool kU = decltype(U)::value, kP2 = decltype(P2)::value;
    double s = 0.0;
    for (int t_b = t0 + tid; t_b < t1; t_b += kBatch * kThreads) {
      double mt[kBatch], vt[kBatch];
#pragma unroll
      for (int r = 0; r < kBatch; ++r) {
        const int t = t_b + r * kThreads;
        const double* pr = P + (long long)(t < t1 ? t : t0) * 2;
        mt[r] = pr[0];
        vt[r] = pr[1];
      }
#pragma unroll
      for (int r = 0; r < kBatch; ++r) {
        const int t = t_b + r * kThreads;
        if (t < t1) {
          const double nt = kU ? nt_u : tile_n(t);
          const double d = mt[r] - m;
          const double var_t = kP2 ? vt[r] * inv_u : vt[r] / nt;
          s += (kU ? w_u : nt / total) * (var_t + d * d);
        }
      }
    }
    return s;
  };
  const double s2 = !uniform ? pass2(std::false_type{}, std::false_type{})
                    : pow2   ? pass2(std::true_type{}, std::true_type{})
                             : pass2(std::true_type{}, std::false_type{});
  const double v = block_sum(s2, sh);
  *cnt = total;
  *mean = m;
  *var = v;
}

// Pass 2: one workgroup per (image n, group g, k): k < nb reports band k's moments (its
// own tiles merged; only when a.want_band_moments); k = nb merges all tiles of the image into the statistics the apply
// uses, rounded to fp32 once, and writes the per-channel scale/shift of the apply.  Each
// result is a fixed function of the tiles, whatever workgroup computes it.
__global__ void __launch_bounds__(kThreads) gn_merge(const NormArgs a, float* coef) {
  __shared__ double sh[kThreads];
  __shared__ float fin[2];
  const BandLayout& L = a.L;
  const int G = a.groups, C = L.C, cpg = C / G;
  const int kparts = a.want_band_moments ? L.nb + 1 : 1;
  const int k = a.want_band_moments ? blockIdx.x % kparts : L.nb;
  const int ng = blockIdx.x / kparts;
  const int n = ng / G, g = ng - (ng / G) * G;
  const int tid = threadIdx.x;
  const int s_idx = n * G + g, ns = L.n_img * G;
  if (k < L.nb) {
    double cb, mb, vb;
    const int t0 = (L.row0[k] / a.slab_rows) * a.chunks;
    const int t1 = ((L.row0[k] + L.rows[k]) / a.slab_rows) * a.chunks;
    merge_tiles(a, n, g, t0, t1, sh, &cb, &mb, &vb);
    if (tid == 0) {
      a.band_moments[(0 * L.nb + k) * (long long)ns + s_idx] = (float)cb;
      a.band_moments[(1 * L.nb + k) * (long long)ns + s_idx] = (float)mb;
      a.band_moments[(2 * L.nb + k) * (long long)ns + s_idx] = (float)vb;
    }
    return;
  }
  double cnt, mean, var;
  merge_tiles(a, n, g, 0, a.slabs * a.chunks, sh, &cnt, &mean, &var);
  if (tid == 0) {
    const float mean_f = (float)mean, var_f = (float)var;
    const float rstd = rsqrtf(var_f + a.eps);
    a.stats[s_idx] = mean_f;
    a.stats[ns + s_idx] = rstd;
    if (a.merged_out) {
      a.merged_out[s_idx] = mean_f;
      a.merged_out[ns + s_idx] = var_f;
    }
    fin[0] = mean_f;
    fin[1] = rstd;
  }
  __syncthreads();
  const float mf = fin[0], rstd = fin[1];
  for (int j = tid; j < cpg; j += kThreads) {
    const int ch = g * cpg + j;
    const float sc = rstd * a.gamma[ch];
    coef[((long long)n * C + ch) * 2] = sc;
    coef[((long long)n * C + ch) * 2 + 1] = a.beta[ch] - mf * sc;
  }
}

// Pass 3: y = act(x * scale_c + shift_c) over every owned row; boundary rows are also
// written into the neighbours' halo slots.  Workgroup = a run of a.apply_pix pixels of
// one (band, image); thread = fixed channel slot, pixels strided by the pixel lanes.
template <typename TO, bool XS, bool NT>
__global__ void __launch_bounds__(kThreads) gn_apply(const NormArgs a, const float* coef) {
  const BandLayout& L = a.L;
  const int C = L.C, S = C / V, PL = kThreads / S;
  int b = 0;
  while (b + 1 < L.nb && (long long)blockIdx.x >= a.item_start[b + 1]) ++b;
  const long long local = blockIdx.x - a.item_start[b];
  const int run = a.apply_pix;
  const long long runs = ((long long)L.rows[b] * L.W + run - 1) / run;
  const int n = (int)(local / runs);
  const long long p0 = (local - n * runs) * run;
  const long long npix = (long long)L.rows[b] * L.W;
  const int tid = threadIdx.x;
  const int slot = tid % S, pl = tid / S;
  if (pl >= PL) return;
  const long long xrow = row_offset(L, b, n, 0);
  TO* Y = reinterpret_cast<TO*>(a.y);
  const long long ybase = row_offset(L, b, n, 0) + slot * V;
  float sc[V], sh[V];
  const float* cf = coef + ((long long)n * C + slot * V) * 2;
#pragma unroll
  for (int e = 0; e < V; ++e) {
    sc[e] = cf[2 * e];
    sh[e] = cf[2 * e + 1];
  }
  const long long row_up = b > 0 ? row_offset(L, b - 1, n, L.rows[b - 1]) + slot * V : 0;
  const long long row_dn = b + 1 < L.nb ? row_offset(L, b + 1, n, -1) + slot * V : 0;
  const long long last_row_start = (long long)(L.rows[b] - 1) * L.W;
  for (long long p = p0 + pl; p < p0 + run && p < npix; p += PL) {
    float x[V];
    loadx4<XS, NT>(a.x, xrow + p * C, C, slot * V, x);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      x[e] = gn_affine_act(x[e], sc[e], sh[e], a.act);
    }
    Out<TO>::store4(Y + ybase + p * C, x);
    if (p < L.W && b > 0) Out<TO>::store4(Y + row_up + p * C, x);
    if (p >= last_row_start && b + 1 < L.nb) Out<TO>::store4(Y + row_dn + (p - last_row_start) * C, x);
  }
}

// Channel RMSNorm: y_c = gamma_c x_c / sqrt(mean_c x^2 + eps) (+SiLU), per pixel.
template <typename TO, bool XS, bool NT>
__global__ void __launch_bounds__(kThreads) rms_apply(const NormArgs a) {
  __shared__ float part[kThreads];
  __shared__ float rs[kThreads];
  const BandLayout& L = a.L;
  const int C = L.C, S = C / V, PX = kThreads / S;
  const int tid = threadIdx.x;
  const int slot = tid % S, px = tid / S;
  const long long ptotal = a.item_start[L.nb];
  TO* Y = reinterpret_cast<TO*>(a.y);
  for (long long base = (long long)blockIdx.x * PX; base < ptotal; base += (long long)gridDim.x * PX) {
    const long long gp = base + px;
    const bool act = px < PX && gp < ptotal;
    float x[V];
    long long off = 0;
    int b = 0, n = 0, r = 0, c = 0;
    float ss = 0.f;
    if (act) {
      while (b + 1 < L.nb && gp >= a.item_start[b + 1]) ++b;
      const long long p = gp - a.item_start[b];
      const long long per_img = (long long)L.rows[b] * L.W;
      n = (int)(p / per_img);
      const long long rem = p - n * per_img;
      r = (int)(rem / L.W);
      c = (int)(rem - (long long)r * L.W);
      off = row_offset(L, b, n, r) + (long long)c * C + slot * V;
      loadx4<XS, NT>(a.x, off - slot * V, C, slot * V, x);
#pragma unroll
      for (int e = 0; e < V; ++e) ss += x[e] * x[e];
    }
    part[tid] = ss;
    __syncthreads();
    if (act && slot == 0) {
      float t = 0.f;
      for (int j = 0; j < S; ++j) t += part[px * S + j];
      rs[px] = rsqrtf(t / (float)C + a.eps);
    }
    __syncthreads();
    if (act) {
      const float rr = rs[px];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float y = x[e] * rr * a.gamma[slot * V + e];
        x[e] = a.act ? silu(y) : y;
      }
      Out<TO>::store4(Y + off, x);
      if (r == 0 && b > 0)
        Out<TO>::store4(Y + row_offset(L, b - 1, n, L.rows[b - 1]) + (long long)c * C + slot * V, x);
      if (r == L.rows[b] - 1 && b + 1 < L.nb)
        Out<TO>::store4(Y + row_offset(L, b + 1, n, -1) + (long long)c * C + slot * V, x);
    }
    __syncthreads();
  }
}

// Channel RMSNorm, one wave per run of P pixels: the run's P*C fp32 values are K float4
// per lane, contiguous (P*C = 256*K), so every load and store of a wave covers one
// contiguous span.  The per-pixel sums of squares are combined through the wave's own
// LDS rows (no workgroup barrier), then every lane scales its values by the rstd of
// their pixel.  A run never crosses an image or band (the last run of one is partial).
// item_start holds the first run of each band.
template <typename TO, bool XS, bool NT, int K>
__global__ void __launch_bounds__(kThreads) rms_wave(const NormArgs a, int runs_total) {
  constexpr int P4 = 64 * K;                 // float4 slots of one run
  __shared__ float part[kThreads / 64][P4];
  __shared__ float rsq[kThreads / 64][64];
  const BandLayout& L = a.L;
  const int C = L.C, Q = C / V;              // float4 slots of one pixel
  const int P = P4 / Q;                      // pixels of one run
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  TO* Y = reinterpret_cast<TO*>(a.y);
  const int stride = gridDim.x * (kThreads / 64);
  // a lane's slots sit at the same (pixel, channel) of every run
  int spix[K], sch[K];
  float gam[K][V];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int slot = j * 64 + lane;
    spix[j] = slot / Q;
    sch[j] = (slot - spix[j] * Q) * V;
#pragma unroll
    for (int e = 0; e < V; ++e) gam[j][e] = a.gamma[sch[j] + e];
  }
  for (int u = blockIdx.x * (kThreads / 64) + wv; u < runs_total; u += stride) {
    int b = 0;
    while (b + 1 < L.nb && u >= (int)a.item_start[b + 1]) ++b;
    const int lu = u - (int)a.item_start[b];
    const int img_pix = L.rows[b] * L.W;
    const int runs_img = (img_pix + P - 1) / P;
    const int n = lu / runs_img;
    const int p0 = (lu - n * runs_img) * P;
    const int np = img_pix - p0 < P ? img_pix - p0 : P;
    const long long base = row_offset(L, b, n, 0);
    float x[K][V];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (spix[j] < np) {
        loadx4<XS, NT>(a.x, base + (long long)(p0 + spix[j]) * C, C, sch[j], x[j]);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) x[j][e] = 0.f;
      }
      float q = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) q = fmaf(x[j][e], x[j][e], q);
      part[wv][j * 64 + lane] = q;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < P) {
      float t = 0.f;
      for (int i = 0; i < Q; ++i) t += part[wv][lane * Q + i];
      rsq[wv][lane] = rsqrtf(t / (float)C + a.eps);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int last_row = (L.rows[b] - 1) * L.W;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (spix[j] >= np) continue;
      const float rr = rsq[wv][spix[j]];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float y = x[j][e] * rr * gam[j][e];
        x[j][e] = a.act ? silu(y) : y;
      }
      const int p = p0 + spix[j];
      Out<TO>::store4(Y + base + (long long)p * C + sch[j], x[j]);
      if (p < L.W && b > 0)
        Out<TO>::store4(Y + row_offset(L, b - 1, n, L.rows[b - 1]) + (long long)p * C + sch[j], x[j]);
      if (p >= last_row && b + 1 < L.nb)
        Out<TO>::store4(Y + row_offset(L, b + 1, n, -1) + (long long)(p - last_row) * C + sch[j], x[j]);
    }
    // the next run reuses part / rsq
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Standalone merge of caller-supplied shard moments (one thread per statistic).
__global__ void moment_merge(int n_shards, int n_stats, const float* mean, const float* var,
                             const int64_t* counts, float* mean_out, float* var_out) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_stats) return;
  double total = 0.0;
  for (int i = 0; i < n_shards; ++i) total += (double)counts[(long long)i * n_stats + s];
  if (total <= 0.0) {
    mean_out[s] = 0.f;
    var_out[s] = 0.f;
    return;
  }
  float m = 0.f;
  for (int i = 0; i < n_shards; ++i) {
    const float w = (float)((double)counts[(long long)i * n_stats + s] / total);
    m += w * mean[(long long)i * n_stats + s];
  }
  float v = 0.f;
  for (int i = 0; i < n_shards; ++i) {
    const float w = (float)((double)counts[(long long)i * n_stats + s] / total);
    const float d = mean[(long long)i * n_stats + s] - m;
    v += w * (var[(long long)i * n_stats + s] + d * d);
  }
  mean_out[s] = m;
  var_out[s] = v;
}

}  // namespace


// Stats tiling of a layout: slabs of a.slab_rows rows (set by the caller), cut into
// chunks of chunk_pixels() pixels: about 2048 tiles per layer, each between 64 KiB and
// 512 KiB of fp32.  A function of the layer's shape only, never of the band table.
static int chunk_pixels(const BandLayout& L) {
  const long long bytes = (long long)L.n_img * L.H * L.W * L.C * 4;
  long long tb = bytes / 2048;
  if (tb < (64 << 10)) tb = 64 << 10;
  if (tb > (512 << 10)) tb = 512 << 10;
  const long long pix = tb / (4LL * L.C);
  return (int)(pix < 1 ? 1 : pix);
}
// Apply run length: enough workgroups to fill the GPU on small layers.  Tensors below the
// streaming threshold (cache-resident, latency-bound) get runs of four pixels per thread
// lane, so that each thread's loop is four loads long.
static int apply_pixels(const BandLayout& L) {
  const long long pix = (long long)L.n_img * L.H * L.W;
  if (pix * L.C * 4 < kStreamBytes) {
    const int lanes = kThreads / (L.C / V);   // pixel lanes of a workgroup
    return 4 * (lanes < 1 ? 1 : lanes);
  }
  long long run = pix / 2048;
  if (run < 32) run = 32;
  if (run > 256) run = 256;
  return (int)run;
}

static bool plan_stats(NormArgs& a) {
  const BandLayout& L = a.L;
  if (a.pre_chunk > 0) {       // records of the producing conv: one-row slabs, whole chunks
    if (L.W % a.pre_chunk != 0) return false;
    a.slab_rows = 1;
  }
  if (a.slab_rows < 1 || L.H % a.slab_rows != 0) return false;
  for (int b = 0; b < L.nb; ++b)
    if (L.row0[b] % a.slab_rows != 0 || L.rows[b] % a.slab_rows != 0) return false;
  a.slabs = L.H / a.slab_rows;
  a.chunk_pix = a.pre_chunk > 0 ? a.pre_chunk : chunk_pixels(L);
  const long long slab_pix = (long long)a.slab_rows * L.W;
  a.chunks = (int)((slab_pix + a.chunk_pix - 1) / a.chunk_pix);
  return true;
}

size_t gn_partials_floats(const BandLayout& L, int groups, int slab_rows, int chunk) {
  // (in floats) fp64 partials, per-channel coefficients, per-band moments, merged stats
  const int pix = chunk > 0 ? chunk : chunk_pixels(L);
  if (chunk > 0) slab_rows = 1;
  const long long slab_pix = (long long)slab_rows * L.W;
  const long long tiles = (long long)L.n_img * (L.H / slab_rows) * ((slab_pix + pix - 1) / pix);
  return (size_t)(tiles * groups * 4 + 2LL * L.n_img * L.C + 3LL * L.nb * L.n_img * groups +
                  2LL * L.n_img * groups);
}

hipError_t launch_groupnorm(NormArgs& a, int dtype, hipStream_t s) {
  const BandLayout& L = a.L;
  if (L.C % V != 0 || L.C / V > kThreads || L.C % a.groups != 0 || a.groups > 1024)
    return hipErrorInvalidValue;
  if (!plan_stats(a)) return hipErrorInvalidValue;
  const long long blocks_ll = (long long)L.n_img * a.slabs * a.chunks;
  if (blocks_ll > 0x7fffffffLL) return hipErrorInvalidValue;
  const int blocks = (int)blocks_ll;
  // Scratch carve-up inside a.partials (sized by gn_partials_floats).
  float* coef = a.coef_out ? a.coef_out : reinterpret_cast<float*>(a.partials + (size_t)blocks * a.groups * 2);
  a.band_moments = coef + 2LL * L.n_img * L.C;
  a.stats = a.band_moments + 3LL * L.nb * L.n_img * a.groups;
  if (blocks == 0) return hipSuccess;
  // the input's size: fp32, or bf16 hi / lo halves (the same bytes)
  const bool nt = (long long)L.n_img * L.H * L.W * L.C * 4 >= kStreamBytes;
  if (a.pre_chunk <= 0) {   // else the producing conv already wrote the tile records
    if (a.x_split && nt)
      hipLaunchKernelGGL((gn_stats<true, true>), dim3(blocks), dim3(kThreads), 0, s, a);
    else if (a.x_split)
      hipLaunchKernelGGL((gn_stats<true, false>), dim3(blocks), dim3(kThreads), 0, s, a);
    else if (nt)
      hipLaunchKernelGGL((gn_stats<false, true>), dim3(blocks), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((gn_stats<false, false>), dim3(blocks), dim3(kThreads), 0, s, a);
  }
  // band moments (k < nb workgroups) only when the caller reads them
  const int kparts = a.want_band_moments ? L.nb + 1 : 1;
  hipLaunchKernelGGL(gn_merge, dim3(L.n_img * a.groups * kparts), dim3(kThreads), 0, s, a, coef);
  if (a.stats_only) return hipGetLastError();
  a.apply_pix = apply_pixels(L);
  long long nblk = 0;   // apply workgroups: runs of apply_pix pixels per (band, image)
  for (int b = 0; b < L.nb; ++b) {
    a.item_start[b] = nblk;
    nblk += (long long)L.n_img * (((long long)L.rows[b] * L.W + a.apply_pix - 1) / a.apply_pix);
  }
  a.item_start[L.nb] = nblk;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dtype == VAEP_DTYPE_F32 && !a.x_split)
    hipLaunchKernelGGL((gn_apply<float, false, false>), dim3((int)nblk), dim3(kThreads), 0, s, a, coef);
  else if (dtype == VAEP_DTYPE_F32)
    return hipErrorInvalidValue;   // split inputs exist on the bf16 path only
  else if (a.x_split && nt)
    hipLaunchKernelGGL((gn_apply<bf16, true, true>), dim3((int)nblk), dim3(kThreads), 0, s, a, coef);
  else if (a.x_split)
    hipLaunchKernelGGL((gn_apply<bf16, true, false>), dim3((int)nblk), dim3(kThreads), 0, s, a, coef);
  else if (nt)
    hipLaunchKernelGGL((gn_apply<bf16, false, true>), dim3((int)nblk), dim3(kThreads), 0, s, a, coef);
  else
    hipLaunchKernelGGL((gn_apply<bf16, false, false>), dim3((int)nblk), dim3(kThreads), 0, s, a, coef);
  return hipGetLastError();
}

template <typename TO, bool XS, bool NT>
static hipError_t go_rms_wave(NormArgs& a, int k, hipStream_t s) {
  const BandLayout& L = a.L;
  const int P = 64 * k / (L.C / V);
  long long runs = 0;
  for (int b = 0; b < L.nb; ++b) {
    a.item_start[b] = runs;
    runs += (long long)L.n_img * (((long long)L.rows[b] * L.W + P - 1) / P);
  }
  a.item_start[L.nb] = runs;
  if (runs == 0) return hipSuccess;
  // 32-bit run and pixel indices in the kernel
  if (runs > 0x7fffffffLL) return hipErrorInvalidValue;
  for (int b = 0; b < L.nb; ++b)
    if ((long long)L.rows[b] * L.W + P > 0x7fffffffLL) return hipErrorInvalidValue;
  const int r32 = (int)runs;
  long long nblk = (runs + 3) / 4;
  if (nblk > 4096) nblk = 4096;
  if (k == 1) hipLaunchKernelGGL((rms_wave<TO, XS, NT, 1>), dim3((int)nblk), dim3(kThreads), 0, s, a, r32);
  if (k == 2) hipLaunchKernelGGL((rms_wave<TO, XS, NT, 2>), dim3((int)nblk), dim3(kThreads), 0, s, a, r32);
  if (k == 3) hipLaunchKernelGGL((rms_wave<TO, XS, NT, 3>), dim3((int)nblk), dim3(kThreads), 0, s, a, r32);
  if (k == 4) hipLaunchKernelGGL((rms_wave<TO, XS, NT, 4>), dim3((int)nblk), dim3(kThreads), 0, s, a, r32);
  return hipGetLastError();
}

// float4 slots per lane of the wave-per-run RMSNorm for C channels: the smallest k with
// 64 * k a multiple of C / 4, if it is at most 4 (else 0: the per-pixel kernel runs).
static int rms_wave_k(int C) {
  const int q = C / V;
  for (int k = 1; k <= 4; ++k)
    if ((64 * k) % q == 0 && 64 * k / q <= 64) return k;
  return 0;
}

hipError_t launch_rmsnorm(NormArgs& a, int dtype, hipStream_t s) {
  const BandLayout& L = a.L;
  if (L.C % V != 0 || L.C / V > kThreads) return hipErrorInvalidValue;
  const int k = rms_wave_k(L.C);
  if (k > 0 && dtype == VAEP_DTYPE_BF16) {
    long long elems = 0;
    for (int b = 0; b < L.nb; ++b) elems += (long long)L.n_img * L.rows[b] * L.W * L.C;
    const bool nt = elems * 4 >= kStreamBytes;
    if (a.x_split && nt) return go_rms_wave<bf16, true, true>(a, k, s);
    if (a.x_split) return go_rms_wave<bf16, true, false>(a, k, s);
    if (nt) return go_rms_wave<bf16, false, true>(a, k, s);
    return go_rms_wave<bf16, false, false>(a, k, s);
  }
  long long pt = 0;
  for (int b = 0; b < L.nb; ++b) {
    a.item_start[b] = pt;
    pt += (long long)L.n_img * L.rows[b] * L.W;
  }
  a.item_start[L.nb] = pt;
  const int PX = kThreads / (L.C / V);
  long long nblk = (pt + PX - 1) / PX;
  if (nblk > 65536) nblk = 65536;
  if (nblk == 0) return hipSuccess;
  const bool nt = pt * L.C * 4 >= kStreamBytes;
  if (dtype == VAEP_DTYPE_F32 && !a.x_split)
    hipLaunchKernelGGL((rms_apply<float, false, false>), dim3((int)nblk), dim3(kThreads), 0, s, a);
  else if (dtype == VAEP_DTYPE_F32)
    return hipErrorInvalidValue;
  else if (a.x_split && nt)
    hipLaunchKernelGGL((rms_apply<bf16, true, true>), dim3((int)nblk), dim3(kThreads), 0, s, a);
  else if (a.x_split)
    hipLaunchKernelGGL((rms_apply<bf16, true, false>), dim3((int)nblk), dim3(kThreads), 0, s, a);
  else if (nt)
    hipLaunchKernelGGL((rms_apply<bf16, false, true>), dim3((int)nblk), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((rms_apply<bf16, false, false>), dim3((int)nblk), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_moment_merge(int n_shards, int n_stats, const float* mean, const float* var,
                               const int64_t* counts, float* mean_out, float* var_out,
                               hipStream_t s) {
  if (n_stats == 0) return hipSuccess;
  hipLaunchKernelGGL(moment_merge, dim3((n_stats + 255) / 256), dim3(256), 0, s, n_shards, n_stats,
                     mean, var, counts, mean_out, var_out);
  return hipGetLastError();
}

}  // namespace vaep
