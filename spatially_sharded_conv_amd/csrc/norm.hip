// GroupNorm with band-merged statistics, channel RMSNorm, and the moment merge.
//
// GroupNorm (ChituDiffusion "VAEP" feature page, GroupNorm section; "Static Layer-Wise
// VAE Decode", GroupNorm row and the formula below the table): every band computes
// FP32 central moments per (sample, group) of its own rows; the bands' moments are
// merged with actual-element-count weights,
//     mean = sum_i w_i mean_i,  var = sum_i w_i (var_i + (mean_i - mean)^2),
// and every band normalises with the merged statistics, then the channel affine and
// (in the decoder's norm -> SiLU pairs) SiLU.  The same weighted merge combines the
// per-workgroup tiles of a band into the band's moments.
//
// Data movement: the stats pass reads the band's rows once (16-byte loads, each
// workgroup a contiguous slab of one band and image), two-pass in registers per tile;
// the apply pass streams the rows again and writes the result plus the boundary rows
// into the neighbours' halo slots.  Channel RMSNorm is local to a pixel and needs no
// merge.
#include "vaep_internal.h"

namespace vaep {
namespace {

constexpr int kThreads = 256;
constexpr int kPixPerThread = 8;   // 16-byte vectors held in registers by one thread per stats tile
constexpr int V = 4;               // channels per 16-byte load of the fp32 input

__device__ __forceinline__ void load4(const float* p, float* v) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}

template <typename T> struct Out;
template <> struct Out<float> {
  __device__ static void store4(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Out<bf16> {
  __device__ static unsigned short rne(float f) {
    __hip_bfloat16 h = __float2bfloat16(f);
    return *reinterpret_cast<unsigned short*>(&h);
  }
  __device__ static void store4(bf16* p, const float* v) {
    uint2 q;
    q.x = rne(v[0]) | ((unsigned)rne(v[1]) << 16);
    q.y = rne(v[2]) | ((unsigned)rne(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = q;
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

__device__ __forceinline__ float silu(float v) { return v / (1.f + __expf(-v)); }

// Pass 1: central moments of one tile (kThreads/S pixel lanes x kPixPerThread pixels) of
// one (band, image): partials[blk][g] = (mean, M2) of group g over the tile, two-pass
// from registers, accumulated in fp64 so that the merged statistics do not depend on
// where the band boundaries cut the image.
__global__ void __launch_bounds__(kThreads) gn_stats(const NormArgs a) {
  __shared__ double red[kThreads * V];
  __shared__ double gmean[1024];
  const BandLayout& L = a.L;
  const int C = L.C, S = C / V, PL = kThreads / S;
  const int G = a.groups, cpg = C / G;
  const int blk = blockIdx.x;
  const int b = band_of_block(a.blk_start, L.nb, blk);
  const int local = blk - a.blk_start[b];
  const int n = local / a.blk_per_img[b];
  const int tile = local - n * a.blk_per_img[b];
  const long long npix = (long long)L.rows[b] * L.W;
  const long long p0 = (long long)tile * a.pix_per_blk[b];
  const int tid = threadIdx.x;
  const int slot = tid % S, pl = tid / S;
  const bool active = pl < PL;
  const float* base = reinterpret_cast<const float*>(a.x) + row_offset(L, b, n, 0) + (long long)slot * V;

  float x[kPixPerThread][V];
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kPixPerThread; ++k) {
    const long long p = p0 + (long long)k * PL + pl;
    if (active && p < npix) {
      load4(base + p * C, x[k]);
      ++cnt;
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) x[k][e] = 0.f;
    }
  }
  long long tp = npix - p0;
  if (tp > (long long)PL * kPixPerThread) tp = (long long)PL * kPixPerThread;
  const double n_el = (double)(tp * cpg);

  if (active) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      double s = 0.0;
#pragma unroll
      for (int k = 0; k < kPixPerThread; ++k) s += (double)x[k][e];
      red[pl * C + slot * V + e] = s;
    }
  }
  __syncthreads();
  if (tid < G) {
    double s = 0.0;
    for (int p = 0; p < PL; ++p)
      for (int j = 0; j < cpg; ++j) s += red[p * C + tid * cpg + j];
    gmean[tid] = s / n_el;
  }
  __syncthreads();
  double s2[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const double m = gmean[(slot * V + e) / cpg];
    s2[e] = 0.0;
#pragma unroll
    for (int k = 0; k < kPixPerThread; ++k) {
      const double d = (double)x[k][e] - m;
      s2[e] += (k < cnt) ? d * d : 0.0;
    }
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int e = 0; e < V; ++e) red[pl * C + slot * V + e] = s2[e];
  }
  __syncthreads();
  if (tid < G) {
    double s = 0.0;
    for (int p = 0; p < PL; ++p)
      for (int j = 0; j < cpg; ++j) s += red[p * C + tid * cpg + j];
    double* out = a.partials + ((long long)blk * G + tid) * 2;
    out[0] = gmean[tid];
    out[1] = s;
  }
}

// Pass 2: one workgroup per (image n, group g).  The tiles of each band merge into the
// band's (count, mean, var) with count weights; then the bands merge with the pages'
// formula.  fp64 throughout; the merged mean and variance are rounded to fp32 once.
// Writes the per-band moments, the merged mean / rstd and the per-channel scale/shift.
__global__ void __launch_bounds__(kThreads) gn_merge(const NormArgs a, float* coef) {
  __shared__ double sh[kThreads];
  __shared__ double bmean[kMaxBands], bvar[kMaxBands], bcnt[kMaxBands];
  __shared__ float fin[2];
  const BandLayout& L = a.L;
  const int G = a.groups, C = L.C, cpg = C / G;
  const int n = blockIdx.x / G, g = blockIdx.x - (blockIdx.x / G) * G;
  const int tid = threadIdx.x;
  for (int b = 0; b < L.nb; ++b) {
    const int nt = a.blk_per_img[b];
    const long long npix = (long long)L.rows[b] * L.W;
    const double total = (double)(npix * cpg);
    const int first = a.blk_start[b] + n * nt;
    double s = 0.0;
    for (int t = tid; t < nt; t += kThreads) {
      long long tp = npix - (long long)t * a.pix_per_blk[b];
      if (tp > a.pix_per_blk[b]) tp = a.pix_per_blk[b];
      s += ((double)(tp * cpg) / total) * a.partials[((long long)(first + t) * G + g) * 2];
    }
    sh[tid] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (tid < w) sh[tid] += sh[tid + w];
      __syncthreads();
    }
    const double mb = sh[0];
    __syncthreads();
    s = 0.0;
    for (int t = tid; t < nt; t += kThreads) {
      long long tp = npix - (long long)t * a.pix_per_blk[b];
      if (tp > a.pix_per_blk[b]) tp = a.pix_per_blk[b];
      const double nt_el = (double)(tp * cpg);
      const double* pr = a.partials + ((long long)(first + t) * G + g) * 2;
      const double d = pr[0] - mb;
      s += (nt_el / total) * (pr[1] / nt_el + d * d);
    }
    sh[tid] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (tid < w) sh[tid] += sh[tid + w];
      __syncthreads();
    }
    if (tid == 0) {
      bmean[b] = mb;
      bvar[b] = sh[0];
      bcnt[b] = total;
    }
    __syncthreads();
  }
  if (tid == 0) {
    double tot = 0.0;
    for (int b = 0; b < L.nb; ++b) tot += bcnt[b];
    double mean = 0.0;
    for (int b = 0; b < L.nb; ++b) mean += (bcnt[b] / tot) * bmean[b];
    double var = 0.0;
    for (int b = 0; b < L.nb; ++b) {
      const double d = bmean[b] - mean;
      var += (bcnt[b] / tot) * (bvar[b] + d * d);
    }
    const int s = n * G + g, ns = L.n_img * G;
    for (int b = 0; b < L.nb; ++b) {
      a.band_moments[(0 * L.nb + b) * (long long)ns + s] = (float)bcnt[b];
      a.band_moments[(1 * L.nb + b) * (long long)ns + s] = (float)bmean[b];
      a.band_moments[(2 * L.nb + b) * (long long)ns + s] = (float)bvar[b];
    }
    const float mean_f = (float)mean, var_f = (float)var;
    const float rstd = rsqrtf(var_f + a.eps);
    a.stats[s] = mean_f;
    a.stats[ns + s] = rstd;
    if (a.merged_out) {
      a.merged_out[s] = mean_f;
      a.merged_out[ns + s] = var_f;
    }
    fin[0] = mean_f;
    fin[1] = rstd;
  }
  __syncthreads();
  const float mean = fin[0], rstd = fin[1];
  for (int j = tid; j < cpg; j += kThreads) {
    const int ch = g * cpg + j;
    const float sc = rstd * a.gamma[ch];
    coef[((long long)n * C + ch) * 2] = sc;
    coef[((long long)n * C + ch) * 2 + 1] = a.beta[ch] - mean * sc;
  }
}

// Pass 3: y = act(x * scale_c + shift_c) over every owned row; boundary rows are also
// written into the neighbours' halo slots.
template <typename TO>
__global__ void __launch_bounds__(kThreads) gn_apply(const NormArgs a, const float* coef) {
  const BandLayout& L = a.L;
  const int C = L.C, S = C / V;
  const long long vtotal = a.item_start[L.nb];
  const float* X = reinterpret_cast<const float*>(a.x);
  TO* Y = reinterpret_cast<TO*>(a.y);
  for (long long gid = (long long)blockIdx.x * kThreads + threadIdx.x; gid < vtotal;
       gid += (long long)gridDim.x * kThreads) {
    int b = 0;
    while (b + 1 < L.nb && gid >= a.item_start[b + 1]) ++b;
    const long long v = gid - a.item_start[b];
    const long long per_img = (long long)L.rows[b] * L.W * S;
    const int n = (int)(v / per_img);
    const long long rem = v - n * per_img;
    const long long pix = rem / S;
    const int slot = (int)(rem - pix * S);
    const int r = (int)(pix / L.W);
    const int c = (int)(pix - (long long)r * L.W);
    const long long off = row_offset(L, b, n, r) + (long long)c * C + slot * V;
    float x[V];
    load4(X + off, x);
    const float* cf = coef + ((long long)n * C + slot * V) * 2;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float y = x[e] * cf[2 * e] + cf[2 * e + 1];
      x[e] = a.act ? silu(y) : y;
    }
    Out<TO>::store4(Y + off, x);
    if (r == 0 && b > 0)
      Out<TO>::store4(Y + row_offset(L, b - 1, n, L.rows[b - 1]) + (long long)c * C + slot * V, x);
    if (r == L.rows[b] - 1 && b + 1 < L.nb)
      Out<TO>::store4(Y + row_offset(L, b + 1, n, -1) + (long long)c * C + slot * V, x);
  }
}

// Channel RMSNorm: y_c = gamma_c x_c / sqrt(mean_c x^2 + eps) (+SiLU), per pixel.
template <typename TO>
__global__ void __launch_bounds__(kThreads) rms_apply(const NormArgs a) {
  __shared__ float part[kThreads];
  __shared__ float rs[kThreads];
  const BandLayout& L = a.L;
  const int C = L.C, S = C / V, PX = kThreads / S;
  const int tid = threadIdx.x;
  const int slot = tid % S, px = tid / S;
  const long long ptotal = a.item_start[L.nb];
  const float* X = reinterpret_cast<const float*>(a.x);
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
      load4(X + off, x);
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


// Stats tiling of a layout: blocks per band and image, pixels per block.
static void plan_stats(NormArgs& a, int dtype) {
  const int S = a.L.C / V;
  const int PL = kThreads / S;
  const int pix = PL * kPixPerThread;
  int t = 0;
  for (int b = 0; b < a.L.nb; ++b) {
    a.blk_start[b] = t;
    const long long np = (long long)a.L.rows[b] * a.L.W;
    a.blk_per_img[b] = (int)((np + pix - 1) / pix);
    a.pix_per_blk[b] = pix;
    t += a.blk_per_img[b] * a.L.n_img;
  }
  a.blk_start[a.L.nb] = t;
}

size_t gn_partials_floats(const BandLayout& L, int groups, int dtype) {
  // Bound over every band table with L.nb bands: sum_i ceil(rows_i W / pix) <= ceil(H W / pix) + nb.
  const int S = L.C / V;
  const int pix = (kThreads / S) * kPixPerThread;
  const long long blocks = (long long)L.n_img * (((long long)L.H * L.W + pix - 1) / pix + L.nb);
  // (in floats) fp64 partials, per-channel coefficients, per-band moments, merged stats
  return (size_t)(blocks * groups * 4 + 2LL * L.n_img * L.C + 3LL * L.nb * L.n_img * groups +
                  2LL * L.n_img * groups);
}

hipError_t launch_groupnorm(NormArgs& a, int dtype, hipStream_t s) {
  const BandLayout& L = a.L;
  if (L.C % V != 0 || L.C / V > kThreads || L.C % a.groups != 0 || a.groups > 1024)
    return hipErrorInvalidValue;
  plan_stats(a, dtype);
  const int blocks = a.blk_start[L.nb];
  // Scratch carve-up inside a.partials (sized by gn_partials_floats).
  float* coef = reinterpret_cast<float*>(a.partials + (size_t)blocks * a.groups * 2);
  a.band_moments = coef + 2LL * L.n_img * L.C;
  a.stats = a.band_moments + 3LL * L.nb * L.n_img * a.groups;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(gn_stats, dim3(blocks), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(gn_merge, dim3(L.n_img * a.groups), dim3(kThreads), 0, s, a, coef);
  long long vt = 0;
  for (int b = 0; b < L.nb; ++b) {
    a.item_start[b] = vt;
    vt += (long long)L.n_img * L.rows[b] * L.W * (L.C / V);
  }
  a.item_start[L.nb] = vt;
  long long nblk = (vt + kThreads - 1) / kThreads;
  if (nblk > 65536) nblk = 65536;
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(gn_apply<float>, dim3((int)nblk), dim3(kThreads), 0, s, a, coef);
  else
    hipLaunchKernelGGL(gn_apply<bf16>, dim3((int)nblk), dim3(kThreads), 0, s, a, coef);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(NormArgs& a, int dtype, hipStream_t s) {
  const BandLayout& L = a.L;
  if (L.C % V != 0 || L.C / V > kThreads) return hipErrorInvalidValue;
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
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(rms_apply<float>, dim3((int)nblk), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(rms_apply<bf16>, dim3((int)nblk), dim3(kThreads), 0, s, a);
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
