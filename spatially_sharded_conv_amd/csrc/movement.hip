// Data movement around the band buffers: scatter a whole tensor into bands (with the
// neighbours' boundary rows in the halo slots), gather bands back, the first frame of
// the causal temporal upsample, and weight repacking.
#include "vaep_internal.h"
#include "split8.h"

namespace vaep {
namespace {

template <typename T>
__global__ void pack_kernel(const T* src, int c_src, T* dst, const BandLayout L, int tr) {
  const int b = blockIdx.y;
  const long long total = (long long)L.n_img * (L.rows[b] + 2) * L.W * L.C;
  const long long HW = (long long)L.H * L.W;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int ch = (int)(i % L.C);
    const long long pix = i / L.C;
    const int c = (int)(pix % L.W);
    const long long rr = pix / L.W;
    const int rp = (int)(rr % (L.rows[b] + 2));
    const int n = (int)(rr / (L.rows[b] + 2));
    const int g = L.row0[b] + rp - 1;   // global row of this slot
    T v = T(0.f);
    if (ch < c_src && g >= 0 && g < L.H) {
      const int bs = n / L.frames, t = n - bs * L.frames;
      const long long pix = tr ? (long long)c * L.H + g : (long long)g * L.W + c;
      v = src[(((long long)bs * c_src + ch) * L.frames + t) * HW + pix];
    }
    dst[L.off[b] + i] = v;
  }
}

template <typename T>
__global__ void unpack_kernel(const T* src, const BandLayout L, T* dst, int c_dst) {
  const long long HW = (long long)L.H * L.W;
  const long long total = (long long)L.n_img * c_dst * HW;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % L.W);
    const int g = (int)((i / L.W) % L.H);
    const long long rest = i / HW;               // (bs, ch, t)
    const int t = (int)(rest % L.frames);
    const int ch = (int)((rest / L.frames) % c_dst);
    const int bs = (int)(rest / ((long long)L.frames * c_dst));
    const int n = bs * L.frames + t;
    int b = 0;
    while (b + 1 < L.nb && g >= L.row0[b + 1]) ++b;
    const int r = g - L.row0[b];
    dst[i] = src[L.off[b] + (((long long)n * (L.rows[b] + 2) + r + 1) * L.W + c) * L.C + ch];
  }
}

template <typename T>
__global__ void copy_frame0_kernel(const T* src, const BandLayout Ls, T* dst, const BandLayout Ld) {
  const int b = blockIdx.y;
  const int bs = blockIdx.z;
  const long long per = (long long)(Ls.rows[b] + 2) * Ls.W * Ls.C;   // one frame, halos included
  const T* s = src + Ls.off[b] + (long long)(bs * Ls.frames) * per;
  T* d = dst + Ld.off[b] + (long long)(bs * Ld.frames) * per;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < per;
       i += (long long)gridDim.x * blockDim.x)
    d[i] = s[i];
}

// Debug fill of every halo slot (the row above and below each band, per image) with 0xFF
// bytes: NaN as fp32, bf16 and either fp8 format.  Slot blockIdx.y = (band, image, side);
// the row holds row_words 32-bit words.
__global__ void poison_halo_kernel(unsigned* buf, const BandLayout L, int elem_bytes) {
  const int k = blockIdx.y;
  const int side = k & 1, bn = k >> 1;
  const int b = bn / L.n_img, n = bn - b * L.n_img;
  const long long row_elems = (long long)L.W * L.C;
  const long long slot = (long long)n * (L.rows[b] + 2) + (side ? L.rows[b] + 1 : 0);
  const long long first = (L.off[b] + slot * row_elems) * elem_bytes / 4;
  const long long words = row_elems * elem_bytes / 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (long long)gridDim.x * blockDim.x)
    buf[first + i] = 0xffffffffu;
}

template <typename T>
__global__ void pack_weight_kernel(const T* src, int co, int ci, int taps, T* dst, int co_pad,
                                   int ci_pad, int rep, int tr) {
  // rep copies of the ci_pad input channels per tap (rep = 2: one per bf16 part of a
  // split operand)
  const int row = ci_pad * rep;
  const long long total = (long long)co_pad * taps * row;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % row) % ci_pad;
    const int t = (int)((i / row) % taps);
    const int o = (int)(i / ((long long)row * taps));
    T v = T(0.f);
    // the transposed kernel swaps the two spatial tap indices within each time tap
    const int ts = tr ? (t / 9) * 9 + (t % 3) * 3 + (t % 9) / 3 : t;
    if (o < co && c < ci) v = src[((long long)o * ci + c) * taps + ts];
    dst[i] = v;
  }
}

// Sub-pixel form of nearest-2x + 3x3 conv.  For output phase py (row parity), kernel row
// dy reads source row offset floor((py + dy - 1) / 2), which is -1, 0, 0 for py = 0 and
// 0, 0, 1 for py = 1; folded row tap a of phase py sums the kernel rows whose offset is
// a - 1 + py (columns likewise).  The fp32 sum is stored as bf16 hi and lo parts.
// Largest |w| of n bf16 weights -> scale[1] (float bits).  One workgroup of 1024 threads;
// with vec (src 16-byte aligned, n a multiple of 8) each thread keeps eight 16-byte loads
// in flight, else it reads one weight at a time.
__global__ void __launch_bounds__(1024) absmax_kernel(const bf16* src, long long n, int vec, int* scale) {
  constexpr int kT = 1024, kU = 8;
  __shared__ float part[kT];
  float m = 0.f;
  if (vec) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    const long long n8 = n / 8;
    for (long long i0 = 0; i0 < n8; i0 += (long long)kT * kU) {
      uint4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const long long i = i0 + (long long)u * kT + threadIdx.x;
        v[u] = i < n8 ? s4[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const unsigned w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          m = fmaxf(m, fabsf(__uint_as_float(w[e] << 16)));
          m = fmaxf(m, fabsf(__uint_as_float(w[e] & 0xffff0000u)));
        }
      }
    }
  } else {
    for (long long i = threadIdx.x; i < n; i += kT) m = fmaxf(m, fabsf((float)src[i]));
  }
  part[threadIdx.x] = m;
  __syncthreads();
  for (int w = kT / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] = fmaxf(part[threadIdx.x], part[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) scale[1] = __float_as_int(part[0]);
}

// Folded weights in the encoding of split8.h.  A folded weight sums at most four
// weights, so 4 max |w| bounds it; s follows from that bound.  Thread 0 stores the MFMA
// scale of A, E8M0 of 2^-(s+9) in every byte, at scale[0].
__global__ void fold_subpixel_kernel(const bf16* src, int co, int ci, unsigned char* dst, int co_pad, int tr,
                                     int* scale) {
  const int sh = split8::weight_shift(4.f * __int_as_float(scale[1]));
  const float up = ldexpf(1.f, sh), up_lo = ldexpf(1.f, sh + split8::kLoShift);
  if (blockIdx.x == 0 && threadIdx.x == 0 && !tr)
    scale[0] = (127 - sh - split8::kLoShift) * 0x01010101;
  const long long total = 4LL * co_pad * 4 * ci;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % ci);
    const int tap = (int)((i / ci) % 4);
    const int o = (int)((i / (4LL * ci)) % co_pad);
    const int ph = (int)(i / (4LL * ci * co_pad));
    const int py = ph >> 1, px = ph & 1, ta = tap >> 1, tb = tap & 1;
    float w = 0.f;
    if (o < co) {
      for (int dy = 0; dy < 3; ++dy) {
        if (((py + dy - 1) >> 1) != ta - 1 + py) continue;
        for (int dx = 0; dx < 3; ++dx) {
          if (((px + dx - 1) >> 1) != tb - 1 + px) continue;
          w += (float)src[(((long long)o * ci + c) * 3 + (tr ? dx : dy)) * 3 + (tr ? dy : dx)];
        }
      }
    }
    const bf16 hi = bf16(w);
    // row of this (phase, output channel, tap): ci bf16 hi parts, then 2 ci fp8 bytes
    unsigned char* d = dst + ((((long long)ph * co_pad + o) * 4 + tap) * 4LL) * ci;
    *reinterpret_cast<bf16*>(d + 2LL * c) = hi;
    const long long f = split8::lo_byte(ci, c);
    d[f] = (unsigned char)split8::to_e4m3(w * up);
    d[f + 64] = (unsigned char)split8::to_e4m3((w - (float)hi) * up_lo);
  }
}

// fp32 pixel of C channels -> the operand encoding of split8.h (4C bytes), four channels
// per thread.
__global__ void split_kernel(const float* src, long long n4, int C, unsigned char* dst) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    const float4 f = reinterpret_cast<const float4*>(src)[i];
    const float v[4] = {f.x, f.y, f.z, f.w};
    const long long pix = (4 * i) / C;
    const int ch = (int)(4 * i - pix * C);
    unsigned char* d = dst + pix * 4LL * C;
    uint2 h;
    h.x = (unsigned)__bfloat16_as_ushort(__float2bfloat16(v[0])) |
          ((unsigned)__bfloat16_as_ushort(__float2bfloat16(v[1])) << 16);
    h.y = (unsigned)__bfloat16_as_ushort(__float2bfloat16(v[2])) |
          ((unsigned)__bfloat16_as_ushort(__float2bfloat16(v[3])) << 16);
    *reinterpret_cast<uint2*>(d + 2LL * ch) = h;
    unsigned lo, xs;
    split8::operand_bytes4(v, &lo, &xs);
    const long long fb = split8::lo_byte(C, ch);
    *reinterpret_cast<unsigned*>(d + fb) = lo;
    *reinterpret_cast<unsigned*>(d + fb + 64) = xs;
  }
}

__global__ void add_f32_kernel(const float* a, const float* b, float* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = a[i] + b[i];
}

template <typename T>
__global__ void to_f32_kernel(const T* src, int n, float* dst, int n_pad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_pad) dst[i] = (src != nullptr && i < n) ? (float)src[i] : 0.f;
}

int grid_for(long long n) {
  long long g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  return g < 1 ? 1 : (int)g;
}

// Latent tile: rows [i, i + th), columns [j, j + tw) of every (sample, channel, frame)
// plane of an NC[T]HW tensor, stored contiguously.
template <typename T>
__global__ void crop_kernel(const T* src, long long planes, int h, int w, int i, int j, int th, int tw, T* dst) {
  const long long total = planes * th * tw;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int x = (int)(e % tw);
    const int y = (int)((e / tw) % th);
    const long long p = e / ((long long)th * tw);
    dst[e] = src[(p * h + i + y) * w + j + x];
  }
}

// Linear cross-fade of a tile's first e rows (axis 0) or columns (axis 1) from the last
// ones of its neighbour, in place: v = nb * (1 - k / e) + v * (k / e), k = row / column.
// Tiles are [planes][th][tw] fp32; the neighbour has the same width (rows) or height
// (columns) and nb_len rows / columns.
__global__ void blend_kernel(const float* nb, float* tile, long long planes, int th, int tw, int nb_len, int e,
                             int axis) {
  const int other = axis == 0 ? tw : th;
  const long long total = planes * e * other;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int o = (int)(idx % other);
    const int k = (int)((idx / other) % e);
    const long long p = idx / ((long long)e * other);
    const float wt = (float)k / (float)e;
    float* v;
    float n;
    if (axis == 0) {
      v = tile + (p * th + k) * tw + o;
      n = nb[(p * nb_len + nb_len - e + k) * tw + o];
    } else {
      v = tile + (p * th + o) * tw + k;
      n = nb[(p * th + o) * nb_len + nb_len - e + k];
    }
    *v = n * (1.f - wt) + *v * wt;
  }
}

// Output of the tiled decode: output row y, column x comes from tile (y / keep, x / keep)
// at (y % keep, x % keep).  Tile (gi, gj) sits in slot tile_slot(...), [planes][th][tw].
__global__ void tiles_gather_kernel(const float* slots, long long slot_elems, long long planes, int H, int W,
                                    int keep, int tile_out, int nc, int full_r, int full_c, int lat_h, int lat_w,
                                    int stride, int up, float* out) {
  const long long total = planes * H * W;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int x = (int)(e % W);
    const int y = (int)((e / W) % H);
    const long long p = e / ((long long)H * W);
    const int gi = y / keep, gj = x / keep;
    const int th = min(tile_out, (lat_h - gi * stride) * up);
    const int tw = min(tile_out, (lat_w - gj * stride) * up);
    const float* t = slots + (long long)tile_slot(gi, gj, nc, full_r, full_c) * slot_elems;
    out[e] = t[(p * th + (y - gi * keep)) * tw + (x - gj * keep)];
  }
}

}  // namespace

hipError_t launch_crop(const void* src, long long planes, int h, int w, int i, int j, int th, int tw, void* dst,
                       int dtype, hipStream_t s) {
  const long long total = planes * th * tw;
  if (total == 0) return hipSuccess;
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(crop_kernel<float>, dim3(grid_for(total)), dim3(256), 0, s, (const float*)src, planes, h, w,
                       i, j, th, tw, (float*)dst);
  else
    hipLaunchKernelGGL(crop_kernel<bf16>, dim3(grid_for(total)), dim3(256), 0, s, (const bf16*)src, planes, h, w,
                       i, j, th, tw, (bf16*)dst);
  return hipGetLastError();
}

hipError_t launch_blend(const float* nb, float* tile, long long planes, int th, int tw, int nb_len, int e, int axis,
                        hipStream_t s) {
  const long long total = planes * e * (axis == 0 ? tw : th);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(blend_kernel, dim3(grid_for(total)), dim3(256), 0, s, nb, tile, planes, th, tw, nb_len, e, axis);
  return hipGetLastError();
}

hipError_t launch_tiles_gather(const float* slots, long long slot_elems, long long planes, int H, int W, int keep,
                               int tile_out, int nc, int full_r, int full_c, int lat_h, int lat_w, int stride, int up,
                               float* out, hipStream_t s) {
  const long long total = planes * H * W;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(tiles_gather_kernel, dim3(grid_for(total)), dim3(256), 0, s, slots, slot_elems, planes, H, W,
                     keep, tile_out, nc, full_r, full_c, lat_h, lat_w, stride, up, out);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, int c_src, void* dst, const BandLayout& L, int dtype,
                       hipStream_t s, bool transposed) {
  long long mx = 0;
  for (int b = 0; b < L.nb; ++b) {
    const long long e = (long long)L.n_img * (L.rows[b] + 2) * L.W * L.C;
    if (e > mx) mx = e;
  }
  dim3 grid(grid_for(mx), L.nb);
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(pack_kernel<float>, grid, dim3(256), 0, s, (const float*)src, c_src, (float*)dst, L,
                       transposed ? 1 : 0);
  else
    hipLaunchKernelGGL(pack_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)src, c_src, (bf16*)dst, L,
                       transposed ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_unpack(const void* src, const BandLayout& L, void* dst, int c_dst, int dtype,
                         hipStream_t s) {
  const long long total = (long long)L.n_img * c_dst * L.H * L.W;
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(unpack_kernel<float>, dim3(grid_for(total)), dim3(256), 0, s, (const float*)src, L, (float*)dst, c_dst);
  else
    hipLaunchKernelGGL(unpack_kernel<bf16>, dim3(grid_for(total)), dim3(256), 0, s, (const bf16*)src, L, (bf16*)dst, c_dst);
  return hipGetLastError();
}

hipError_t launch_copy_frame0(const void* src, const BandLayout& Ls, void* dst, const BandLayout& Ld,
                              int dtype, hipStream_t s) {
  long long mx = 0;
  for (int b = 0; b < Ls.nb; ++b) {
    const long long e = (long long)(Ls.rows[b] + 2) * Ls.W * Ls.C;
    if (e > mx) mx = e;
  }
  const int batch = Ls.n_img / Ls.frames;
  dim3 grid(grid_for(mx), Ls.nb, batch);
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(copy_frame0_kernel<float>, grid, dim3(256), 0, s, (const float*)src, Ls, (float*)dst, Ld);
  else
    hipLaunchKernelGGL(copy_frame0_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)src, Ls, (bf16*)dst, Ld);
  return hipGetLastError();
}

hipError_t launch_poison_halos(void* buf, const BandLayout& L, int elem_bytes, hipStream_t s) {
  const long long slots = 2LL * L.nb * L.n_img;
  if (slots == 0 || L.W == 0 || L.C == 0) return hipSuccess;
  if (slots > 65535 || (elem_bytes != 2 && elem_bytes != 4) || ((long long)L.W * L.C * elem_bytes) % 4 != 0 ||
      (reinterpret_cast<unsigned long long>(buf) & 3) != 0)
    return hipErrorInvalidValue;
  const long long words = (long long)L.W * L.C * elem_bytes / 4;
  dim3 grid((unsigned)std::min<long long>((words + 255) / 256, 64), (unsigned)slots);
  hipLaunchKernelGGL(poison_halo_kernel, grid, dim3(256), 0, s, reinterpret_cast<unsigned*>(buf), L, elem_bytes);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const void* src, int co, int ci, int taps, void* dst, int co_pad,
                              int ci_pad, int dtype, hipStream_t s, int rep, bool transposed) {
  if (transposed && taps % 9 != 0) return hipErrorInvalidValue;
  const long long total = (long long)co_pad * taps * ci_pad * rep;
  const int tr = transposed ? 1 : 0;
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(pack_weight_kernel<float>, dim3(grid_for(total)), dim3(256), 0, s,
                       (const float*)src, co, ci, taps, (float*)dst, co_pad, ci_pad, rep, tr);
  else
    hipLaunchKernelGGL(pack_weight_kernel<bf16>, dim3(grid_for(total)), dim3(256), 0, s,
                       (const bf16*)src, co, ci, taps, (bf16*)dst, co_pad, ci_pad, rep, tr);
  return hipGetLastError();
}

hipError_t launch_fold_subpixel_weight(const void* src, int co, int ci, void* dst, int co_pad, int* scale,
                                       hipStream_t s, bool transposed) {
  if (ci % 64 != 0) return hipErrorInvalidValue;
  if (!transposed) {
    const long long n = 9LL * co * ci;
    const int vec = (reinterpret_cast<uintptr_t>(src) % 16 == 0 && n % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(absmax_kernel, dim3(1), dim3(1024), 0, s, (const bf16*)src, n, vec, scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long total = 4LL * co_pad * 4 * ci;
  hipLaunchKernelGGL(fold_subpixel_kernel, dim3(grid_for(total)), dim3(256), 0, s, (const bf16*)src, co, ci,
                     (unsigned char*)dst, co_pad, transposed ? 1 : 0, scale);
  return hipGetLastError();
}

hipError_t launch_split(const float* src, const BandLayout& L, void* dst, hipStream_t s) {
  if (L.C % 64 != 0) return hipErrorInvalidValue;
  const long long n = layout_elems(L);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(split_kernel, dim3(grid_for(n / 4)), dim3(256), 0, s, src, n / 4, L.C, (unsigned char*)dst);
  return hipGetLastError();
}

hipError_t launch_add_f32(const float* a, const float* b, float* out, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(add_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a, b, out, n);
  return hipGetLastError();
}

hipError_t launch_to_f32(const void* src, int n, float* dst, int n_pad, int dtype, hipStream_t s) {
  if (n_pad <= 0) return hipSuccess;
  if (dtype == VAEP_DTYPE_F32)
    hipLaunchKernelGGL(to_f32_kernel<float>, dim3((n_pad + 255) / 256), dim3(256), 0, s, (const float*)src, n, dst, n_pad);
  else
    hipLaunchKernelGGL(to_f32_kernel<bf16>, dim3((n_pad + 255) / 256), dim3(256), 0, s, (const bf16*)src, n, dst, n_pad);
  return hipGetLastError();
}

}  // namespace vaep
