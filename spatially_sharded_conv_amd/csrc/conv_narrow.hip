// Narrow-output convolution: the decoder's last conv (a few image channels out of 96-512
// normalised channels), written straight into the NC[T]HW output tensor.
//
// Same operation and band rules as conv.hip (ChituDiffusion "VAEP" feature page, conv
// section; "Static Layer-Wise VAE Decode", operator table, "Spatial convolution" row):
// the band reads its own rows and the neighbours' halo rows, zero padding only outside
// the image (and before frame 0 for causal 3x3x3 kernels).
//
// Layout of the work: D[pixel][co] = X[pixel][k] W[k][co] with v_mfma_f32_16x16x32_bf16,
// pixels as the 16 rows and the output channels (zero-padded to 16) as the columns, so
// the matrix cores spend their width on pixels rather than on a mostly empty
// output-channel tile.  One 256-thread workgroup covers 128 pixels of kRows consecutive
// rows of one band and image, wave w computing row w (8 blocks of 16 pixels).  For each
// input frame of the causal window and each 32-channel chunk of the input it first
// stages the kRows + 2 rows x 130 pixels the taps read (the tile plus one column each
// side; zeros outside the image and before frame 0) in LDS, then runs those taps' MFMAs
// from there: each input row crosses the memory hierarchy (kRows + 2) / kRows times per
// frame instead of three times.
#include "vaep_internal.h"

namespace vaep {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

namespace {

constexpr int kNarrowPix = 128;              // pixels of one row per workgroup
constexpr int kStageW = kNarrowPix + 2;      // staged pixels per row (one halo column each side)
constexpr int kRows = 4;                     // output rows per workgroup (one per wave)

__device__ __forceinline__ int band_of_tile(const ConvArgs& a, int mt) {
  int b = 0;
  while (b + 1 < a.in.nb && mt >= a.tile_start[b + 1]) ++b;
  return b;
}

// LDS position (in 16-byte chunks) of chunk q (8 channels) of staged pixel i of staged
// row `row` with QN chunks per pixel, XOR-swizzled within groups of four by the pixel so
// that the 16 lanes of a fragment read (16 consecutive pixels, one chunk) fall in
// distinct banks.
template <int QN>
__device__ __forceinline__ int stage_slot(int row, int i, int q) {
  return (row * kStageW + i) * QN + (q ^ ((i >> 1) & 3));
}

// One round stages one 32-channel chunk of one input frame.
template <int KT, int NC>
__global__ void __launch_bounds__(256) conv_narrow(const ConvArgs a) {
  constexpr int ROWS = kRows + 2;             // staged rows: the tile's rows and one above / below
  constexpr int TAPS = KT * 9;
  constexpr int QN = 4;                       // 16-byte chunks per staged pixel
  constexpr int SLOTS = ROWS * kStageW * QN;  // 16-byte chunks staged per round
  constexpr int PER = (SLOTS + 255) / 256;    // per thread
  constexpr int NB = kNarrowPix / 16;         // 16-pixel blocks per wave (its row)
  __shared__ __attribute__((aligned(16))) u32x4_t sx[SLOTS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int mt = blockIdx.x;
  const int band = band_of_tile(a, mt);
  const int tile = mt - a.tile_start[band];
  const int rows_in = a.in.rows[band];
  const int W = a.in.W, H = a.in.H, C = a.in.C;
  const int tiles_row = (W + kNarrowPix - 1) / kNarrowPix;
  const int groups = (rows_in + kRows - 1) / kRows;  // row groups per image
  const int lg = tile / tiles_row;                 // image * groups + row group
  const int c0 = (tile - lg * tiles_row) * kNarrowPix;
  const int n = lg / groups, r0 = (lg - (lg / groups) * groups) * kRows;
  const int t = n % a.in.frames;
  const int g0 = a.in.row0[band] + r0;             // global row of the tile's first row
  const unsigned short* xb = reinterpret_cast<const unsigned short*>(a.x) + a.in.off[band];
  const long long ktot = (long long)TAPS * C;
  // B fragments: W[co = lane%16][tap][chunk * 32 + 8 * (lane/16) ..] (rows past cout are zero)
  const unsigned short* wrow = reinterpret_cast<const unsigned short*>(a.w) + (long long)(lane & 15) * ktot + 8 * (lane >> 4);

  f32x4_t acc[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) acc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int dt = 0; dt < KT; ++dt) {
    if (t + dt - (KT - 1) < 0) continue;          // frame before 0: these taps read zeros
    const unsigned short* fb = xb + (long long)(n + dt - (KT - 1)) * (rows_in + 2) * W * C;
    for (int ch = 0; ch < NC; ++ch) {
      // stage: row s holds band row r0 + s - 1 (slot r0 + s of the image), pixels c0 - 1 ..
      // c0 + 128, channels 32 ch ..; rows past the band's bottom halo slot belong to the
      // next image and feed only rows this tile does not store: zeros
      u32x4_t v[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int sl = tid + 256 * k;
        v[k] = u32x4_t{0u, 0u, 0u, 0u};
        if (sl < SLOTS) {
          const int e = sl / QN, q = sl - (sl / QN) * QN;
          const int row = e / kStageW, i = e - row * kStageW;
          const int c = c0 + i - 1, gr = g0 + row - 1, slot = r0 + row;
          if (c >= 0 && c < W && gr >= 0 && gr < H && slot <= rows_in + 1)
            v[k] = *reinterpret_cast<const u32x4_t*>(fb + ((long long)slot * W + c) * C + ch * 32 + q * 8);
        }
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int sl = tid + 256 * k;
        if (sl < SLOTS) {
          const int e = sl / QN, q = sl - (sl / QN) * QN;
          sx[stage_slot<QN>(e / kStageW, e % kStageW, q)] = v[k];
        }
      }
      __syncthreads();
#pragma unroll
      for (int tp = 0; tp < 9; ++tp) {
        const int dy = tp / 3, dx = tp % 3;
        const bf16x8_t bw = *reinterpret_cast<const bf16x8_t*>(wrow + (long long)(dt * 9 + tp) * C + ch * 32);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const int i = 16 * bb + (lane & 15) + dx;   // staged pixel of this tap
          const bf16x8_t ax = __builtin_bit_cast(bf16x8_t, sx[stage_slot<QN>(wave + dy, i, lane >> 4)]);
          acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, acc[bb], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }

  // lane holds output channel lane%16 for pixels c0 + 16*bb + 4*(lane/16) + v of row r0 + wave
  const int co = lane & 15;
  if (co >= a.cout || r0 + wave >= rows_in) return;
  const int g = g0 + wave;
  const float bias = a.bias[co];
  const int T = a.final_frames;
  const long long hw = (long long)H * W;
  const int bs = n / T, tt = n - bs * T;
  float* out = reinterpret_cast<float*>(a.y) + ((long long)bs * a.cout + co) * T * hw + (long long)tt * hw;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = c0 + 16 * bb + 4 * (lane >> 4) + v;
      if (c >= W) continue;
      const long long pix = a.out_transposed ? (long long)c * H + g : (long long)g * W + c;
      out[pix] = acc[bb][v] + bias;
    }
}

}  // namespace

bool conv_narrow_fits(const ConvArgs& a) {
  return a.mode == kModeFinal && a.cout <= 16 && a.cout_pad >= 16 && (a.in.C == 96 || a.in.C == 128) && !a.x_f32 &&
         !a.x_split && !a.ups && !a.down && a.ks == 3 && (a.kt == 1 || a.kt == 3);
}

hipError_t launch_conv_narrow(ConvArgs& a, hipStream_t s) {
  const int tiles_row = (a.in.W + kNarrowPix - 1) / kNarrowPix;
  int t = 0;
  for (int b = 0; b < a.in.nb; ++b) {
    a.tile_start[b] = t;
    const long long m = (long long)a.in.n_img * ((a.in.rows[b] + kRows - 1) / kRows) * tiles_row;
    if (t + m > 0x7fffffffLL) return hipErrorInvalidValue;
    t += (int)m;
  }
  a.tile_start[a.in.nb] = t;
  a.tiles_total = t;
  a.kernel_used = VAEP_KERNEL_CONV_NARROW;
  if (t == 0) return hipSuccess;
  const bool c128 = a.in.C == 128;
  if (a.kt == 3 && c128)
    hipLaunchKernelGGL((conv_narrow<3, 4>), dim3(t), dim3(256), 0, s, a);
  else if (a.kt == 3)
    hipLaunchKernelGGL((conv_narrow<3, 3>), dim3(t), dim3(256), 0, s, a);
  else if (c128)
    hipLaunchKernelGGL((conv_narrow<1, 4>), dim3(t), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((conv_narrow<1, 3>), dim3(t), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace vaep
