// Internal declarations shared by the host executor and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <cstddef>
#include <cstdint>

#include "../../include/vaep.h"

namespace vaep {

constexpr int kMaxBands = VAEP_MAX_BANDS;

using bf16 = __hip_bfloat16;

// Per-band activation buffers.  Band i holds `rows[i]` owned rows plus one halo row
// above and one below, for every image (batch x frames), channels innermost:
//   element (band i, image n, row r in [-1, rows[i]], col c, channel ch) lives at
//   off[i] + ((n * (rows[i] + 2) + r + 1) * W + c) * C + ch.
// The halo rows of band i hold copies of the neighbours' boundary rows, written by
// the producer of the tensor (the "halo push"); rows outside the image are never read.
struct BandLayout {
  int nb;          // number of bands
  int n_img;       // images = batch * frames
  int frames;      // frames per sample (1 for images)
  int H, W, C;     // global height, width, channel stride
  int rows[kMaxBands];
  int row0[kMaxBands];      // global index of the band's first row
  long long off[kMaxBands]; // element offset of band i's buffer
};

// Total elements of a layout (all bands, halo rows included).
inline long long layout_elems(const BandLayout& L) {
  long long e = 0;
  for (int i = 0; i < L.nb; ++i) e += (long long)L.n_img * (L.rows[i] + 2) * L.W * L.C;
  return e;
}

// Slots (rows, halo slots included) of band b's buffer that one conv tile of `bn` compute
// pixels can read: the conv kernels give every tile a buffer resource over the slots from
// its first pixel's row - 1, kt - 1 images back, to its last pixel's row + 1 (with ups, the
// source rows of a compute grid of twice the rows and width).  A tile's compute rows within
// one image number at most c = ceil(bn / wc) + 1; when the tile also reaches into the next
// image the range adds that image's first rows: at most (kt - 1)(rows + 2) + 2c + 4 slots
// while an image holds at least bn compute pixels.  Capped at the whole buffer.
// With down (a stride-2 conv: compute grid of half the rows and width) c compute rows read
// 2c + 1 source rows.
inline long long tile_read_slots(const BandLayout& in, int b, int kt, int bn, bool ups, bool down = false) {
  const long long R = in.rows[b], wc = ups ? 2LL * in.W : (down ? in.W / 2 : in.W);
  const long long plane = (ups ? 2 * R : (down ? R / 2 : R)) * wc;
  if (wc < 1 || plane < 1) return (long long)in.n_img * (R + 2);
  const long long c = (bn + wc - 1) / wc + 1;
  const long long src = down ? 2 * c + 1 : c;
  long long slots = plane >= bn ? (kt - 1) * (R + 2) + 2 * src + 4 : (kt + 1 + (bn + plane - 1) / plane) * (R + 2);
  const long long all = (long long)in.n_img * (R + 2);
  return slots < all ? slots : all;
}

// Fill a layout from band row counts; bands are stored back to back from element 0.
BandLayout make_layout(int nb, const int* rows, int n_img, int frames, int W, int C);
// The same bands after a nearest-2x upsample: rows and width double.
BandLayout upsampled(const BandLayout& L, int C);
// Same rows/width, a different channel count and image count.
BandLayout reshaped(const BandLayout& L, int C, int n_img, int frames);

// ------------------------------------------------------------------ conv
enum ConvMode : int {
  kModeBand = 0,            // band-layout output (+bias, +residual), halo push
  kModeQKV = 1,             // global token-major Q, K and transposed V
  kModeFinal = 2,           // NC[T]HW output, first `cout` channels
  kModeTimeInterleave = 3,  // causal temporal upsample frame layout, halo push
  kModeBandSplit = 4,       // band-layout output stored as bf16 parts [hi (cout) | lo (cout)]
                            // (+bias, +residual), halo push; the operand of a split-input conv
};

struct ConvArgs {
  const void* x;        // input band buffer
  const void* w;        // packed weights [cout_pad][taps][cin]
  const float* bias;    // [cout_pad] fp32
  const void* res;      // fp32 residual, output layout (nullable)
  void* y;              // fp32 output (band buffer, or final tensor for kModeFinal)
  void* q;              // kModeQKV: Q [n_img][tokens][c]
  void* k;              //           K [n_img][tokens][c]
  void* vt;             //           V^T [n_img][c][tokens]
  BandLayout in;
  BandLayout out;       // output layout (kModeBand / kModeTimeInterleave)
  int cin;              // == in.C
  int cout;             // true output channels
  int cout_pad;         // rows of the packed weight
  int kt, ks;           // temporal taps (1 or 3, causal), spatial kernel (1 or 3)
  int ups;              // nearest-2x fused into the load
  int down;             // stride 2 (3x3, input zero-padded by one row / column at the bottom /
                        // right only): output rows and width are half the input's
  int mode;
  int x_f32;            // bf16 path: operand source stored as fp32 (rounded on load)
  int x_split;          // bf16 path: operand source stored as bf16 [hi | lo] parts, channel
                        // stride in.C = 2 * cin (written by a kModeBandSplit conv)
  int sub;              // nearest-2x + 3x3 conv in sub-pixel form: w holds the phase-folded
                        // weights of launch_fold_subpixel_weight; needs x_split
  const int* sub_scale; // sub: the fp8 products' MFMA scale (launch_fold_subpixel_weight)
  int split8;           // kModeBandSplit output in the sub-pixel operand encoding (split8.h)
                        // instead of bf16 [hi | lo]
  const void* x2;       // wide kernel, kModeBand: a second bf16 operand in the input's band
  int cin2;             // geometry with cin2 channels, read at the output pixel itself (a 1x1
                        // conv folded in: K grows by cin2, its weights follow the taps' in
                        // every packed row); NULL / 0 for none
  const float* x_norm;  // bf16 path, tile128 kernel, kModeBand 3x3 convs: the input is the raw
  int x_norm_act;       // fp32 output of the previous conv and a GroupNorm apply is folded into
                        // the operand load -- x * scale_c + shift_c (SiLU when x_norm_act) with
                        // x_norm = [n_img][cin][2] (scale, shift) per image and channel, taps
                        // outside the image reading zero; NULL for none
  int final_frames;     // kModeFinal: frames per sample of the output tensor
  int out_transposed;   // kModeFinal: the bands cut the output's columns -- band-layout row g,
                        // column c is output pixel (row c, column g) of an in.W x in.H image
  int tiles_total;      // M tiles over all bands
  int tile_start[kMaxBands + 1];  // prefix of M tiles per band
  int kernel_used;      // set by the launch: VAEP_KERNEL_*
  // GroupNorm statistics of the output for the norm that consumes it (kModeBand /
  // kModeBandSplit).  The caller sets gn_part (fp64 tile records, [n_img][gn_groups][tiles
  // of one image][2] mean and M2) and gn_groups; the launch keeps gn_part only if the kernel it picks forms
  // the records in its epilogue (pixel tiles of whole rows), sets gn_chunk to the tile
  // width in pixels, and else clears gn_part and gn_chunk.  Tile index:
  // (image * out.H + row) * (out.W / gn_chunk) + column / gn_chunk.
  double* gn_part;
  int gn_groups;
  int gn_chunk;
};

// Launch the convolution described by `a` (fills tile fields).  dtype: VAEP_DTYPE_*.
hipError_t launch_conv(ConvArgs& a, int dtype, hipStream_t s);
// Pixel tile of the MFMA kernel along M and output-channel tile along N.
constexpr int kConvTileM = 128;
constexpr int kConvTileN = 128;
// Workgroup tile of the wide kernel, output channels x pixels: 256 x 256, 128 x 256 or
// 128 x 512.
struct WideTile {
  int bm, bn;
};
WideTile wide_tile(const ConvArgs& a);
// Whether the wide kernel runs the conv described by `a` (bf16 path): K in steps of 64
// channels, output channels a multiple of 128, band-layout epilogues.  Sub-pixel convs
// always run there.
bool conv_wide_fits(const ConvArgs& a);
// Whether launch_conv runs the conv described by `a` on the tile128 kernel with a folded
// GroupNorm apply (a.x_norm set): the shape it would run there anyway unfolded, 3x3, band
// mode, 64-channel K steps, cin <= 512, every band's pixels a multiple of the 128-pixel tile.
bool conv_norm_fold_ok(const ConvArgs& a);
hipError_t launch_conv_wide(ConvArgs& a, hipStream_t s);
// Plain 3x3 convs on the halo-tile kernel (conv_halo.hip): 4-row pixel tiles aligned to
// global rows, the pixel operand staged once per 32-channel block.
bool conv_halo_fits(const ConvArgs& a);
hipError_t launch_conv_halo(ConvArgs& a, hipStream_t s);
// The final conv (kModeFinal) with at most 16 output channels: pixels on the MFMA rows.
bool conv_narrow_fits(const ConvArgs& a);
hipError_t launch_conv_narrow(ConvArgs& a, hipStream_t s);
// Phase-folded weights of a nearest-2x + 3x3 conv: src [co][ci][3][3] bf16 ->
// dst [4 phases][co_pad][4 taps][4 ci bytes in the weight encoding of split8.h]; zero rows
// past co; ci a multiple of 64.  scale: 2 ints of device memory: the untransposed fold
// stores the largest |w| at scale[1] and the MFMA scale of the fp8 products at scale[0]
// (run it first).  transposed: fold the transposed 3x3 kernel (decodes on the
// transposed image).
hipError_t launch_fold_subpixel_weight(const void* src, int co, int ci, void* dst, int co_pad, int* scale,
                                       hipStream_t s, bool transposed = false);
// fp32 band buffer (channels C, a multiple of 64) -> the sub-pixel operand encoding of
// split8.h (4C bytes per pixel, C bf16 elements of channel stride 2C), halo rows included.
hipError_t launch_split(const float* src, const BandLayout& L, void* dst, hipStream_t s);
// out[i] = a[i] + b[i], i < n (fp32 device arrays).
hipError_t launch_add_f32(const float* a, const float* b, float* out, int n, hipStream_t s);

// ------------------------------------------------------------------ norms
// Local moments per (band, image, group): partial records of tiles, merged per band and
// then across bands with the element-count-weighted merge.
struct NormArgs {
  const void* x;         // fp32 input (conv outputs are fp32 in every configuration), or
                         // with x_split its bf16 hi / lo halves (2C channels per pixel)
  int x_split;
  void* y;               // output in the operand dtype
  BandLayout L;
  int groups;
  float eps;
  const float* gamma;
  const float* beta;
  int act;               // SiLU after the affine
  double* partials;      // [n_img][groups][blocks of one image][2] fp64 (mean, M2) of each
                         // stats block, then scratch
  float* band_moments;   // [3][nb][n_img*groups] count, mean, var (device scratch)
  int want_band_moments; // GroupNorm: also fill band_moments (each band's own tiles merged)
  float* coef_out;       // GroupNorm: the apply's per-(image, channel) (scale, shift) go here
                         // ([n_img][C][2]) instead of into the scratch (NULL: scratch)
  int stats_only;         // GroupNorm: stop after the merge (the apply is folded into the
                         // next conv, which reads coef_out)
  float* stats;          // [2][n_img*groups] merged mean, rstd
  float* merged_out;     // optional [2][n_img*groups] merged mean, var
  // GroupNorm statistics tiles.  The image is cut into slabs of `slab_rows` rows (the
  // finest row unit any band table of this layer can own: 2^level rows of a decode, one
  // row for a single step); a slab is split into chunks of `chunk_pix` pixels.  The tile
  // set depends only on the image, never on where the bands cut it.
  int slab_rows;
  int slabs;             // slabs per image = H / slab_rows
  int chunks;            // chunks per slab
  int chunk_pix;         // pixels per chunk (last chunk of a slab may be shorter)
  int apply_pix;         // pixels per apply workgroup
  // > 0: the producing conv already wrote the tile records into `partials` (one-row slabs,
  // chunks of pre_chunk pixels, see ConvArgs::gn_part); the statistics pass is skipped.
  int pre_chunk;
  long long item_start[kMaxBands + 1];  // apply pass: first vector (GN) / pixel (RMS) of band i
};

// Scratch of a GroupNorm launch in floats; slab_rows as in NormArgs; chunk > 0: tile
// records of `chunk` pixels of one row (statistics formed by the producing conv).
size_t gn_partials_floats(const BandLayout& L, int groups, int slab_rows, int chunk = 0);
hipError_t launch_groupnorm(NormArgs& a, int dtype, hipStream_t s);
hipError_t launch_rmsnorm(NormArgs& a, int dtype, hipStream_t s);
hipError_t launch_moment_merge(int n_shards, int n_stats, const float* mean, const float* var,
                               const int64_t* counts, float* mean_out, float* var_out,
                               hipStream_t s);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  const void* q;    // [n_img][tokens][c]
  const void* k;    // [n_img][tokens][c]
  const void* vt;   // [n_img][c][tokens]
  void* o;          // band layout output, c channels
  BandLayout L;     // layout of o (band rows, image = attention span)
  int c;
  int tokens;       // H * W of one span
  float scale;
  int tiles_total;
  int tile_start[kMaxBands + 1];  // query tiles per band (per image)
  float* part;      // bf16 path: scratch of attn_part_floats() for the key-split form, or
                    // NULL; the launch clears it where the split does not pay
};
// Scratch floats of the key-split attention: two halves of unnormalised O and (max, sum).
inline long long attn_part_floats(int n_img, int tokens, int c) { return 2LL * n_img * tokens * (c + 2); }
hipError_t launch_attention(AttnArgs& a, int dtype, hipStream_t s);
// The LDS-staged bf16 kernel for d = 384 and 512 (128 queries per workgroup, tile_start
// counted in such blocks; grid doubled when a.part splits the keys).  Tokens % 8 == 0.
hipError_t launch_attn_lds(const AttnArgs& a, unsigned grid, hipStream_t s);

// ------------------------------------------------------------------ data movement
// NC[T]HW tensor -> band layout (halo rows filled from neighbours, zeros at image
// edges, channels >= c_src zero).  n_img = B*T.  transposed: the bands cut the source's
// columns -- layout row g, column c reads source pixel (row c, column g) of an L.W x L.H
// image.
hipError_t launch_pack(const void* src, int c_src, void* dst, const BandLayout& L, int dtype,
                       hipStream_t s, bool transposed = false);
// band layout -> NC[T]HW tensor with c_dst channels.
hipError_t launch_unpack(const void* src, const BandLayout& L, void* dst, int c_dst, int dtype,
                         hipStream_t s);
// Copy frame 0 of every sample of `src` (frames T) to frame 0 of `dst` (frames 2T-1),
// halo rows included.
// Debug: fill every halo slot of a band buffer (elements of elem_bytes = 2 or 4) with 0xFF
// bytes (NaN in every float format the buffers hold).
hipError_t launch_poison_halos(void* buf, const BandLayout& L, int elem_bytes, hipStream_t s);
hipError_t launch_copy_frame0(const void* src, const BandLayout& Ls, void* dst,
                              const BandLayout& Ld, int dtype, hipStream_t s);
// Conv weight [co][ci][taps] (dtype) -> [co_pad][taps][rep * ci_pad] (dtype), zero padded;
// rep = 2 repeats the input channels for an operand stored as bf16 hi / lo halves.
// transposed (3x3 spatial taps only, taps = kt * 9): packed tap (dt, a, b) takes source
// tap (dt, b, a), the kernel of the same conv on the transposed image.
hipError_t launch_pack_weight(const void* src, int co, int ci, int taps, void* dst, int co_pad,
                              int ci_pad, int dtype, hipStream_t s, int rep = 1, bool transposed = false);
// Any-dtype vector -> fp32 vector of n_pad entries (zero padded); src may be NULL (zeros).
hipError_t launch_to_f32(const void* src, int n, float* dst, int n_pad, int dtype, hipStream_t s);

// Slot of tile (gi, gj) of a tiled decode: the full-size tiles (gi < full_r, gj < full_c)
// first in raster order (they decode as one batch), then the clipped edge tiles in raster
// order.
__host__ __device__ inline int tile_slot(int gi, int gj, int nc, int full_r, int full_c) {
  if (gi < full_r && gj < full_c) return gi * full_c + gj;
  const int before = (gi < full_r ? gi : full_r) * (nc - full_c) + (gi > full_r ? gi - full_r : 0) * nc;
  return full_r * full_c + before + (gi < full_r ? gj - full_c : gj);
}

// Tiled decode (overlap-blending baseline).  crop: rows [i, i+th), columns [j, j+tw) of
// each of `planes` h x w planes -> contiguous [planes][th][tw] (dtype).  blend: linear
// cross-fade of the first e rows (axis 0) / columns (axis 1) of an fp32 [planes][th][tw]
// tile from the last ones of its neighbour (nb_len rows / columns), in place.  gather:
// the merged output from the tile slots (see movement.hip).
hipError_t launch_crop(const void* src, long long planes, int h, int w, int i, int j, int th, int tw, void* dst,
                       int dtype, hipStream_t s);
hipError_t launch_blend(const float* nb, float* tile, long long planes, int th, int tw, int nb_len, int e, int axis,
                        hipStream_t s);
hipError_t launch_tiles_gather(const float* slots, long long slot_elems, long long planes, int H, int W, int keep,
                               int tile_out, int nc, int full_r, int full_c, int lat_h, int lat_w, int stride, int up,
                               float* out, hipStream_t s);

inline size_t dtype_bytes(int dtype) { return dtype == VAEP_DTYPE_F32 ? 4 : 2; }

// Set the thread's vaep_last_error() text and return `code`.
int set_error(int code, const char* msg);

}  // namespace vaep
