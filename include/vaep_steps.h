/*
 * vaep_steps.h -- single-step entry points of the layer-wise decode.
 *
 * Each call runs ONE step of the band-wise decode on every band of a caller-given
 * band table, with the same kernels and launch shapes vaep_decode_bands uses, so
 * that a step can be checked in isolation at its real layer shape.  Inputs and
 * outputs are whole tensors in PyTorch layout; the call scatters the input into the
 * library's per-band buffers (one halo row above and below each band), runs the
 * step band by band, and gathers the bands' own rows into the output.  Weights are
 * passed in PyTorch layout and repacked into the workspace on every call.
 *
 * Shared conventions (see vaep.h): device pointers are caller-owned; work goes on
 * `stream`; return VAEP_OK or a negative error with nothing enqueued.  Tensors are
 * contiguous.  `dtype` is the compute dtype (VAEP_DTYPE_F32 or VAEP_DTYPE_BF16) of
 * the weights and of normalised outputs; conv outputs, residuals and the inputs of
 * norms are fp32, as in vaep_decode_bands.  `frames` is 1 for
 * images; video tensors are (B, C, T, H, W) and images (B, C, H, W).  The band table
 * row_starts (host, n_bands+1 entries) partitions the INPUT rows as in
 * vaep_decode_bands.  ws/ws_bytes: device workspace of at least the size returned
 * through *bytes_out when ws is NULL (a size query: nothing is launched).
 */
#ifndef VAEP_STEPS_H
#define VAEP_STEPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Convolution step (feature page, conv section; validation page, "Spatial
 * convolution" row).  x is stored in x_dtype (fp32, or `dtype` for a normalised
 * activation); fp32 inputs are rounded to `dtype` as the matrix-core operand.
 * y and residual are fp32.  weight (in `dtype`): [cout, cin, kt, kh, kw] with kh = kw in {1, 3},
 * kt in {1, 3}; kt = 3 requires causal = 1 (two zero frames in front, none behind).
 * upsample = 1 applies nearest-2x to x first (fused into the conv's load): the output
 * is (B, cout, [T,] 2h, 2w), its bands own twice their input rows.  bias: [cout]
 * (nullable = 0).  residual (nullable): tensor of the output's shape added after the
 * bias.  y: output.  Halo rows come from the neighbour bands; rows outside the image
 * and columns outside [0, w) read as zero.  cin must be a multiple of 32 unless
 * dtype is F32; cout >= 1. */
int vaep_step_conv(int dtype, int x_dtype, const void* x, int batch, int frames, int cin, int h,
                   int w, const void* weight, const void* bias, int cout, int kt, int kh, int kw,
                   int causal, int upsample, const void* residual,
                   const int32_t* row_starts, int n_bands, void* y,
                   void* ws, size_t ws_bytes, size_t* bytes_out, void* stream);

/* GroupNorm step (feature page, GroupNorm section; validation page, "GroupNorm" row):
 * local fp32 central moments per (band, sample, group), the element-count-weighted
 * merge, then y = (x - mean) / sqrt(var + eps) * gamma + beta, followed by SiLU when
 * act = 1.  x: fp32; y: `dtype`.  gamma/beta: [c] fp32 (device).  band_moments (nullable, device fp32
 * [3][n_bands][batch*groups]): receives count, mean and variance of every band;
 * merged (nullable, device fp32 [2][batch*groups]): the merged mean and variance. */
int vaep_step_groupnorm(int dtype, const void* x, int batch, int frames, int c, int h,
                        int w, int groups, float eps, const float* gamma, const float* beta,
                        int act, const int32_t* row_starts, int n_bands, void* y,
                        float* band_moments, float* merged, void* ws, size_t ws_bytes,
                        size_t* bytes_out, void* stream);

/* Channel RMSNorm step (validation page, "Video temporal operations" row: channel
 * RMSNorm stays local): y_c = gamma_c * x_c / sqrt(mean_c x^2 + eps), then SiLU when
 * act = 1.  x: fp32; y: `dtype`; gamma: [c] fp32 (device). */
int vaep_step_rmsnorm(int dtype, const void* x, int batch, int frames, int c, int h, int w,
                      float eps, const float* gamma, int act, const int32_t* row_starts,
                      int n_bands, void* y, void* ws, size_t ws_bytes, size_t* bytes_out,
                      void* stream);

/* Attention step (feature page, AGKV section; validation page, "Attention" row):
 * h = norm(x) (GroupNorm with `groups` groups and merged statistics, or channel
 * RMSNorm when groups = 0), Q = h Wq^T + bq, K, V likewise, computed band-locally;
 * K and V of every band are written into one global K/V buffer; each band's Q attends
 * to the global K/V of its frame (single head, scale 1/sqrt(c)); then
 * y = x + O Wo^T + bo.  wq, wk, wv, wo: [c, c]; bq, bk, bv, bo: [c]; norm_gamma,
 * norm_beta: [c] fp32 (norm_beta ignored for RMSNorm).  x and y: fp32; weights in
 * `dtype`; Q, K, V and the attention output are held in `dtype`.  Attention spans one
 * frame (video) or the whole image. */
int vaep_step_attention(int dtype, const void* x, int batch, int frames, int c, int h,
                        int w, int groups, float eps, const float* norm_gamma,
                        const float* norm_beta, const void* wq, const void* bq,
                        const void* wk, const void* bk, const void* wv, const void* bv,
                        const void* wo, const void* bo, const int32_t* row_starts,
                        int n_bands, void* y, void* ws, size_t ws_bytes, size_t* bytes_out,
                        void* stream);

/* Causal temporal upsample step (Wan-style decoder, up stages with time upsampling):
 * z = causal (3,1,1) time conv of x from c to 2c channels (weight [2c, c, 3, 1, 1],
 * bias [2c]); output frame 0 = x frame 0, frame 2t-1 = z[t][0:c], frame 2t =
 * z[t][c:2c] for t >= 1.  x: fp32 (B, c, T, h, w); y: fp32 (B, c, 2T-1, h, w). */
int vaep_step_temporal_upsample(int dtype, const void* x, int batch, int frames, int c,
                                int h, int w, const void* weight, const void* bias,
                                const int32_t* row_starts, int n_bands, void* y, void* ws,
                                size_t ws_bytes, size_t* bytes_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VAEP_STEPS_H */
