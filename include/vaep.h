/*
 * vaep.h -- C ABI of the layer-wise, spatially sharded VAE decoder for MI355X (gfx950).
 *
 * The method (ChituDiffusion, "VAEP: VAE 并行解码", sections on height sharding,
 * conv halos, the GroupNorm merge and AGKV; and "Static Layer-Wise VAE Decode",
 * "Semantics and Communication" operator table):
 *   - the latent is split along its height into disjoint row bands, which may be
 *     uneven; every band keeps all channels, the full width and the whole time axis,
 *     and its rows double with every 2x upsample;
 *   - a convolution reads kernel-radius halo rows from the neighbouring bands, with
 *     zero padding only at the global image edges, and keeps only its own output rows;
 *   - GroupNorm computes local FP32 central moments per (sample, group) and merges them
 *     with actual-element-count weights;
 *   - attention computes Q, K, V locally and runs each band's Q against the global K/V;
 *   - activations, pointwise ops, channel RMSNorm and nearest upsampling stay local;
 *   - the decoded rows of every band land in one output (the leader's).
 * On one GPU every band is a share of this device: halo rows, statistics and K/V pass
 * through device memory; there are no collectives.  vaep_decode_sharded cuts latent
 * columns instead (the width-sharded mode of the distributed-VAE strategy page) or lets
 * the per-request `auto` policy choose the axis.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers owned by the caller, unless a
 *     function says otherwise.  Host pointers are read before the call returns.
 *   - All GPU work is enqueued on the caller's stream (a hipStream_t passed as void*;
 *     NULL = the default stream); the caller keeps device buffers alive until the
 *     stream has finished.  No entry point synchronises the stream, except
 *     vaep_model_create (see there).
 *   - Return value: VAEP_OK (0) on success, a positive warning code on success with a
 *     warning, or a negative error code; vaep_last_error() describes the failure.
 *     Argument, shape, band-table and workspace errors (INVALID_ARG, UNSUPPORTED,
 *     WORKSPACE, NOT_READY) are found before anything is enqueued: nothing has run and
 *     output buffers are untouched.  VAEP_ERR_HIP reports a HIP call that failed while
 *     work was being enqueued (a kernel launch the runtime or a kernel's own launch
 *     checks refused, such as a band buffer whose rows exceed a buffer resource's
 *     range); earlier layers of that call may already be enqueued and the output is
 *     then undefined.
 *   - No C++ exception crosses this boundary.
 */
#ifndef VAEP_H
#define VAEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status codes */
enum {
  VAEP_OK = 0,
  VAEP_WARN_FELL_BACK = 1,      /* decoded, but as one dense band (see vaep_decode_bands) */
  VAEP_ERR_INVALID_ARG = -1,    /* bad pointer, shape, band table or size */
  VAEP_ERR_UNSUPPORTED = -2,    /* configuration outside what the library implements */
  VAEP_ERR_WORKSPACE = -3,      /* workspace missing or smaller than vaep_workspace_bytes */
  VAEP_ERR_HIP = -4,            /* a HIP runtime call failed */
  VAEP_ERR_NOT_READY = -5       /* no usable gfx950 device */
};

enum { VAEP_FAMILY_KL2D = 1,    /* AutoencoderKL-style 2-D decoder (GroupNorm) */
       VAEP_FAMILY_WAN3D = 2 }; /* Wan-style causal 3-D video decoder (channel RMSNorm) */
/* Storage policy.  Convolution / projection outputs -- the residual stream, conv1
 * outputs, shortcuts and the decoded image -- are fp32 in every configuration (the
 * fp32 accumulator is stored as is).  The compute dtype is that of the weights, the
 * latent, and the operands of the matrix products: normalised (norm + SiLU)
 * activations and the attention Q, K, V and attention output.  Statistics are fp32
 * (band moments are accumulated and merged in fp64, then rounded once). */
enum { VAEP_DTYPE_F32 = 1,      /* fp32 everywhere */
       VAEP_DTYPE_BF16 = 2 };   /* bf16 weights, latent and matrix-product operands */

#define VAEP_MAX_STAGES 6
#define VAEP_MAX_BANDS 64

/* Decoder description.  Stage i (decode order) ends with `resnets_per_stage` resnets
 * whose first maps the previous width to stage_channels[i]; every stage but the last
 * is followed by nearest-2x + 3x3 conv; for WAN3D the first `temporal_up_stages`
 * of those also run the causal temporal upsample (T -> 2T-1) before it. */
typedef struct vaep_config {
  int32_t family;                           /* VAEP_FAMILY_* */
  int32_t dtype;                            /* VAEP_DTYPE_* */
  int32_t z_channels;                       /* latent channels */
  int32_t n_stages;                         /* 1 .. VAEP_MAX_STAGES */
  int32_t stage_channels[VAEP_MAX_STAGES];  /* output width of each up stage (<= 1024) */
  int32_t resnets_per_stage;
  int32_t norm_groups;                      /* GroupNorm groups (KL2D); 0 for WAN3D */
  int32_t temporal_up_stages;               /* WAN3D only */
  float eps;                                /* norm epsilon */
} vaep_config;

/* Shard axes and strategies (vaep_decode_sharded, vaep_select_axis, vaep_decode_info.axis). */
enum { VAEP_AXIS_AUTO = 0,     /* pick per request (vaep_select_axis) */
       VAEP_AXIS_HEIGHT = 1,   /* bands of latent rows */
       VAEP_AXIS_WIDTH = 2,    /* bands of latent columns */
       VAEP_AXIS_DENSE = 3,    /* result only: one dense band */
       VAEP_AXIS_TILE = 4 };   /* the overlap-blending tile decode (vaep_decode_tiled) */

/* Optional report filled by the decode entry points. */
typedef struct vaep_decode_info {
  int32_t bands_used;        /* number of bands actually decoded */
  int32_t fell_back;         /* 1 if a fallback replaced the request: the dense one-band path
                                (vaep_decode_bands) or the tile decode (vaep_decode_sharded) */
  int32_t n_launches;        /* kernels enqueued by the call */
  int32_t axis;              /* VAEP_AXIS_HEIGHT / _WIDTH of the bands, _DENSE, or _TILE (then
                                bands_used is the number of tiles) */
  uint64_t workspace_bytes;  /* bytes of the workspace the call used */
} vaep_decode_info;

typedef struct vaep_model vaep_model;  /* opaque; owned by the library */

/* Thread-local text of the last error on this thread ("" if none).  Never NULL. */
const char* vaep_last_error(void);

/* Library version string, e.g. "vaep 0.1 gfx950". */
const char* vaep_version(void);

/* Fill *out with preset `id`: 1 tiny KL2D fp32 (4ch 8x8 latent, widths 64/32, GN 8);
 * 2-4 FLUX.1-style KL2D bf16 (16ch latent, widths 512/512/256/128, 3 resnets, GN 32);
 * 5 Wan-style WAN3D bf16 (16ch latent, widths 384/384/192/96, 2 resnets, RMSNorm,
 * 2 temporal upsample stages).  Presets 2-4 share the decoder and differ only in the
 * latent the caller decodes.  Returns VAEP_ERR_INVALID_ARG for other ids. */
int vaep_config_preset(int id, vaep_config* out);

/* Canonical parameter list of a decoder.  vaep_param_count returns the number of
 * parameter tensors (or a negative error).  vaep_param_info writes the name of
 * parameter j (NUL-terminated, truncated to name_cap), its PyTorch-style shape
 * (conv weight [Co, Ci, (kt,) kh, kw], linear weight [Co, Ci], bias/norm [C]) into
 * shape[0..*ndim-1] (at most 5 dims) and returns VAEP_OK. */
int vaep_param_count(const vaep_config* cfg);
int vaep_param_info(const vaep_config* cfg, int j, char* name, int name_cap,
                    int64_t shape[5], int* ndim);

/* Build a decoder.  params[j] is a device pointer to parameter j in canonical order,
 * contiguous, in the config's dtype.  The library copies and repacks every parameter
 * into memory it owns (one hipMalloc), so the caller may free params once this
 * returns; this call synchronises `stream` before returning.  *out receives the model.
 * Errors: INVALID_ARG (NULL pointers, n_params mismatch, channel counts that are not
 * multiples of 32 where the kernels need it), UNSUPPORTED, HIP, NOT_READY. */
int vaep_model_create(const vaep_config* cfg, const void* const* params, int n_params,
                      void* stream, vaep_model** out);

/* Release a model and its device memory.  The caller must have finished every
 * stream that uses it.  NULL is accepted (no-op). */
int vaep_model_destroy(vaep_model* model);

/* Fold the GroupNorm apply (scale, shift, SiLU) of the resnet convs into the conv's
 * operand load where the convolution kernel that runs the conv supports it (3x3 convs on
 * the 128 x 128-pixel-tile kernel: at most 512 input channels, every band's pixel count a
 * multiple of 128), instead of a separate pass that writes the normalised operand.  The
 * GroupNorm statistics and their merge are unchanged (ChituDiffusion "VAEP" feature page,
 * GroupNorm section; "Static Layer-Wise VAE Decode", GroupNorm row: merged statistics,
 * then the local normalisation); the folded apply computes the same operand bits, so the
 * decoded output is the same.  on: 0 (default) or 1.  Affects later decodes of `model`;
 * the workspace size does not depend on it.  Errors: INVALID_ARG (NULL model). */
int vaep_model_set_norm_fold(vaep_model* model, int on);

/* Debug mode for the halo exchange.  Before each layer writes a band buffer (conv, norm
 * and attention outputs), every halo slot of that buffer -- the row above and below each
 * band, per image -- is filled with 0xFF bytes, which is NaN in every float format the
 * buffers hold.  A layer's halo rows must come from its neighbours' boundary rows
 * (ChituDiffusion "VAEP" feature page, convolution section: the halo rows exchanged before
 * each conv; "Static Layer-Wise VAE Decode", operator table, "Spatial convolution" row), and
 * slots past the image edge must never be read (they stand for zero padding); a slot read
 * before its push, or an edge slot read at all, turns outputs into NaN.  A decode that is
 * correct gives the same bits with or without it.  Costs one fill kernel per such layer.
 * on: 0 (default) or 1.  Affects later decodes of `model`.  Errors: INVALID_ARG (NULL model). */
int vaep_model_set_halo_poison(vaep_model* model, int on);

/* Workspace needed to decode a latent of `batch` x [frames x] latent_h x latent_w
 * with up to `n_bands` bands (frames = 1 for KL2D).  The same size serves
 * vaep_decode_full, every band table with at most n_bands bands, and
 * vaep_decode_sharded with at most n_bands shards on either axis. */
int vaep_workspace_bytes(const vaep_model* model, int batch, int frames, int latent_h,
                         int latent_w, int n_bands, size_t* bytes_out);

/* Full-image decode: identical to vaep_decode_bands with the single band {0, latent_h}.
 * latent: device, contiguous (batch, z_channels, [frames,] latent_h, latent_w), in the
 *         config's dtype.
 * out:    device, contiguous fp32 (batch, 3, [frames_out,] 2^(n_stages-1)*latent_h,
 *         2^(n_stages-1)*latent_w), frames_out = frames doubled-minus-one per
 *         temporal upsample stage.
 * ws:     device workspace of ws_bytes >= vaep_workspace_bytes(model, ..., 1). */
int vaep_decode_full(vaep_model* model, const void* latent, int batch, int frames,
                     int latent_h, int latent_w, void* out, void* ws, size_t ws_bytes,
                     void* stream);

/* Band decode -- the layer-wise decode of the feature page ("VAEP: VAE 并行解码",
 * sections on height bands, conv halo exchange, the GroupNorm statistics merge and AGKV
 * attention) with the operator semantics of the validation page ("Static Layer-Wise VAE
 * Decode", "Semantics and Communication").  row_starts: host array of n_bands+1 latent
 * row indices with row_starts[0] = 0 < row_starts[1] < ... < row_starts[n_bands] =
 * latent_h; band i owns latent rows [row_starts[i], row_starts[i+1]) and the matching
 * output rows scaled by 2^(n_stages-1) (uneven bands allowed: the feature page keeps
 * uneven lengths throughout the decode).  Every layer runs on all bands; convs read one
 * halo row from each neighbour band (the 3x3 kernels' radius), so every band must own
 * at least one row.  A table with more than VAEP_MAX_BANDS bands is decoded as one dense
 * band and VAEP_WARN_FELL_BACK is returned (the pages' warn-and-dense fallback for
 * ineligible requests: feature page, usage and validation scope; validation page,
 * eligibility).  Other arguments as for vaep_decode_full; info (nullable) receives a
 * report.
 * Errors: INVALID_ARG (non-monotonic, zero-length or uncovered bands, NULL pointers),
 * WORKSPACE, HIP. */
int vaep_decode_bands(vaep_model* model, const void* latent, int batch, int frames,
                      int latent_h, int latent_w, const int32_t* row_starts, int n_bands,
                      void* out, void* ws, size_t ws_bytes, void* stream,
                      vaep_decode_info* info);

/* Band decode that allocates nothing, for callers that cannot call hipMalloc or hold a
 * workspace of their own (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, kernels, results and errors as
 * vaep_decode_bands, without ws / ws_bytes: the workspace is a static device array of
 * vaep_noalloc_scratch_bytes() bytes (64 MiB) that every GPU the library runs on holds
 * until the process ends.  A decode whose workspace (vaep_workspace_bytes) exceeds it is
 * rejected with VAEP_ERR_WORKSPACE before anything is enqueued.  The array is shared by
 * every call on a GPU: calls that overlap on one GPU (other streams, other threads) race,
 * so serialise them.  The first call on a device looks up the array's device address
 * (hipGetSymbolAddress) and keeps it; no call allocates or frees device memory. */
size_t vaep_noalloc_scratch_bytes(void);
int vaep_decode_bands_noalloc(vaep_model* model, const void* latent, int batch, int frames,
                              int latent_h, int latent_w, const int32_t* row_starts,
                              int n_bands, void* out, void* stream, vaep_decode_info* info);

/* Axis policy of a sharded decode (the distributed-VAE strategy page, "Strategy
 * Selection Contract" and the Wan spatial-shard notes: `auto` takes the longer axis
 * that can cover every shard, width winning ties, and uses the tile decode when neither
 * can).  A shard needs at least one latent row or column (the 3x3 kernels' radius at
 * latent resolution), so an axis covers n_shards when its length is >= n_shards.  Writes
 * VAEP_AXIS_HEIGHT, VAEP_AXIS_WIDTH, VAEP_AXIS_TILE (neither axis covers) or
 * VAEP_AXIS_DENSE (n_shards = 1) to *axis_out.  Host only: touches no device.
 * Deterministic and free of state.
 * Errors: INVALID_ARG (NULL axis_out, sizes < 1). */
int vaep_select_axis(int latent_h, int latent_w, int n_shards, int32_t* axis_out);

/* Sharded decode with a chosen strategy (strategy page, "Strategy Selection Contract":
 * tile, auto, forced height or forced width, decided per request).
 * axis = VAEP_AXIS_HEIGHT: bands of latent rows, exactly vaep_decode_bands.
 * axis = VAEP_AXIS_WIDTH: bands of latent columns; every rule of the band decode holds
 *   with rows and columns exchanged (convs read one halo column from each neighbour
 *   band, zero padding at the global edges; GroupNorm merges the bands' moments;
 *   attention runs each band's queries against the K/V of every band).  Internally the
 *   decode runs on the transposed image with transposed 3x3 kernels (built by
 *   vaep_model_create); latent and output keep their NC[T]HW layout.
 * axis = VAEP_AXIS_TILE: the tile decode of vaep_decode_tiled with latent tiles of 32
 *   rows and columns every 24; starts must be NULL and n_shards is not used.
 * axis = VAEP_AXIS_AUTO: vaep_select_axis picks the strategy; starts must be NULL.
 * starts: host array of n_shards+1 indices along the axis (0 = starts[0] < ... <
 *   starts[n_shards] = axis length), or NULL for even shards (sizes differ by at most
 *   one, larger shards first).
 * Fallback (the contract's "ineligible request" column): an explicit axis with NULL
 *   starts that is shorter than n_shards, or more than VAEP_MAX_BANDS shards, uses the
 *   tile decode and returns VAEP_WARN_FELL_BACK; `auto` with neither axis covering, or
 *   with more than VAEP_MAX_BANDS shards, uses the tile decode and returns VAEP_OK.  In
 *   both cases info->axis = VAEP_AXIS_TILE and info->fell_back = 1.
 * Workspace: ws >= vaep_workspace_bytes(..., n_shards) for band decodes; a request that
 *   runs the tile decode needs vaep_sharded_workspace_bytes(..., n_shards), which covers
 *   every outcome (with less it returns VAEP_ERR_WORKSPACE before enqueuing anything).
 * Other arguments as for vaep_decode_bands.
 * Errors: INVALID_ARG (unknown axis, starts with AUTO or TILE, bad table, NULL pointers),
 * WORKSPACE, HIP. */
int vaep_decode_sharded(vaep_model* model, const void* latent, int batch, int frames,
                        int latent_h, int latent_w, int axis, const int32_t* starts,
                        int n_shards, void* out, void* ws, size_t ws_bytes, void* stream,
                        vaep_decode_info* info);

/* Workspace that serves every outcome of vaep_decode_sharded with at most n_shards
 * shards: the larger of vaep_workspace_bytes(..., n_shards) and the tile decode's
 * vaep_tiled_workspace_bytes at its tile geometry.  Errors as vaep_workspace_bytes. */
int vaep_sharded_workspace_bytes(const vaep_model* model, int batch, int frames, int latent_h,
                                 int latent_w, int n_shards, size_t* bytes_out);

/* Tiled decode with overlap blending -- the comparison baseline the sharded decode
 * replaces (distributed-VAE strategy page, "Tile/Patch Implementation (Decode)"):
 * latent tiles of tile x tile rows and columns start every `stride` rows and columns
 * (clipped at the image edge); each is decoded on its own as a whole image (its own
 * GroupNorm statistics and attention tokens); the merge walks the tiles in raster order,
 * cross-fades each tile's first (tile - stride) * 2^(n_stages-1) output rows linearly
 * from its upper neighbour's last ones (weight of the neighbour 1 - k/e at row k of
 * e = min(neighbour rows, tile rows, overlap)), then its first columns from its left
 * neighbour likewise, keeps stride * 2^(n_stages-1) rows and columns of every tile and
 * crops to the image.  The blend is a reading (the page names it without printing it).
 * Unlike the band decodes this does not reproduce the full-image decode; it exists to be
 * measured against it (seams, time).  latent / out as for vaep_decode_full; ws of at
 * least vaep_tiled_workspace_bytes(...) bytes (it holds every decoded tile).
 * Errors: INVALID_ARG (1 <= stride <= tile violated, NULL pointers), WORKSPACE, HIP. */
int vaep_tiled_workspace_bytes(const vaep_model* model, int batch, int frames, int latent_h,
                               int latent_w, int tile, int stride, size_t* bytes_out);
int vaep_decode_tiled(vaep_model* model, const void* latent, int batch, int frames, int latent_h,
                      int latent_w, int tile, int stride, void* out, void* ws, size_t ws_bytes,
                      void* stream);

/* Tiled encode with overlap blending (distributed-VAE strategy page, "Tile/Patch Encode
 * Implementation": split the image into overlapping tiles, encode every tile on its own
 * -- the encoder, then quant_conv -- and merge the encoded tiles in latent space as the
 * tile decode merges decoded ones).  The page takes a video encoder as its example; this
 * library builds the encoder of the 2-D family (VAEP_FAMILY_KL2D configs), a reading:
 * the decoder's mirror -- conv_in from RGB to the narrowest width, down stages over the
 * reversed stage widths with resnets_per_stage - 1 resnets each (at least one) and, in
 * every stage but the last, a 3x3 stride-2 convolution over the input zero-padded by one
 * row at the bottom and one column at the right, the mid block (resnet, single-head
 * attention, resnet), GroupNorm -> SiLU -> conv_out to 2 z channels (mean | log-variance),
 * and a 1x1 quant_conv over those.  Same storage policy as the decoder: bf16 weights and
 * matrix-core operands, fp32 conv outputs, statistics and output. */
typedef struct vaep_encoder vaep_encoder;   /* opaque; owned by the library */

/* Number of encoder parameters of `cfg`, or a negative error (INVALID_ARG for a bad
 * config, UNSUPPORTED for a video config).  Canonical order, names and shapes as
 * vaep_param_info (weights [Co, Ci, kh, kw], linear weights [Co, Ci], biases [Co]). */
int vaep_encoder_param_count(const vaep_config* cfg);
int vaep_encoder_param_info(const vaep_config* cfg, int j, char* name, int name_cap, int64_t shape[5],
                            int* ndim);

/* Build an encoder (params as for vaep_model_create: device pointers in canonical order,
 * the config's dtype; copied and repacked, so the caller may free them once this returns;
 * synchronises `stream`).  Errors: INVALID_ARG, UNSUPPORTED (video config), HIP,
 * NOT_READY. */
int vaep_encoder_create(const vaep_config* cfg, const void* const* params, int n_params, void* stream,
                        vaep_encoder** out);
/* Release an encoder (the caller has finished every stream that uses it).  NULL is a no-op. */
int vaep_encoder_destroy(vaep_encoder* enc);

/* Workspace of vaep_encode_tiled for these arguments.  Errors as vaep_encode_tiled's
 * argument checks. */
int vaep_encode_tiled_workspace_bytes(const vaep_encoder* enc, int batch, int height, int width, int tile,
                                      int stride, size_t* bytes_out);

/* Encode `batch` images.
 * image: device, contiguous (batch, 3, height, width) in the config's dtype; height and
 *        width positive multiples of 2^(n_stages-1).
 * tile, stride: in latent pixels (image pixels / 2^(n_stages-1)); image tiles of
 *        tile * 2^(n_stages-1) pixels start every stride * 2^(n_stages-1) pixels (clipped at
 *        the edge); each is encoded as a whole image (its own GroupNorm statistics and
 *        attention tokens); the merge cross-fades each encoded tile's first tile - stride
 *        rows from its upper neighbour and then its first columns from its left neighbour
 *        (the linear blend of vaep_decode_tiled), keeps stride rows and columns of every
 *        tile and crops to the latent size.  One tile covering the image (tile >= both
 *        latent sides) is the whole-image encode.
 * out:   device, contiguous fp32 (batch, 2 z, height / 2^(n_stages-1), width / 2^(n_stages-1)).
 * ws:    device workspace of at least vaep_encode_tiled_workspace_bytes(...) bytes.
 * info (nullable): bands_used = number of tiles, axis = VAEP_AXIS_TILE, n_launches,
 *        workspace_bytes.
 * Errors: INVALID_ARG (NULL pointers, image sizes, 1 <= stride <= tile violated),
 * WORKSPACE (nothing enqueued), HIP (earlier work may remain enqueued). */
int vaep_encode_tiled(vaep_encoder* enc, const void* image, int batch, int height, int width, int tile,
                      int stride, void* out, void* ws, size_t ws_bytes, void* stream, vaep_decode_info* info);

/* Launch timing.  While profiling is on for a model, every kernel launch of its decodes
 * is bracketed by two HIP events on the caller's stream and the library records the
 * step's kind, shape and algorithmic work (each tensor counted once; convolution flops
 * 2*M*N*K with true channel counts; attention 4*Nq*Nk*C).  vaep_profile_begin creates
 * 2*max_launches events (host-side HIP objects, no device memory) and clears earlier
 * records; launches beyond max_launches are not recorded.  vaep_profile_end waits for
 * the recorded events, writes up to `cap` entries in launch order, sets *n_out to the
 * number recorded, turns profiling off and releases the events.  The events serialise
 * nothing beyond the caller's own stream order. */
enum { VAEP_STEP_CONV = 1, VAEP_STEP_GROUPNORM = 2, VAEP_STEP_RMSNORM = 3,
       VAEP_STEP_ATTENTION = 4, VAEP_STEP_MOVE = 5 };
/* Convolution kernel that ran a conv step: 128x128 tiles two per CU, the wide kernel
 * with 256 x 256, 128 x 256 or 128 x 512 (channels x pixels) tiles, the narrow-output
 * kernel, the fp32 kernel, the halo-tile kernel (2-D pixel tiles, the pixel operand
 * staged once per channel block), and the halo-tile kernel with a folded 1x1 second
 * operand (a resnet's shortcut run as extra K steps of its conv2). */
enum { VAEP_KERNEL_OTHER = 0, VAEP_KERNEL_CONV_TILE128 = 1, VAEP_KERNEL_CONV_WIDE256 = 2,
       VAEP_KERNEL_CONV_WIDE128 = 3, VAEP_KERNEL_CONV_NARROW = 4, VAEP_KERNEL_CONV_F32 = 5,
       VAEP_KERNEL_CONV_WIDE128X512 = 6, VAEP_KERNEL_CONV_HALO = 7, VAEP_KERNEL_CONV_HALO_X2 = 8 };
typedef struct vaep_profile_entry {
  int32_t step;        /* VAEP_STEP_* */
  int32_t n_kernels;   /* kernels inside the bracket */
  int32_t kt, ks;      /* conv: temporal taps and spatial kernel size */
  int32_t cin, cout;   /* conv: true input / output channels; norm and attention: channels */
  int32_t ups, mode;   /* conv: fused nearest-2x; epilogue mode (internal) */
  int64_t pixels;      /* conv: output pixels; norm: positions; attention: queries */
  double flops;        /* algorithmic flops */
  double bytes;        /* algorithmic HBM bytes */
  float ms;            /* time between the bracketing events */
  int32_t kernel;      /* conv: VAEP_KERNEL_* */
} vaep_profile_entry;
int vaep_profile_begin(vaep_model* model, int max_launches);
int vaep_profile_end(vaep_model* model, vaep_profile_entry* out, int cap, int* n_out);

/* GroupNorm statistics merge (feature page, GroupNorm section; validation page,
 * formula under the operator table): for each of n_stats (sample, group) entries,
 *   w_i  = counts[i][s] / sum_j counts[j][s]
 *   mean = sum_i w_i * local_mean[i][s]
 *   var  = sum_i w_i * (local_var[i][s] + (local_mean[i][s] - mean)^2)
 * All arrays are device, row-major [n_shards][n_stats]; local_var is the population
 * (divide-by-count) variance.  A shard whose count is 0 has weight 0.  Computed in fp32
 * with the shards in index order.  Errors: INVALID_ARG (NULL, n_shards < 1, n_stats < 0,
 * n_shards > 4096); an entry whose counts all are 0 yields mean = var = 0. */
int vaep_groupnorm_merge(int n_shards, int n_stats, const float* local_mean,
                         const float* local_var, const int64_t* counts, float* mean_out,
                         float* var_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VAEP_H */
