"""CPU oracle for the layer-wise, height-sharded VAE decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never calls it and shares no code with it; the two meet only through
the seeded inputs of the ``synth`` package.

What it computes follows the pages on the method:

* ChituDiffusion, "VAEP: VAE 并行解码" (feature page) -- sections on height
  sharding, conv halo exchange, the GroupNorm statistics merge and AGKV
  attention.
* ChituDiffusion, "Static Layer-Wise VAE Decode" (validation page) -- the
  "Semantics and Communication" operator table and the merge formula below it.
* The distributed-VAE strategy page -- "Strategy Selection Contract" and the
  Wan spatial-shard notes (height or width sharding, the ``auto`` axis
  policy), and the tile/patch decode (split / exec / merge with overlap
  blending), the comparison baseline in ``tiled.py``, and the tile/patch encode
  (``encoder.py``: the encoder of the 2-D presets on overlapping image tiles).

Both pages state that the layer-wise decode keeps full-image semantics, so the
oracle's primary output is the plain full-image decoder forward
(``decoder.decode_full``).  ``decoder.decode_bands`` is a separate band-mode
implementation (per-band buffers, halo rows fetched from neighbours, merged
statistics, global K/V) used to pin that invariant.

Arithmetic: every operator evaluates its definition in float64 (convolution
sums, moments, softmax); activations are stored as float32 between operators
and, in bf16 emulation mode, rounded to bfloat16 at each materialised tensor.

Parity status of every function is listed in ``oracle/PINS.md``.
"""
from .ops import (conv_padded, conv_full, conv_band, groupnorm_moments, merge_moments,
                  groupnorm_apply, rmsnorm, silu, attention_rows, upsample_nearest2x,
                  temporal_upsample_interleave, downsample_conv)
from .decoder import decode_full, decode_bands, decode_auto, choose_axis, even_starts, Precision
from .tiled import blend_h, blend_v, decode_tiled, row_seam, tile_origins
from .encoder import encode_full, encode_tiled

__all__ = [
    "conv_padded", "conv_full", "conv_band", "groupnorm_moments", "merge_moments",
    "groupnorm_apply", "rmsnorm", "silu", "attention_rows", "upsample_nearest2x",
    "temporal_upsample_interleave", "decode_full", "decode_bands", "decode_auto", "choose_axis",
    "even_starts", "Precision", "blend_h", "blend_v", "decode_tiled", "row_seam", "tile_origins",
    "downsample_conv", "encode_full", "encode_tiled",
]
