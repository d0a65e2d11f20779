"""Layer-wise, spatially sharded VAE decode for MI355X (gfx950).

The decoder runs band by band on disjoint latent row bands (or column bands,
or the axis a per-request policy picks): convolutions read
halo rows from the neighbouring bands, GroupNorm merges per-band moments with
element-count weights, attention runs band-local queries against the global
K/V, and every kernel is hand-written HIP for gfx950 behind the C ABI of
``include/vaep.h`` (``libvaep.so``).  The same kernels also run the tiled encode
of the 2-D family (``Encoder``).  This package is the thin Python binding.
"""
from . import _lib
from .api import (Decoder, Encoder, encoder_param_info, config_preset, make_config, param_info,
                  groupnorm_merge, profile_begin,
                  profile_end, select_axis, step_conv,
                  step_groupnorm, step_rmsnorm, step_attention, step_temporal_upsample, version)

__all__ = [
    "_lib", "Decoder", "Encoder", "encoder_param_info", "config_preset", "make_config", "param_info",
    "groupnorm_merge",
    "profile_begin", "profile_end", "select_axis",
    "step_conv", "step_groupnorm", "step_rmsnorm", "step_attention", "step_temporal_upsample",
    "version",
]
