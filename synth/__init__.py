"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package holds only workload descriptions (decoder presets, band tables,
parameter lists) and a counter-based random generator.  It contains none of
the decoder's arithmetic: both sides receive the same latents and weights
from here and compute independently.
"""
from .configs import DecoderConfig, PRESETS, preset, param_specs, encoder_param_specs, ParamSpec
from .gen import (splitmix64, normal_draws, make_latent, make_params, make_encoder_params, make_image,
                  round_bf16)

__all__ = [
    "DecoderConfig", "PRESETS", "preset", "param_specs", "encoder_param_specs", "ParamSpec",
    "splitmix64", "normal_draws", "make_latent", "make_params", "make_encoder_params", "make_image",
    "round_bf16",
]
