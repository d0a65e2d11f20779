"""Counter-based seeded generator for latents and weights.

Stream: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014).  Output i of the stream with seed s is
``mix(s + (i + 1) * 0x9E3779B97F4A7C15)`` with the published finaliser, so any
element can be computed directly from its index.

Normals: Box-Muller.  Normal k uses outputs 2k (a) and 2k+1 (b):
``u1 = ((a >> 11) + 0.5) * 2^-53``, ``u2 = (b >> 11) * 2^-53``,
``z = sqrt(-2 ln u1) * cos(2 pi u2)``, in double precision.

Weights of parameter j (canonical order) use seed ``0x5EED0000 + 1000*cfg + j``
and are ``z / sqrt(fan_in)``; biases are 0 and norm scales 1 / shifts 0 unless
``affine='random'`` asks for seeded non-trivial values (used by tests so that a
dropped bias or affine term cannot hide).  Latent sample b uses seed
``1000*cfg + b``.  For bf16 presets every value is rounded to the nearest
bfloat16 (ties to even) here, before either consumer sees it.
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from .configs import DecoderConfig, encoder_param_specs, param_specs

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start .. start+n-1 of the SplitMix64 stream seeded with ``seed``."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def normal_draws(seed: int, n: int) -> np.ndarray:
    """n standard normal doubles from the stream (Box-Muller, cosine branch)."""
    u = splitmix64(seed, 2 * n)
    a = u[0::2] >> np.uint64(11)
    b = u[1::2] >> np.uint64(11)
    u1 = (a.astype(np.float64) + 0.5) * (2.0 ** -53)
    u2 = b.astype(np.float64) * (2.0 ** -53)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def uniform_draws(seed: int, n: int) -> np.ndarray:
    """n doubles uniform in [0, 1) from the top 53 bits of the stream."""
    return (splitmix64(seed, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def round_bf16(x: torch.Tensor) -> torch.Tensor:
    """fp32 tensor whose values are rounded to the nearest bfloat16 (ties to even)."""
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float32)


def _finish(a: np.ndarray, shape, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a.astype(np.float32).reshape(shape))
    return round_bf16(t) if dtype == "bf16" else t


def make_latent(cfg: DecoderConfig, batch=None, frames=None, latent_h=None, latent_w=None,
                seed_base=None) -> torch.Tensor:
    """Latent (B, z, [T,] H, W) as fp32 (bf16-representable for bf16 presets)."""
    shape = cfg.latent_shape(batch, frames, latent_h, latent_w)
    base = 1000 * cfg.id if seed_base is None else seed_base
    per = int(np.prod(shape[1:]))
    parts = [normal_draws(base + b, per) for b in range(shape[0])]
    return _finish(np.concatenate(parts), shape, cfg.dtype)


def make_params(cfg: DecoderConfig, affine: str = "default", seed_base=None) -> Dict[str, torch.Tensor]:
    """Ordered dict name -> fp32 tensor for every parameter of ``cfg``'s decoder."""
    base = 0x5EED0000 + 1000 * cfg.id if seed_base is None else seed_base
    return _draw(param_specs(cfg), base, affine, cfg.dtype)


def make_encoder_params(cfg: DecoderConfig, affine: str = "default", seed_base=None) -> Dict[str, torch.Tensor]:
    """Ordered dict name -> fp32 tensor for every parameter of ``cfg``'s encoder (2-D presets);
    parameter j uses seed ``0x5EEE0000 + 1000*cfg + j``."""
    base = 0x5EEE0000 + 1000 * cfg.id if seed_base is None else seed_base
    return _draw(encoder_param_specs(cfg), base, affine, cfg.dtype)


def make_image(cfg: DecoderConfig, batch=None, latent_h=None, latent_w=None, seed_base=None) -> torch.Tensor:
    """Image (B, 3, H, W) for the encoder, uniform in [-1, 1) (the value range of a
    normalised RGB image); sample b uses seed ``1000*cfg + 500 + b``."""
    shape = cfg.image_shape(batch, latent_h, latent_w)
    base = 1000 * cfg.id + 500 if seed_base is None else seed_base
    per = int(np.prod(shape[1:]))
    parts = [2.0 * uniform_draws(base + b, per) - 1.0 for b in range(shape[0])]
    return _finish(np.concatenate(parts), shape, cfg.dtype)


def _draw(specs, base: int, affine: str, dtype: str) -> Dict[str, torch.Tensor]:
    out: Dict[str, torch.Tensor] = {}
    for j, p in enumerate(specs):
        n = int(np.prod(p.shape))
        if p.kind == "weight":
            a = normal_draws(base + j, n) / np.sqrt(p.fan_in)
        elif affine == "random":
            z = normal_draws(base + j, n)
            if p.kind == "gamma":
                a = 1.0 + 0.25 * z
            else:
                a = 0.1 * z
        elif p.kind == "gamma":
            a = np.ones(n)
        else:
            a = np.zeros(n)
        out[p.name] = _finish(a, p.shape, dtype)
    return out
