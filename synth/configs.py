"""Decoder presets and the canonical parameter list.

The five presets are the synthetic stand-ins for the workloads the validation
page of the layer-wise decode measures (a FLUX.1 / Z-Image-style
AutoencoderKL decoder at 512^2 and 1024^2, and a Wan-style causal-3D video
decoder at 17x480x832), plus a tiny fp32 decoder.  Pretrained weights are not
available, so every preset is decoded with seeded random weights.

Channel plans follow the plainest reading of "AutoencoderKL decoder": a
conv_in to the widest channel count, a mid block (resnet, single-head
attention, resnet), up blocks over the reversed ``block_out_channels`` whose
first resnet changes the channel count, a nearest-2x + 3x3 conv after every
up block but the last, and GroupNorm -> SiLU -> conv_out to RGB.  The Wan
variant swaps GroupNorm for channel RMSNorm, 2D convs for causal 3x3x3 convs,
runs the mid attention per frame, and adds a causal temporal upsample in the
first ``temporal_up_stages`` up stages.

The 2-D presets also describe the encoder of the tiled encode (``encoder_param_specs``):
the decoder's mirror -- conv_in from RGB to the narrowest width, down stages over
``block_out_channels`` with one resnet fewer than the decoder's up stages (the
common AutoencoderKL layout: two per down block, three per up block) and a 3x3
stride-2 convolution after every stage but the last, the same mid block, then
GroupNorm -> SiLU -> conv_out to 2 x z channels (mean and log-variance) and a 1x1
``quant_conv`` over them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class DecoderConfig:
    id: int
    name: str
    family: str                 # "kl2d" or "wan3d"
    dtype: str                  # "f32" or "bf16" (storage of weights/activations)
    z_channels: int
    stage_channels: Tuple[int, ...]   # output channels of up stage 0..L-1 (decode order)
    resnets_per_stage: int
    norm_groups: int            # GroupNorm groups (kl2d); 0 for RMSNorm (wan3d)
    eps: float
    temporal_up_stages: int     # wan3d: stages whose upsample also doubles time
    batch: int
    frames: int                 # latent frames (1 for kl2d)
    latent_h: int
    latent_w: int
    band_starts: Tuple[int, ...]  # latent row boundaries s_0=0 < ... < s_n = H

    @property
    def top_channels(self) -> int:
        return self.stage_channels[0]

    @property
    def n_stages(self) -> int:
        return len(self.stage_channels)

    @property
    def is_video(self) -> bool:
        return self.family == "wan3d"

    def stage_upsamples(self, i: int) -> bool:
        return i < self.n_stages - 1

    def stage_time_upsamples(self, i: int) -> bool:
        return self.is_video and self.stage_upsamples(i) and i < self.temporal_up_stages

    def output_shape(self, batch: Optional[int] = None, frames: Optional[int] = None,
                     latent_h: Optional[int] = None, latent_w: Optional[int] = None):
        b = self.batch if batch is None else batch
        t = self.frames if frames is None else frames
        h = self.latent_h if latent_h is None else latent_h
        w = self.latent_w if latent_w is None else latent_w
        ups = self.n_stages - 1
        if self.is_video:
            for i in range(self.n_stages):
                if self.stage_time_upsamples(i):
                    t = 2 * t - 1
            return (b, 3, t, h << ups, w << ups)
        return (b, 3, h << ups, w << ups)

    def latent_shape(self, batch=None, frames=None, latent_h=None, latent_w=None):
        b = self.batch if batch is None else batch
        h = self.latent_h if latent_h is None else latent_h
        w = self.latent_w if latent_w is None else latent_w
        if self.is_video:
            t = self.frames if frames is None else frames
            return (b, self.z_channels, t, h, w)
        return (b, self.z_channels, h, w)

    @property
    def encoder_resnets(self) -> int:
        """Resnets per encoder down stage (2-D presets): one fewer than per decoder up stage."""
        return max(1, self.resnets_per_stage - 1)

    def image_shape(self, batch=None, latent_h=None, latent_w=None):
        """The image an encoder reads: (B, 3, H, W) at the decoder's output resolution."""
        b = self.batch if batch is None else batch
        h = self.latent_h if latent_h is None else latent_h
        w = self.latent_w if latent_w is None else latent_w
        ups = self.n_stages - 1
        return (b, 3, h << ups, w << ups)

    def moments_shape(self, batch=None, latent_h=None, latent_w=None):
        """The encoder's output: (B, 2 z, H / 2^(n_stages-1), W / 2^(n_stages-1)), mean | log-variance."""
        b = self.batch if batch is None else batch
        h = self.latent_h if latent_h is None else latent_h
        w = self.latent_w if latent_w is None else latent_w
        return (b, 2 * self.z_channels, h, w)

    def with_size(self, **kw) -> "DecoderConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return DecoderConfig(**d)


def _kl(id, name, dtype, z, block_out, resnets, groups, batch, h, w, starts):
    return DecoderConfig(id=id, name=name, family="kl2d", dtype=dtype, z_channels=z,
                         stage_channels=tuple(reversed(block_out)), resnets_per_stage=resnets,
                         norm_groups=groups, eps=1e-6, temporal_up_stages=0, batch=batch,
                         frames=1, latent_h=h, latent_w=w, band_starts=tuple(starts))


PRESETS = {
    1: _kl(1, "kl2d-tiny-f32-8x8", "f32", 4, (32, 64), 2, 8, 1, 8, 8, (0, 3, 8)),
    2: _kl(2, "kl2d-flux-bf16-64x64", "bf16", 16, (128, 256, 512, 512), 3, 32, 1, 64, 64,
           (0, 32, 64)),
    3: _kl(3, "kl2d-flux-bf16-128x128", "bf16", 16, (128, 256, 512, 512), 3, 32, 1, 128, 128,
           (0, 31, 64, 96, 128)),
    4: _kl(4, "kl2d-flux-bf16-4x128x128", "bf16", 16, (128, 256, 512, 512), 3, 32, 4, 128, 128,
           (0, 15, 32, 48, 64, 79, 96, 112, 128)),
    5: DecoderConfig(id=5, name="wan3d-bf16-5x60x104", family="wan3d", dtype="bf16",
                     z_channels=16, stage_channels=(384, 384, 192, 96), resnets_per_stage=2,
                     norm_groups=0, eps=1e-6, temporal_up_stages=2, batch=1, frames=5,
                     latent_h=60, latent_w=104, band_starts=(0, 14, 30, 45, 60)),
}


def preset(i: int) -> DecoderConfig:
    return PRESETS[i]


@dataclass(frozen=True)
class ParamSpec:
    name: str
    shape: Tuple[int, ...]
    kind: str           # "weight", "bias", "gamma", "beta"
    fan_in: int = 0


def _conv(name, co, ci, kernel):
    fan = ci
    for k in kernel:
        fan *= k
    return [ParamSpec(name + ".weight", (co, ci) + tuple(kernel), "weight", fan),
            ParamSpec(name + ".bias", (co,), "bias")]


def _lin(name, co, ci):
    return [ParamSpec(name + ".weight", (co, ci), "weight", ci),
            ParamSpec(name + ".bias", (co,), "bias")]


def _norm(name, c, video):
    if video:   # channel RMSNorm: scale only
        return [ParamSpec(name + ".weight", (c,), "gamma")]
    return [ParamSpec(name + ".weight", (c,), "gamma"), ParamSpec(name + ".bias", (c,), "beta")]


def _resnet_specs(out, prefix, ci, co, v):
    k3 = (3, 3, 3) if v else (3, 3)
    k1 = (1, 1, 1) if v else (1, 1)
    out.extend(_norm(prefix + ".norm1", ci, v))
    out.extend(_conv(prefix + ".conv1", co, ci, k3))
    out.extend(_norm(prefix + ".norm2", co, v))
    out.extend(_conv(prefix + ".conv2", co, co, k3))
    if ci != co:
        out.extend(_conv(prefix + ".shortcut", co, ci, k1))


def _mid_specs(out, c, v):
    _resnet_specs(out, "mid.res0", c, c, v)
    out.extend(_norm("mid.attn.norm", c, v))
    for p in ("q", "k", "v", "out"):
        out.extend(_lin("mid.attn." + p, c, c))
    _resnet_specs(out, "mid.res1", c, c, v)


def param_specs(cfg: DecoderConfig) -> List[ParamSpec]:
    """Canonical, ordered parameter list of the decoder described by ``cfg``."""
    v = cfg.is_video
    k3 = (3, 3, 3) if v else (3, 3)
    out: List[ParamSpec] = []

    def resnet(prefix, ci, co):
        _resnet_specs(out, prefix, ci, co, v)

    c = cfg.top_channels
    out.extend(_conv("conv_in", c, cfg.z_channels, k3))
    _mid_specs(out, c, v)
    prev = c
    for i, co in enumerate(cfg.stage_channels):
        for j in range(cfg.resnets_per_stage):
            resnet(f"up{i}.res{j}", prev, co)
            prev = co
        if cfg.stage_time_upsamples(i):
            out.extend(_conv(f"up{i}.time_conv", 2 * co, co, (3, 1, 1)))
        if cfg.stage_upsamples(i):
            out.extend(_conv(f"up{i}.upsample", co, co, (3, 3)))
    out.extend(_norm("norm_out", prev, v))
    out.extend(_conv("conv_out", 3, prev, k3))
    return out


def encoder_param_specs(cfg: DecoderConfig) -> List[ParamSpec]:
    """Canonical, ordered parameter list of the encoder of a 2-D preset (see the module text)."""
    if cfg.is_video:
        raise ValueError("the tiled encode is built for the 2-D (AutoencoderKL) presets only")
    block_out = tuple(reversed(cfg.stage_channels))
    out: List[ParamSpec] = []
    out.extend(_conv("conv_in", block_out[0], 3, (3, 3)))
    prev = block_out[0]
    for i, co in enumerate(block_out):
        for j in range(cfg.encoder_resnets):
            _resnet_specs(out, f"down{i}.res{j}", prev, co, False)
            prev = co
        if i < len(block_out) - 1:
            out.extend(_conv(f"down{i}.downsample", co, co, (3, 3)))
    _mid_specs(out, prev, False)
    out.extend(_norm("norm_out", prev, False))
    out.extend(_conv("conv_out", 2 * cfg.z_channels, prev, (3, 3)))
    out.extend(_conv("quant_conv", 2 * cfg.z_channels, 2 * cfg.z_channels, (1, 1)))
    return out
