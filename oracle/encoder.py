"""Encoder graph of the oracle and the tiled encode with overlap blending.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The distributed-VAE strategy page ("Tile/Patch Encode Implementation") splits the
input image into overlapping tiles, encodes every tile on its own (the encoder
followed by ``quant_conv``) and merges the encoded tiles in latent space the way
the tile decode merges decoded tiles: raster order, blend from the upper
neighbour over the overlap rows, then from the left neighbour over the overlap
columns, keep ``stride`` rows and columns of every tile, crop to the latent size.
The page takes Wan2.2's video encoder as its example; here the same steps run on
the encoder of the 2-D (AutoencoderKL) presets.

The encoder structure is a reading (the pages do not print it): the decoder's
mirror --

* ``conv_in`` (RGB -> the narrowest width) -> down stages -> mid block (resnet,
  single-head attention, resnet) -> GroupNorm -> SiLU -> ``conv_out`` (2 z
  channels: mean and log-variance) -> ``quant_conv`` (1x1, 2 z -> 2 z);
* down stage i: ``encoder_resnets`` resnets (the first changes the channel count),
  then, in every stage but the last, a 3x3 stride-2 convolution over the input
  zero-padded by one row at the bottom and one column at the right
  (``ops.downsample_conv``).

Resnets, norms and attention are the decoder's operators (``decoder._resnet``,
``decoder.FullOps``).  Tile geometry is in latent units: tiles of ``tile``
latent rows and columns (``tile * 2^(n_stages-1)`` image pixels) start every
``stride`` latent rows and columns; the blend overlap is ``tile - stride``.
"""
from __future__ import annotations

from typing import Dict, Tuple

import torch

from . import ops
from .decoder import FullOps, Precision, _as5d, _resnet
from .tiled import blend_h, blend_v, tile_origins


def _encoder_graph(o: FullOps, cfg, p: Dict[str, torch.Tensor], image: torch.Tensor) -> torch.Tensor:
    x = o.enter(image)
    x = o.conv(x, p["conv_in.weight"], p["conv_in.bias"])
    n = cfg.n_stages
    for i in range(n):
        for j in range(cfg.encoder_resnets):
            x = _resnet(o, p, f"down{i}.res{j}", x)
        if i < n - 1:
            x = ops.downsample_conv(x, _as5d(p[f"down{i}.downsample.weight"]), p[f"down{i}.downsample.bias"],
                                    o.acc)
    x = _resnet(o, p, "mid.res0", x)
    x = o.attention(x, p)
    x = _resnet(o, p, "mid.res1", x)
    x = o.norm(x, p, "norm_out", act=True)
    x = o.conv(x, p["conv_out.weight"], p["conv_out.bias"])
    x = o.conv(x, p["quant_conv.weight"], p["quant_conv.bias"])
    return o.leave(x)


def encode_full(cfg, params: Dict[str, torch.Tensor], image: torch.Tensor, prec: Precision = None) -> torch.Tensor:
    """Whole-image encode of ``image`` [N, 3, H, W] (H, W multiples of 2^(n_stages-1)) ->
    float32 moments [N, 2 z, H / 2^(n_stages-1), W / 2^(n_stages-1)]."""
    if cfg.is_video:
        raise ValueError("the encoder is built for the 2-D presets")
    up = 2 ** (cfg.n_stages - 1)
    assert image.dim() == 4 and image.shape[1] == 3 and image.shape[2] % up == 0 and image.shape[3] % up == 0
    prec = prec or Precision(cfg.dtype)
    with torch.no_grad():
        return _encoder_graph(FullOps(cfg, prec), cfg, params, image)


def encode_tiled(cfg, params: Dict[str, torch.Tensor], image: torch.Tensor, tile: int, stride: int,
                 prec: Precision = None) -> torch.Tensor:
    """Tiled encode of ``image`` [N, 3, H, W] -> moments like encode_full (tile, stride in latent units)."""
    assert 0 < stride <= tile
    up = 2 ** (cfg.n_stages - 1)
    lh, lw = image.shape[2] // up, image.shape[3] // up
    rows, cols = tile_origins(lh, stride), tile_origins(lw, stride)
    enc: Dict[Tuple[int, int], torch.Tensor] = {}
    for gi, i in enumerate(rows):
        for gj, j in enumerate(cols):
            sub = image[:, :, i * up:(i + tile) * up, j * up:(j + tile) * up].contiguous()
            enc[(gi, gj)] = encode_full(cfg, params, sub, prec).unsqueeze(2).to(torch.float64)
    blend = tile - stride
    out_rows = []
    for gi in range(len(rows)):
        row = []
        for gj in range(len(cols)):
            t = enc[(gi, gj)]
            if gi > 0:
                t = blend_v(enc[(gi - 1, gj)], t, blend)
            if gj > 0:
                t = blend_h(enc[(gi, gj - 1)], t, blend)
            row.append(t[:, :, :, :stride, :stride])
        out_rows.append(torch.cat(row, dim=4))
    return torch.cat(out_rows, dim=3)[:, :, 0, :lh, :lw].to(torch.float32)
