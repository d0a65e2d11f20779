"""Tiled decode with overlap blending: the comparison baseline of the sharded decode.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The distributed-VAE strategy page ("Tile/Patch Implementation (Decode)", the
split / exec / merge steps) decodes overlapping latent tiles independently and
stitches them: tiles start every ``stride`` latent rows and columns and span
``tile`` latent rows and columns (clipped at the image edge); each tile is
decoded on its own, as a whole image; the merge walks the tiles in raster
order, blends each tile with its already-merged upper neighbour over the
overlap rows, then with its left neighbour over the overlap columns, and keeps
the first ``stride`` output rows and columns of every tile; the result is
cropped to the image size.  The overlap is ``tile - stride`` latent rows,
i.e. that many times the upsampling factor in output rows.

The pages call the blends (``blend_v`` / ``blend_h``) without printing them.
Reading: the linear cross-fade of the common AutoencoderKL implementations --
over an overlap of ``e = min(rows of the upper tile, rows of this tile,
extent)`` rows, output row ``y < e`` of this tile becomes
``upper[-e + y] * (1 - y / e) + this[y] * (y / e)`` (columns likewise), in
place, so later tiles blend against merged neighbours.

Each tile sees only its own GroupNorm statistics and attention tokens, which
is why this baseline does not reproduce the full-image decode (the
validation page's motivation for layer-wise sharding).
"""
from __future__ import annotations

from typing import Dict, Tuple

import torch

from .decoder import Precision, decode_full


def blend_v(upper: torch.Tensor, tile: torch.Tensor, extent: int) -> torch.Tensor:
    """Cross-fade the first rows of ``tile`` from the last rows of ``upper`` (in place).

    Tensors are [N, C, T, H, W]; rows are dimension 3.
    """
    e = min(upper.shape[3], tile.shape[3], extent)
    for y in range(e):
        tile[:, :, :, y, :] = upper[:, :, :, -e + y, :] * (1 - y / e) + tile[:, :, :, y, :] * (y / e)
    return tile


def blend_h(left: torch.Tensor, tile: torch.Tensor, extent: int) -> torch.Tensor:
    """Cross-fade the first columns of ``tile`` from the last columns of ``left`` (in place)."""
    e = min(left.shape[4], tile.shape[4], extent)
    for x in range(e):
        tile[:, :, :, :, x] = left[:, :, :, :, -e + x] * (1 - x / e) + tile[:, :, :, :, x] * (x / e)
    return tile


def tile_origins(length: int, stride: int):
    """Latent start indices of the tiles along one axis: 0, stride, 2 stride, ... < length."""
    return list(range(0, length, stride))


def decode_tiled(cfg, params: Dict[str, torch.Tensor], latent: torch.Tensor, tile: int, stride: int,
                 prec: Precision = None) -> torch.Tensor:
    """Tiled decode of ``latent`` ([N, Cz, H, W] or [N, Cz, T, H, W]) -> output like decode_full."""
    assert 0 < stride <= tile
    video = latent.dim() == 5
    z5 = latent if video else latent.unsqueeze(2)
    h, w = z5.shape[-2:]
    up = 2 ** (cfg.n_stages - 1)
    blend = (tile - stride) * up          # overlap in output rows / columns
    keep = stride * up                    # output rows / columns each tile contributes
    decoded: Dict[Tuple[int, int], torch.Tensor] = {}
    rows = tile_origins(h, stride)
    cols = tile_origins(w, stride)
    for gi, i in enumerate(rows):
        for gj, j in enumerate(cols):
            sub = z5[:, :, :, i:i + tile, j:j + tile].contiguous()
            y = decode_full(cfg, params, sub if video else sub[:, :, 0], prec)
            decoded[(gi, gj)] = (y if video else y.unsqueeze(2)).to(torch.float64)
    out_rows = []
    for gi in range(len(rows)):
        row = []
        for gj in range(len(cols)):
            t = decoded[(gi, gj)]
            if gi > 0:
                t = blend_v(decoded[(gi - 1, gj)], t, blend)
            if gj > 0:
                t = blend_h(decoded[(gi, gj - 1)], t, blend)
            row.append(t[:, :, :, :keep, :keep])
        out_rows.append(torch.cat(row, dim=4))
    y = torch.cat(out_rows, dim=3)[:, :, :, :h * up, :w * up].to(torch.float32)
    return y if video else y[:, :, 0]


def row_seam(x: torch.Tensor) -> torch.Tensor:
    """Seam metric of the validation page ("Original Seam Reproduction"): per pair of
    adjacent output rows, the mean over columns of the absolute difference of the pixels'
    RGB channel means, in 0-255 units for decoder values in [-1, 1].

    x: [N, 3, H, W] (or [N, 3, T, H, W]); returns [H - 1] (averaged over samples and frames).
    """
    x5 = x if x.dim() == 5 else x.unsqueeze(2)
    m = (x5.to(torch.float64).mean(dim=1) + 1.0) * 127.5        # [N, T, H, W]
    d = (m[:, :, 1:, :] - m[:, :, :-1, :]).abs().mean(dim=3)    # [N, T, H - 1]
    return d.mean(dim=(0, 1))
