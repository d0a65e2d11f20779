"""The tiled-decode baseline of the oracle (CPU only).

Strategy page, "Tile/Patch Implementation (Decode)": overlapping tiles decoded
independently, blended in raster order (upper neighbour over the overlap rows,
then left neighbour over the overlap columns), each tile keeping its first
``stride`` output rows and columns, cropped to the image.  Pins: the linear
cross-fade on hand-made tensors, a single covering tile equals the full decode,
non-overlapping tiles are the concatenation of independent tile decodes, one
overlap row and column recomputed from the two tile decodes by the formula,
and the seam metric on hand-made images.
"""
import pytest
import torch

from oracle import blend_h, blend_v, decode_full, decode_tiled, row_seam, tile_origins
from synth import make_latent, make_params, preset

CFG1 = preset(1)    # tiny fp32 decoder: upsampling factor 2


def test_blend_v_linear_crossfade():
    a = torch.ones(1, 1, 1, 6, 3)
    b = torch.zeros(1, 1, 1, 5, 3)
    out = blend_v(a, b, 4)
    assert out is b                      # in place
    col = out[0, 0, 0, :, 1].tolist()
    assert col == pytest.approx([1.0, 0.75, 0.5, 0.25, 0.0])


def test_blend_h_linear_crossfade_and_clipped_extent():
    a = torch.full((1, 1, 1, 2, 2), 2.0)
    b = torch.zeros(1, 1, 1, 2, 5)
    blend_h(a, b, 8)                     # extent clipped to the left tile's 2 columns
    assert b[0, 0, 0, 0].tolist() == pytest.approx([2.0, 1.0, 0.0, 0.0, 0.0])


def test_blend_of_agreeing_overlaps_is_identity():
    # when the neighbour's last rows (columns) equal this tile's first ones, the cross-fade
    # changes nothing
    img = torch.randn(1, 2, 1, 10, 10, generator=torch.Generator().manual_seed(1), dtype=torch.float64)
    upper, tile = img[..., 0:6, :].clone(), img[..., 2:10, :].clone()
    b = tile.clone()
    blend_v(upper, b, 4)
    assert torch.allclose(b, tile, atol=1e-15)
    left, tile = img[..., :, 0:6].clone(), img[..., :, 2:10].clone()
    b = tile.clone()
    blend_h(left, b, 4)
    assert torch.allclose(b, tile, atol=1e-15)


def test_tile_origins():
    assert tile_origins(8, 3) == [0, 3, 6]
    assert tile_origins(8, 8) == [0]
    assert tile_origins(128, 24) == [0, 24, 48, 72, 96, 120]


def test_single_covering_tile_is_the_full_decode():
    p = make_params(CFG1, affine="random")
    z = make_latent(CFG1)
    assert torch.equal(decode_tiled(CFG1, p, z, 8, 8), decode_full(CFG1, p, z))
    assert torch.equal(decode_tiled(CFG1, p, z, 10, 9), decode_full(CFG1, p, z))


def test_non_overlapping_tiles_are_independent_decodes():
    p = make_params(CFG1, affine="random")
    z = make_latent(CFG1)
    y = decode_tiled(CFG1, p, z, 4, 4)
    for i in (0, 4):
        for j in (0, 4):
            t = decode_full(CFG1, p, z[..., i:i + 4, j:j + 4].contiguous())
            assert torch.allclose(y[..., 2 * i:2 * i + 8, 2 * j:2 * j + 8], t, atol=1e-6)


def test_overlap_row_and_column_follow_the_crossfade():
    p = make_params(CFG1, affine="random")
    z = make_latent(CFG1)
    tile, stride, up = 5, 3, 2
    y = decode_tiled(CFG1, p, z, tile, stride).double()
    e = (tile - stride) * up                                  # 4 output rows / columns
    d = lambda i, j: decode_full(CFG1, p, z[..., i:i + tile, j:j + tile].contiguous()).double()
    t00, t10 = d(0, 0), d(3, 0)
    # output rows 6 .. 9 at columns 0 .. 3 (inside tile (0,0)'s kept columns, no left blend):
    # tile (1,0) rows 0 .. 3 blended with tile (0,0) rows 6 .. 9
    for yy in range(e):
        want = t00[..., stride * up + yy, :stride * up] * (1 - yy / e) + t10[..., yy, :stride * up] * (yy / e)
        assert torch.allclose(y[..., stride * up + yy, :stride * up], want, atol=1e-6)
    # the baseline is not the full decode: each tile has its own statistics
    full = decode_full(CFG1, p, z).double()
    assert (y - full).abs().max().item() > 1e-3


def test_row_seam_metric():
    flat = torch.zeros(1, 3, 4, 5)
    assert torch.all(row_seam(flat) == 0)
    step = torch.zeros(1, 3, 4, 5)
    step[:, :, 2:] = 2.0 / 255.0                            # +1 unit in 0-255 scale below row 2
    s = row_seam(step)
    assert s.shape == (3,)
    assert s[1].item() == pytest.approx(1.0) and s[0].item() == 0 and s[2].item() == 0
