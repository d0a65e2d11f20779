"""Whole-decoder invariants of the oracle (CPU only).

* band decode equals full decode for any partition into row bands or column
  bands (the width-sharded mode of the strategy page) (both
  pages: the layer-wise decode keeps full-image semantics, with no seam
  blending; the validation page compares full decoded tensors including
  boundary rows, for even and uneven heights, batches and video frames);
* batch independence (GroupNorm statistics are per sample and group);
* causality of the video decoder (causal time convs, per-frame attention);
* output shapes of every preset;
* the per-request ``auto`` axis policy (strategy page, Wan spatial-shard
  notes: the longer axis that covers every shard, width winning ties, else the
  tile decode).
"""
import pytest
import torch

from oracle import choose_axis, decode_auto, decode_bands, decode_full, decode_tiled, even_starts, Precision
from synth import make_latent, make_params, preset


def _rel(a, b):
    return ((a.double() - b.double()).norm() / b.double().norm()).item()


CFG1 = preset(1)


@pytest.mark.parametrize("starts", [(0, 3, 8), (0, 8), (0, 1, 2, 3, 4, 5, 6, 7, 8), (0, 7, 8)])
def test_band_equals_full_cfg1_fp32(starts):
    p = make_params(CFG1, affine="random")
    z = make_latent(CFG1)
    full = decode_full(CFG1, p, z)
    band = decode_bands(CFG1, p, z, starts)
    assert band.shape == full.shape == (1, 3, 16, 16)
    assert _rel(band, full) <= 1e-6
    assert (band - full).abs().max().item() <= 1e-5


def _reduced(cfg_id, **kw):
    return preset(cfg_id).with_size(**kw)


@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_band_equals_full_kl2d_reduced(prec):
    # configs 2-4 architecture (512-channel mid block, 3 upsamples) at latent 8x6, uneven bands
    cfg = _reduced(3, latent_h=8, latent_w=6, band_starts=(0, 3, 4, 8))
    p = make_params(cfg, affine="random")
    z = make_latent(cfg)
    full = decode_full(cfg, p, z, Precision(prec))
    band = decode_bands(cfg, p, z, cfg.band_starts, Precision(prec))
    assert full.shape == (1, 3, 64, 48)
    assert _rel(band, full) <= (1e-6 if prec == "f32" else 1e-3)


def test_band_equals_full_wan_reduced():
    cfg = _reduced(5, frames=3, latent_h=5, latent_w=6, band_starts=(0, 1, 3, 5))
    p = make_params(cfg, affine="random")
    z = make_latent(cfg)
    full = decode_full(cfg, p, z, Precision("f32"))
    band = decode_bands(cfg, p, z, cfg.band_starts, Precision("f32"))
    assert full.shape == (1, 3, 9, 40, 48)
    assert _rel(band, full) <= 1e-6


def test_batch_independence_kl2d():
    cfg = _reduced(4, batch=2, latent_h=4, latent_w=4, band_starts=(0, 1, 4))
    p = make_params(cfg, affine="random")
    z = make_latent(cfg)
    both = decode_bands(cfg, p, z, cfg.band_starts, Precision("f32"))
    for b in range(2):
        one = decode_full(cfg, p, z[b:b + 1].clone(), Precision("f32"))
        assert _rel(both[b:b + 1], one) <= 1e-6


def test_wan_causality():
    cfg = _reduced(5, frames=3, latent_h=3, latent_w=4, band_starts=(0, 1, 3))
    p = make_params(cfg, affine="random")
    z = make_latent(cfg)
    y0 = decode_full(cfg, p, z, Precision("f32"))
    for k in (1, 2):
        z2 = z.clone()
        z2[:, :, k] += 1.0
        y1 = decode_full(cfg, p, z2, Precision("f32"))
        first = 1 + 4 * (k - 1)
        assert torch.equal(y1[:, :, :first], y0[:, :, :first])
        assert not torch.equal(y1[:, :, first], y0[:, :, first])


def test_output_shapes_of_presets():
    want = {1: (1, 3, 16, 16), 2: (1, 3, 512, 512), 3: (1, 3, 1024, 1024),
            4: (4, 3, 1024, 1024), 5: (1, 3, 17, 480, 832)}
    for i, shape in want.items():
        assert preset(i).output_shape() == shape


def test_band_table_presets():
    for i in range(1, 6):
        s = preset(i).band_starts
        assert s[0] == 0 and s[-1] == preset(i).latent_h
        assert all(a < b for a, b in zip(s, s[1:]))
    assert [b - a for a, b in zip(preset(3).band_starts, preset(3).band_starts[1:])] == [31, 33, 32, 32]
    sizes4 = [b - a for a, b in zip(preset(4).band_starts, preset(4).band_starts[1:])]
    assert len(sizes4) == 8 and min(sizes4) == 15 and max(sizes4) == 17
    assert [b - a for a, b in zip(preset(5).band_starts, preset(5).band_starts[1:])] == [14, 16, 15, 15]


@pytest.mark.parametrize("starts", [(0, 3, 8), (0, 1, 2, 3, 4, 5, 6, 7, 8), (0, 7, 8)])
def test_width_bands_equal_full_cfg1_fp32(starts):
    p = make_params(CFG1, affine="random")
    z = make_latent(CFG1)
    full = decode_full(CFG1, p, z)
    band = decode_bands(CFG1, p, z, starts, axis="width")
    assert band.shape == full.shape
    assert _rel(band, full) <= 1e-6
    assert (band - full).abs().max().item() <= 1e-5


@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_width_bands_equal_full_kl2d_reduced(prec):
    cfg = _reduced(3, latent_h=5, latent_w=9)
    p = make_params(cfg, affine="random")
    z = make_latent(cfg)
    full = decode_full(cfg, p, z, Precision(prec))
    band = decode_bands(cfg, p, z, (0, 2, 3, 9), Precision(prec), axis="width")
    assert band.shape == full.shape == (1, 3, 40, 72)
    assert _rel(band, full) <= (1e-6 if prec == "f32" else 1e-3)


def test_width_bands_equal_full_wan_reduced():
    cfg = _reduced(5, frames=3, latent_h=4, latent_w=7)
    p = make_params(cfg, affine="random")
    z = make_latent(cfg)
    full = decode_full(cfg, p, z, Precision("f32"))
    band = decode_bands(cfg, p, z, (0, 1, 4, 7), Precision("f32"), axis="width")
    assert band.shape == full.shape == (1, 3, 9, 32, 56)
    assert _rel(band, full) <= 1e-6


def test_width_bands_are_not_row_bands():
    # a band table read on the wrong axis is a different (wrong) tensor shape or cut:
    # on a non-square latent the width bands must cover the width, not the height
    p = make_params(CFG1, affine="random")
    z = make_latent(CFG1)[..., :6]          # 8 x 6 latent
    with pytest.raises(AssertionError):
        decode_bands(CFG1, p, z, (0, 3, 8), axis="width")
    y = decode_bands(CFG1, p, z, (0, 3, 6), axis="width")
    assert _rel(y, decode_full(CFG1, p, z)) <= 1e-6


@pytest.mark.parametrize("h,w,n,axis", [
    (60, 104, 4, "width"),     # the Wan workload: width is the longer axis
    (64, 64, 2, "width"),      # a tie goes to width
    (128, 64, 4, "height"),    # height longer and it covers the shards
    (3, 2, 3, "height"),       # width longer-or-equal fails to cover: height
    (2, 3, 3, "width"),
    (2, 5, 3, "width"),
    (5, 2, 3, "height"),
    (2, 2, 3, "tile"),         # neither axis covers the shards: the tile decode
    (8, 8, 1, "dense"),        # one shard is the dense decode
    (8, 8, 8, "width"),
    (8, 7, 8, "height"),
])
def test_choose_axis(h, w, n, axis):
    assert choose_axis(h, w, n) == axis


@pytest.mark.parametrize("length,n", [(8, 2), (8, 3), (128, 8), (104, 4), (60, 7), (5, 5)])
def test_even_starts(length, n):
    s = even_starts(length, n)
    sizes = [b - a for a, b in zip(s, s[1:])]
    assert s[0] == 0 and s[-1] == length and len(sizes) == n
    assert max(sizes) - min(sizes) <= 1 and sizes == sorted(sizes, reverse=True)


def test_decode_auto_cfg1():
    p = make_params(CFG1, affine="random")
    z = make_latent(CFG1)[..., :5]          # 8 x 5: height is longer
    full = decode_full(CFG1, p, z)
    y, axis = decode_auto(CFG1, p, z, 2)
    assert axis == "height" and _rel(y, full) <= 1e-6
    y, axis = decode_auto(CFG1, p, z, 6)    # width 5 cannot cover 6 shards, height 8 can
    assert axis == "height" and _rel(y, full) <= 1e-6
    zt = z.transpose(-1, -2).contiguous()   # 5 x 8
    y, axis = decode_auto(CFG1, p, zt, 3)
    assert axis == "width" and _rel(y, decode_full(CFG1, p, zt)) <= 1e-6


def test_decode_auto_uses_tiles_when_no_axis_covers():
    # strategy page: "If neither axis can cover the group, auto mode uses tile decode"
    cfg = CFG1.with_size(latent_h=40, latent_w=3, band_starts=(0, 40))
    p = make_params(cfg, affine="random")
    z = make_latent(cfg)
    y, axis = decode_auto(cfg, p, z, 41)
    assert axis == "tile"
    assert torch.equal(y, decode_tiled(cfg, p, z, 32, 24))
    assert _rel(y, decode_full(cfg, p, z)) > 1e-3          # tiles are not the full decode
