"""Whole-decoder invariants of the oracle (CPU only).

* band decode equals full decode for any partition into row bands (both
  pages: the layer-wise decode keeps full-image semantics, with no seam
  blending; the validation page compares full decoded tensors including
  boundary rows, for even and uneven heights, batches and video frames);
* batch independence (GroupNorm statistics are per sample and group);
* causality of the video decoder (causal time convs, per-frame attention);
* output shapes of every preset.
"""
import pytest
import torch

from oracle import decode_bands, decode_full, Precision
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
