"""Tiled decode with overlap blending (the comparison baseline), HIP path vs the oracle.

Strategy page, "Tile/Patch Implementation (Decode)": the HIP path decodes each
latent tile with the same kernels as a one-band decode and merges them with the
cross-fade of ``oracle.tiled``; the oracle decodes and merges the same tiles.
Also: a covering tile is exactly the full decode, argument errors, and the
baseline differs from the full decode while the band decodes do not.
"""
import pytest
import torch

from spatially_sharded_conv_amd import _lib as L
from oracle import Precision, decode_tiled as oracle_tiled
from synth import make_latent, preset
from tests._util import REFERENCE_PRECISION, TOL, assert_close, errors, to_dev
from tests.test_gpu_decode import gpu_decode, make_decoder

pytestmark = pytest.mark.gpu


def tiled(dec, cfg, latent, tile, stride):
    lat = to_dev(latent, cfg.dtype)
    b = latent.shape[0]
    t = latent.shape[2] if latent.dim() == 5 else 1
    h, w = latent.shape[-2:]
    out = torch.full(cfg.output_shape(b, t, h, w), float("nan"), dtype=torch.float32, device="cuda")
    ws = dec.tiled_workspace(b, t, h, w, tile, stride)
    rc = dec.decode_tiled(lat, tile, stride, out, ws)
    torch.cuda.synchronize()
    return out, rc


def _check(cfg, tile, stride):
    dec, params = make_decoder(cfg, affine="random")
    z = make_latent(cfg)
    y, rc = tiled(dec, cfg, z, tile, stride)
    assert rc == 0
    ref = oracle_tiled(cfg, params, z, tile, stride, Precision(REFERENCE_PRECISION))
    assert_close(y, ref, *TOL[cfg.dtype], what=f"{cfg.name} tiles {tile}/{stride}")
    full, _, _ = gpu_decode(dec, cfg, z, (0, cfg.latent_h))
    dec.close()
    return y, full


def test_cfg1_tiny_fp32_tiled(gpu_lib):
    y, full = _check(preset(1), 5, 3)
    assert errors(y, full)[0] > 1e-3          # tiles see their own statistics


def test_kl_reduced_tiled_bf16(gpu_lib):
    cfg = preset(3).with_size(latent_h=10, latent_w=13, band_starts=(0, 10))
    _check(cfg, 6, 4)


def test_wan_reduced_tiled(gpu_lib):
    cfg = preset(5).with_size(frames=3, latent_h=6, latent_w=9, band_starts=(0, 6))
    _check(cfg, 4, 3)


def test_covering_tile_is_the_full_decode(gpu_lib):
    cfg = preset(3).with_size(latent_h=9, latent_w=7, band_starts=(0, 9))
    dec, _ = make_decoder(cfg, affine="random")
    z = make_latent(cfg)
    full, _, _ = gpu_decode(dec, cfg, z, (0, 9))
    for tile, stride in [(9, 9), (12, 10)]:
        y, rc = tiled(dec, cfg, z, tile, stride)
        assert rc == 0 and torch.equal(y, full)
    dec.close()


def test_tiled_argument_errors(gpu_lib):
    cfg = preset(3).with_size(latent_h=8, latent_w=8, band_starts=(0, 8))
    dec, _ = make_decoder(cfg)
    z = to_dev(make_latent(cfg), "bf16")
    out = torch.full(cfg.output_shape(), 7.0, dtype=torch.float32, device="cuda")
    ws = dec.tiled_workspace(1, 1, 8, 8, 4, 3)
    for tile, stride in [(4, 5), (0, 1), (4, 0)]:
        with pytest.raises(L.VaepError) as e:
            dec.decode_tiled(z, tile, stride, out, ws)
        assert e.value.code == L.VAEP_ERR_INVALID_ARG
    with pytest.raises(L.VaepError) as e:
        dec.decode_tiled(z, 4, 3, out, ws[: ws.numel() // 2])
    assert e.value.code == L.VAEP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    dec.close()
