"""Tiled encode of the HIP path against the oracle, through the C ABI.

* tiny fp32 preset and a reduced 1024^2-family graph (bf16): one covering tile (the
  whole-image encode) and overlapping tiles with clipped edge tiles, against
  oracle.encode_full / oracle.encode_tiled (the exact oracle: fp32 storage, fp64 math);
* batch 2; a merged block that no blend touches equals the encode of that tile alone;
* the full-size 1024^2 image on 32-latent tiles every 24: finite moments, and the first
  tile's unblended block against the oracle's encode of that 256 x 256 tile;
* argument errors leave the output untouched.
"""
import ctypes as C

import pytest
import torch

import spatially_sharded_conv_amd as vaep
from spatially_sharded_conv_amd import _lib as L
from oracle import Precision, encode_full, encode_tiled
from synth import make_encoder_params, make_image, preset
from tests._util import REFERENCE_PRECISION, TOL, assert_close, to_dev

pytestmark = pytest.mark.gpu


def make_encoder(cfg, affine="random"):
    params = make_encoder_params(cfg, affine=affine)
    lc = vaep.make_config(cfg.family, cfg.dtype, cfg.z_channels, cfg.stage_channels, cfg.resnets_per_stage,
                          cfg.norm_groups, cfg.temporal_up_stages, cfg.eps)
    dev = [to_dev(params[n], cfg.dtype) for n, _ in vaep.encoder_param_info(lc)]
    enc = vaep.Encoder(lc, dev)
    del dev
    return enc, params


def gpu_encode(enc, cfg, image, tile, stride):
    img = to_dev(image, cfg.dtype)
    b, _, h, w = image.shape
    up = 2 ** (cfg.n_stages - 1)
    out = torch.full((b, 2 * cfg.z_channels, h // up, w // up), float("nan"), dtype=torch.float32, device="cuda")
    ws = enc.workspace(b, h, w, tile, stride)
    rc, info = enc.encode_tiled(img, tile, stride, out, ws)
    torch.cuda.synchronize()
    return out, rc, info


def _check(cfg, tables, batch=1):
    enc, params = make_encoder(cfg)
    img = make_image(cfg, batch=batch)
    prec = Precision(REFERENCE_PRECISION)
    lh, lw = cfg.latent_h, cfg.latent_w
    for tile, stride in tables:
        y, rc, info = gpu_encode(enc, cfg, img, tile, stride)
        assert rc == 0 and info.axis == L.AXIS_TILE
        assert info.bands_used == ((lh + stride - 1) // stride) * ((lw + stride - 1) // stride)
        if tile >= max(lh, lw):
            ref = encode_full(cfg, params, img, prec)
        else:
            ref = encode_tiled(cfg, params, img, tile, stride, prec)
        assert_close(y, ref, *TOL[cfg.dtype], what=f"{cfg.name} encode tiles {tile}/{stride} batch {batch}",
                     log=True)
    enc.close()


def test_encode_tiny_fp32():
    """Covering tile; overlapping tiles; stride 1 (64 tiles, edge tiles of eight sizes down
    to one latent pixel, i.e. 2 x 2-pixel images through the whole encoder)."""
    cfg = preset(1)
    _check(cfg, [(8, 8), (4, 3), (3, 2), (3, 1)])


def test_encode_reduced_bf16():
    cfg = preset(2).with_size(latent_h=8, latent_w=12)
    _check(cfg, [(12, 12), (4, 3)])


def test_encode_reduced_bf16_batch():
    cfg = preset(2).with_size(latent_h=6, latent_w=10)
    _check(cfg, [(10, 10), (4, 3)], batch=2)


def test_unblended_block_is_the_tile_encode():
    """Tiles of 4 latent rows every 3 (the full tiles run as one batch of images): the first
    tile's first 3 x 3 latent block is untouched by the merge and equals the whole-image
    encode of that tile's 32 x 32 pixels, bit for bit."""
    cfg = preset(2).with_size(latent_h=8, latent_w=12)
    enc, _ = make_encoder(cfg)
    img = make_image(cfg)
    up = 2 ** (cfg.n_stages - 1)
    y, rc, _ = gpu_encode(enc, cfg, img, 4, 3)
    assert rc == 0
    t, rc, _ = gpu_encode(enc, cfg, img[:, :, :4 * up, :4 * up].contiguous(), 4, 4)
    assert rc == 0
    assert torch.equal(y[:, :, :3, :3], t[:, :, :3, :3])
    enc.close()


def test_encode_full_size_1024():
    """The 1024^2 image of the 1024^2 preset on 32-latent tiles every 24 (25 full tiles in one
    batch, 11 clipped edge tiles): finite moments of the right shape, and the first tile's
    unblended 24 x 24 latent block against the oracle's exact encode of that 256 x 256 tile."""
    cfg = preset(3)
    enc, params = make_encoder(cfg)
    img = make_image(cfg)
    y, rc, info = gpu_encode(enc, cfg, img, 32, 24)
    assert rc == 0 and info.bands_used == 36
    assert y.shape == (1, 32, 128, 128) and torch.isfinite(y).all().item()
    up = 2 ** (cfg.n_stages - 1)
    ref = encode_full(cfg, params, img[:, :, :32 * up, :32 * up].contiguous(), Precision(REFERENCE_PRECISION))
    assert_close(y[:, :, :24, :24], ref[:, :, :24, :24], *TOL[cfg.dtype],
                 what="1024^2 encode, first tile's unblended block", log=True)
    enc.close()


def test_encode_errors_leave_output_untouched():
    cfg = preset(2).with_size(latent_h=4, latent_w=4)
    enc, _ = make_encoder(cfg)
    img = to_dev(make_image(cfg), cfg.dtype)
    out = torch.full((1, 32, 4, 4), 7.0, dtype=torch.float32, device="cuda")
    ws = enc.workspace(1, 32, 32, 4, 4)
    lib = L.load()
    info = L.VaepDecodeInfo()
    P = lambda t: t.data_ptr()
    cases = [
        (P(img), 1, 30, 32, 4, 4, P(out), P(ws), ws.numel(), L.VAEP_ERR_INVALID_ARG),   # not a multiple of 8
        (P(img), 1, 32, 32, 4, 5, P(out), P(ws), ws.numel(), L.VAEP_ERR_INVALID_ARG),   # stride > tile
        (P(img), 1, 32, 32, 4, 0, P(out), P(ws), ws.numel(), L.VAEP_ERR_INVALID_ARG),
        (None, 1, 32, 32, 4, 4, P(out), P(ws), ws.numel(), L.VAEP_ERR_INVALID_ARG),
        (P(img), 1, 32, 32, 4, 4, P(out), P(ws), ws.numel() // 2, L.VAEP_ERR_WORKSPACE),
    ]
    for im, b, h, w, tile, stride, o, wsp, nbytes, code in cases:
        rc = lib.vaep_encode_tiled(enc._h, im, b, h, w, tile, stride, o, wsp, nbytes, None, C.byref(info))
        assert rc == code, (h, w, tile, stride, nbytes, rc, L.last_error())
    torch.cuda.synchronize()
    assert (out == 7.0).all().item()
    enc.close()
