"""Width-sharded and ``auto`` decodes of the HIP path against the oracle, through the C ABI.

The distributed-VAE strategy page lets a request shard the latent along its
height or its width, or leave the choice to a per-request ``auto`` policy (the
longer axis that covers every shard, width on ties, else the tile decode).  Every
rule of the band decode holds with rows and columns exchanged, so each width
decode must equal the full-image decode of the oracle to the same bar as a
height decode:

* tiny fp32 preset, reduced 1024^2-graph and video presets on uneven column
  bands (including one-column bands and ragged tiles) against the oracle's
  exact decode;
* full-size 1024^2, batch-4 and video presets on column bands and ``auto``
  against the stored oracle samples;
* column-band tables are bit-identical to one another and to the one-band
  decode of the same orientation (the band-vs-full bar, met exactly).  Row and
  column decodes accumulate in different orders: with bf16 operands the two are
  independent bf16 rounding sequences of the same decode (each about 4.6e-3
  rel-L2 from the exact decode, like the oracle's own bf16 emulation), so the
  cross-orientation bar is the parity bar, CROSS_AXIS;
* ``auto`` picks the policy's axis and uses the tile decode when neither axis
  covers the shards; explicit axes that cannot be honoured warn and use the
  tile decode (the strategy page's contract table); one model serves
  alternating requests.
"""
import numpy as np
import pytest
import torch

from spatially_sharded_conv_amd import _lib as L
from oracle import Precision, choose_axis, decode_full as oracle_full, decode_tiled as oracle_tiled
from synth import make_latent, preset
from tests._util import BAND_VS_FULL_REL, REFERENCE_PRECISION, TOL, assert_close, errors, to_dev
from tests.test_gpu_decode import check_full_size_output, gpu_decode, make_decoder

pytestmark = pytest.mark.gpu

# Row-band vs column-band decode (different accumulation orders): the oracle parity bar
# in rel-L2 for bf16; fp32 keeps the band-vs-full bar.
CROSS_AXIS = {"bf16": TOL["bf16"][1], "f32": BAND_VS_FULL_REL}


def sharded(dec, cfg, latent, axis, n, starts=None, ws=None):
    lat = to_dev(latent, cfg.dtype)
    b = latent.shape[0]
    t = latent.shape[2] if latent.dim() == 5 else 1
    h, w = latent.shape[-2:]
    out = torch.full(cfg.output_shape(b, t, h, w), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = dec.workspace(b, t, h, w, n)
    rc, info = dec.decode_sharded(lat, axis, n, out, ws, starts)
    torch.cuda.synchronize()
    return out, rc, info


def _check_width(cfg, tables, affine="random"):
    dec, params = make_decoder(cfg, affine)
    z = make_latent(cfg)
    ref = oracle_full(cfg, params, z, Precision(REFERENCE_PRECISION))
    first = None
    for starts in tables:    # tables[0] is the one-band (dense) decode on the transposed image
        y, rc, info = sharded(dec, cfg, z, "width", len(starts) - 1, starts)
        assert rc == 0 and info.axis == L.AXIS_WIDTH and info.bands_used == len(starts) - 1
        assert_close(y, ref, *TOL[cfg.dtype], what=f"{cfg.name} column bands {starts}")
        if first is None:
            first = y
        else:
            assert torch.equal(y, first), f"column bands {starts} differ from {tables[0]}"
    full, rc, _ = gpu_decode(dec, cfg, z, (0, cfg.latent_h))
    assert errors(first, full)[1] <= CROSS_AXIS[cfg.dtype]
    dec.close()


def test_cfg1_tiny_fp32_width(gpu_lib):
    cfg = preset(1)
    _check_width(cfg, [(0, 8), (0, 3, 8), tuple(range(9))])


def test_kl_reduced_width_uneven(gpu_lib):
    cfg = preset(3).with_size(latent_h=10, latent_w=13, band_starts=(0, 10))
    _check_width(cfg, [(0, 13), (0, 4, 5, 9, 13), (0, 1, 13)])


def test_kl_reduced_width_batch(gpu_lib):
    cfg = preset(4).with_size(batch=2, latent_h=6, latent_w=11, band_starts=(0, 6))
    _check_width(cfg, [(0, 11), (0, 3, 7, 11)])


def test_wan_reduced_width(gpu_lib):
    cfg = preset(5).with_size(frames=3, latent_h=6, latent_w=10, band_starts=(0, 6))
    _check_width(cfg, [(0, 10), (0, 3, 4, 10)])


def test_auto_follows_the_policy(gpu_lib):
    # tall, wide and square latents: auto takes the policy's axis and even shards; where
    # neither axis covers the shards it uses the tile decode (strategy page, contract table)
    for h, w, n in [(12, 7, 3), (7, 12, 3), (9, 9, 2), (5, 3, 4), (3, 2, 4), (40, 3, 41)]:
        cfg = preset(3).with_size(latent_h=h, latent_w=w, band_starts=(0, h))
        dec, params = make_decoder(cfg, affine="random")
        z = make_latent(cfg)
        want = choose_axis(h, w, n)
        if want == "tile":
            ref = oracle_tiled(cfg, params, z, 32, 24, Precision(REFERENCE_PRECISION))
            ws = dec.sharded_workspace(1, 1, h, w, n)
        else:
            ref = oracle_full(cfg, params, z, Precision(REFERENCE_PRECISION))
            ws = None
        y, rc, info = sharded(dec, cfg, z, "auto", n, ws=ws)
        code = {"height": L.AXIS_HEIGHT, "width": L.AXIS_WIDTH, "dense": L.AXIS_DENSE, "tile": L.AXIS_TILE}[want]
        assert rc == 0 and info.axis == code, (h, w, n, info.axis)
        tiles = ((h + 23) // 24) * ((w + 23) // 24)
        assert info.bands_used == {"dense": 1, "tile": tiles}.get(want, n)
        assert info.fell_back == (want == "tile")
        assert_close(y, ref, *TOL["bf16"], what=f"auto {h}x{w} / {n} ({want})", log=True)
        dec.close()


def test_explicit_axis_that_cannot_cover_falls_back_to_tile(gpu_lib):
    # strategy page, contract table: a forced axis that is ineligible warns and uses tile
    cfg = preset(3).with_size(latent_h=30, latent_w=3, band_starts=(0, 30))
    dec, params = make_decoder(cfg, affine="random")
    z = make_latent(cfg)
    full, _, _ = gpu_decode(dec, cfg, z, (0, 30))
    ws = dec.sharded_workspace(1, 1, 30, 3, 4)
    small = dec.tiled_workspace(1, 1, 30, 3, 32, 24)
    with pytest.raises(L.VaepError) as e:            # a workspace short of the tile decode's
        sharded(dec, cfg, z, "width", 4, ws=small[: small.numel() // 2])
    assert e.value.code == L.VAEP_ERR_WORKSPACE
    y, rc, info = sharded(dec, cfg, z, "width", 4, ws=ws)
    assert rc == L.VAEP_WARN_FELL_BACK and info.fell_back == 1 and info.axis == L.AXIS_TILE
    assert info.bands_used == 2                       # latent tile rows 0..31 and 24..29
    ref = oracle_tiled(cfg, params, z, 32, 24, Precision(REFERENCE_PRECISION))
    assert_close(y, ref, *TOL["bf16"], what="width 4 on 30x3 (tile fallback)", log=True)
    # the explicit tile mode gives the same decode, without the warning
    t, rc, info = sharded(dec, cfg, z, "tile", 1, ws=ws)
    assert rc == 0 and info.fell_back == 0 and info.axis == L.AXIS_TILE and torch.equal(t, y)
    # the same request on the height axis is honoured
    y, rc, info = sharded(dec, cfg, z, "height", 4, ws=ws)
    assert rc == 0 and info.axis == L.AXIS_HEIGHT and info.bands_used == 4
    assert torch.equal(y, full)
    # more shards than the band limit: tile, with the warning
    y, rc, info = sharded(dec, cfg, z, "height", 65, ws=dec.sharded_workspace(1, 1, 30, 3, 65))
    assert rc == L.VAEP_WARN_FELL_BACK and info.axis == L.AXIS_TILE
    dec.close()


def test_width_errors_leave_output_untouched(gpu_lib):
    cfg = preset(3).with_size(latent_h=6, latent_w=8, band_starts=(0, 6))
    dec, _ = make_decoder(cfg)
    z = to_dev(make_latent(cfg), "bf16")
    out = torch.full(cfg.output_shape(), 7.0, dtype=torch.float32, device="cuda")
    ws = dec.workspace(1, 1, 6, 8, 2)
    # a width table must cover the width (8), not the height (6)
    for bad in [(0, 3, 6), (0, 4, 4, 8), (0, 5, 3, 8), (1, 4, 8)]:
        with pytest.raises(L.VaepError) as e:
            dec.decode_sharded(z, "width", len(bad) - 1, out, ws, bad)
        assert e.value.code == L.VAEP_ERR_INVALID_ARG
    with pytest.raises(L.VaepError) as e:           # auto decides the axis itself
        dec.decode_sharded(z, "auto", 2, out, ws, (0, 4, 8))
    assert e.value.code == L.VAEP_ERR_INVALID_ARG
    with pytest.raises(L.VaepError) as e:
        dec.decode_sharded(z, "width", 2, out, ws[: ws.numel() // 2], (0, 4, 8))
    assert e.value.code == L.VAEP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    dec.close()


def test_alternating_axes_on_one_model(gpu_lib):
    cfg = preset(3).with_size(latent_h=9, latent_w=11, band_starts=(0, 9))
    dec, _ = make_decoder(cfg, affine="random")
    z = make_latent(cfg)
    ws = dec.workspace(1, 1, 9, 11, 4)
    h1, _, _ = sharded(dec, cfg, z, "height", 3, ws=ws)
    w1, _, i1 = sharded(dec, cfg, z, "width", 4, ws=ws)
    a1, _, ia = sharded(dec, cfg, z, "auto", 4, ws=ws)
    h2, _, _ = sharded(dec, cfg, z, "height", 3, ws=ws)
    w2, _, _ = sharded(dec, cfg, z, "width", 2, (0, 5, 11), ws=ws)
    assert i1.axis == L.AXIS_WIDTH and ia.axis == L.AXIS_WIDTH
    assert torch.equal(h1, h2) and torch.equal(w1, w2) and torch.equal(a1, w1)
    assert errors(w1, h1)[1] <= CROSS_AXIS["bf16"]
    dec.close()


@pytest.mark.parametrize("i,axis", [(3, "width"), (4, "width"), (5, "auto")])
def test_full_size_width_against_oracle(gpu_lib, i, axis):
    # the full decode's stored oracle outputs; the width (or auto) decode must meet the
    # same bar, on the configuration's own shard sizes laid across the columns
    cfg = preset(i)
    dec, _ = make_decoder(cfg)
    z = make_latent(cfg)
    n = len(cfg.band_starts) - 1
    if axis == "width":
        sizes = np.diff(cfg.band_starts)
        starts = tuple(int(v) for v in np.concatenate([[0], np.cumsum(sizes)]))
        assert starts[-1] == cfg.latent_w
        y, rc, info = sharded(dec, cfg, z, "width", n, starts)
    else:
        y, rc, info = sharded(dec, cfg, z, "auto", n)
    assert rc == 0 and info.axis == L.AXIS_WIDTH and info.bands_used == n
    dense_t, rc, _ = sharded(dec, cfg, z, "width", 1, (0, cfg.latent_w))
    assert rc == 0 and torch.equal(y, dense_t)      # band vs full, same orientation
    del dense_t
    full, rc, _ = gpu_decode(dec, cfg, z, (0, cfg.latent_h))
    assert errors(y, full)[1] <= CROSS_AXIS["bf16"]
    del full
    dec.close()
    check_full_size_output(i, y, f"{axis} decode")
