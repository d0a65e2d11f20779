"""Whole-decode parity of the HIP path against the oracle, through the C ABI.

* tiny fp32 preset and the 512^2 preset against the oracle's full decode, as
  full and band decodes;
* reduced-size variants of the 1024^2 presets and of the video preset (same
  graphs, latents small enough for the oracle) with uneven and one-row bands;
* full-size 1024^2, batch-4 and video presets against oracle outputs stored by
  tests/golden/make_full_size_golden.py (the whole 1024^2 output; rows around every
  band boundary and image edge, samples, and the whole output when generated, for the
  others), in the configuration bench.py times;
* band decode against full decode on the GPU; error paths; repeated and
  alternating calls on one model.
"""
import importlib.util
import json
import os

import numpy as np
import pytest
import torch

import spatially_sharded_conv_amd as vaep
from spatially_sharded_conv_amd import _lib as L
from oracle import Precision, decode_full as oracle_full
from synth import make_latent, make_params, preset
from tests._util import BAND_VS_FULL_REL, REFERENCE_PRECISION, TOL, assert_close, errors, to_dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def make_decoder(cfg, affine="default"):
    params = make_params(cfg, affine=affine)
    lc = vaep.make_config(cfg.family, cfg.dtype, cfg.z_channels, cfg.stage_channels,
                          cfg.resnets_per_stage, cfg.norm_groups, cfg.temporal_up_stages, cfg.eps)
    dev = [to_dev(params[n], cfg.dtype) for n, _ in vaep.param_info(lc)]
    dec = vaep.Decoder(lc, dev)
    del dev
    return dec, params


def gpu_decode(dec, cfg, latent, starts, ws=None):
    lat = to_dev(latent, cfg.dtype)
    b = latent.shape[0]
    t = latent.shape[2] if latent.dim() == 5 else 1
    h, w = latent.shape[-2:]
    out = torch.empty(cfg.output_shape(b, t, h, w), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = dec.workspace(b, t, h, w, len(starts) - 1)
    rc, info = dec.decode_bands(lat, starts, out, ws)
    torch.cuda.synchronize()
    return out, rc, info


def _check_against_oracle(cfg, starts_list, affine="default"):
    dec, params = make_decoder(cfg, affine)
    z = make_latent(cfg)
    # the exact decode (fp32 storage, fp64 arithmetic); see REFERENCE_PRECISION in _util
    ref = oracle_full(cfg, params, z, Precision(REFERENCE_PRECISION))
    outs = []
    for starts in starts_list:
        y, rc, info = gpu_decode(dec, cfg, z, starts)
        assert rc == 0 and info.bands_used == len(starts) - 1
        assert_close(y, ref, *TOL[cfg.dtype], what=f"{cfg.name} bands {starts}", log=True)
        outs.append(y)
    full = outs[0]
    for y in outs[1:]:
        assert errors(y, full)[1] <= BAND_VS_FULL_REL
    dec.close()


def test_cfg1_tiny_fp32_full_and_bands(gpu_lib):
    cfg = preset(1)
    _check_against_oracle(cfg, [(0, 8), cfg.band_starts, tuple(range(9))], affine="random")


def test_cfg1_default_init(gpu_lib):
    cfg = preset(1)
    _check_against_oracle(cfg, [(0, 8), cfg.band_starts])


def test_cfg2_512_bf16_full_and_bands(gpu_lib):
    cfg = preset(2)
    _check_against_oracle(cfg, [(0, 64), cfg.band_starts])


def test_kl_reduced_uneven_bands(gpu_lib):
    cfg = preset(3).with_size(latent_h=12, latent_w=20, band_starts=(0, 3, 7, 8, 12))
    _check_against_oracle(cfg, [(0, 12), cfg.band_starts], affine="random")


def test_kl_reduced_batch(gpu_lib):
    cfg = preset(4).with_size(batch=2, latent_h=10, latent_w=8, band_starts=(0, 3, 6, 10))
    _check_against_oracle(cfg, [(0, 10), cfg.band_starts, (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10)],
                          affine="random")


def test_wan_reduced_video(gpu_lib):
    cfg = preset(5).with_size(frames=3, latent_h=6, latent_w=10, band_starts=(0, 2, 3, 6))
    _check_against_oracle(cfg, [(0, 6), cfg.band_starts], affine="random")


def _golden_module():
    spec = importlib.util.spec_from_file_location("mk", os.path.join(GOLDEN, "make_full_size_golden.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    return mk


def check_full_size_output(i, y, what):
    """Compare a full-size decode of preset i with every stored oracle output: samples, the
    whole 1024^2 output or the rows near band boundaries and edges, and the whole output
    when generated (tests/golden/full/).  y: the decoded tensor (any device)."""
    mk = _golden_module()
    meta = json.load(open(os.path.join(GOLDEN, f"cfg{i}_oracle_summary.json")))
    cfg = preset(i)
    bar = TOL[cfg.dtype]
    assert list(y.shape) == meta["shape"]
    pos = torch.from_numpy(mk.sample_positions(i, y.numel()))
    ref = torch.from_numpy(np.load(os.path.join(GOLDEN, f"cfg{i}_oracle_samples.npy"))).double()
    assert_close(y.reshape(-1)[pos.to(y.device)].double().cpu(), ref, *bar, what=f"config {i} {what} samples")
    y = y.cpu()
    if i == 3:
        whole = torch.from_numpy(np.load(os.path.join(GOLDEN, "cfg3_oracle_full.npy")))
        assert_close(y, whole, *bar, what=f"config 3 {what} whole output", log=True)
    else:
        d = np.load(os.path.join(GOLDEN, f"cfg{i}_oracle_rows.npz"))
        rows = torch.from_numpy(d["rows"])
        assert torch.equal(rows, torch.from_numpy(mk.boundary_rows(cfg)))
        assert_close(y.index_select(-2, rows), torch.from_numpy(d["values"]), *bar,
                     what=f"config {i} {what} rows near band boundaries and edges ({rows.numel()} rows)", log=True)
        full_path = os.path.join(GOLDEN, "full", f"cfg{i}_oracle_full.npy")
        if os.path.exists(full_path):
            assert_close(y, torch.from_numpy(np.load(full_path)), *bar, what=f"config {i} {what} whole output",
                         log=True)
    # whole-tensor summary statistics of the oracle output
    yd = y.double()
    assert abs(yd.mean().item() - meta["mean"]) < 1e-3
    assert abs(yd.std().item() - meta["std"]) / meta["std"] < 1e-3


@pytest.mark.parametrize("i", [3, 4, 5])
def test_full_size_parity(gpu_lib, i):
    """Full-size presets in the configuration bench.py times, against stored oracle outputs
    (tests/golden/make_full_size_golden.py): the whole 1024^2 output; for the batch-4 and
    video presets every output row within 8 rows of a band boundary or an image edge, the
    sampled positions and, when generated, the whole output (tests/golden/full/).  The band
    decode equals the full decode bit for bit."""
    cfg = preset(i)
    dec, _ = make_decoder(cfg)
    z = make_latent(cfg)
    y_full, rc, _ = gpu_decode(dec, cfg, z, (0, cfg.latent_h))
    assert rc == 0
    y_band, rc, info = gpu_decode(dec, cfg, z, cfg.band_starts)
    assert rc == 0 and info.bands_used == len(cfg.band_starts) - 1
    dec.close()
    assert torch.equal(y_band, y_full), f"config {i}: band decode differs from the full decode"
    del y_full
    check_full_size_output(i, y_band, "band decode")


def test_error_paths_leave_output_untouched(gpu_lib):
    cfg = preset(3).with_size(latent_h=8, latent_w=8, band_starts=(0, 4, 8))
    dec, _ = make_decoder(cfg)
    z = to_dev(make_latent(cfg), "bf16")
    out = torch.full(cfg.output_shape(), 7.0, dtype=torch.float32, device="cuda")
    ws = dec.workspace(1, 1, 8, 8, 2)
    small = ws[: ws.numel() // 2]
    with pytest.raises(L.VaepError) as e:
        dec.decode_bands(z, (0, 4, 8), out, small)
    assert e.value.code == L.VAEP_ERR_WORKSPACE
    for bad in [(0, 4, 4, 8), (0, 5, 3, 8), (0, 4, 7), (1, 4, 8)]:
        with pytest.raises(L.VaepError) as e:
            dec.decode_bands(z, bad, out, ws)
        assert e.value.code == L.VAEP_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    dec.close()


def test_too_many_bands_fall_back_to_dense(gpu_lib):
    cfg = preset(3).with_size(latent_h=70, latent_w=4, band_starts=(0, 70))
    dec, _ = make_decoder(cfg)
    z = make_latent(cfg)
    full, rc, _ = gpu_decode(dec, cfg, z, (0, 70))
    starts = tuple(range(71))
    y, rc, info = gpu_decode(dec, cfg, z, starts)
    assert rc == L.VAEP_WARN_FELL_BACK and info.fell_back == 1 and info.bands_used == 1
    assert torch.equal(y, full)
    dec.close()


def test_repeat_and_alternating_calls(gpu_lib):
    cfg = preset(3).with_size(latent_h=10, latent_w=12, band_starts=(0, 3, 10))
    dec, _ = make_decoder(cfg, affine="random")
    z = make_latent(cfg)
    ws = dec.workspace(1, 1, 10, 12, 4)
    a, _, _ = gpu_decode(dec, cfg, z, (0, 3, 10), ws)
    b, _, _ = gpu_decode(dec, cfg, z, (0, 10), ws)
    c, _, _ = gpu_decode(dec, cfg, z, (0, 1, 5, 9, 10), ws)
    d, _, _ = gpu_decode(dec, cfg, z, (0, 3, 10), ws)
    assert torch.equal(a, d)
    assert errors(b, a)[1] <= BAND_VS_FULL_REL and errors(c, a)[1] <= BAND_VS_FULL_REL
    dec.close()


def test_full_size_bands_bit_identical_and_kernels(gpu_lib):
    # The 1024^2 decode runs every conv kernel family (128x128 tiles, wide tiles for the
    # sub-pixel upsamples and split outputs, halo tiles with GroupNorm moments in the
    # epilogue for the plain 3x3 convs and, with the 1x1 shortcut folded in as extra K
    # steps, for the resnets that change the channel count, narrow conv_out); its band
    # decode must equal the full decode bit for bit.
    cfg = preset(3)
    dec, _ = make_decoder(cfg)
    z = make_latent(cfg)
    ws = dec.workspace(1, 1, cfg.latent_h, cfg.latent_w, len(cfg.band_starts) - 1)
    y_full, rc, _ = gpu_decode(dec, cfg, z, (0, cfg.latent_h), ws)
    assert rc == 0
    vaep.profile_begin(dec)
    y_band, rc, _ = gpu_decode(dec, cfg, z, cfg.band_starts, ws)
    recs = vaep.profile_end(dec)
    assert rc == 0
    used = {r["kernel"] for r in recs if r["step"] == L.STEP_CONV}
    for k in (L.KERNEL_CONV_TILE128, L.KERNEL_CONV_WIDE256, L.KERNEL_CONV_HALO, L.KERNEL_CONV_HALO_X2,
              L.KERNEL_CONV_NARROW):
        assert k in used, (k, used)
    assert torch.equal(y_band, y_full)
    dec.close()


def test_norm_fold_gives_the_same_decode(gpu_lib):
    """With the GroupNorm apply folded into the operand load of the latent-resolution resnet
    convs (vaep_model_set_norm_fold), the decode is bit-identical to the one with separate
    apply passes: the fold computes the same operand bits (same scale/shift, SiLU and
    rounding, zero padding), and the halo rows it reads are the producing conv's raw rows.
    Also on a band table whose odd bands keep the convs unfolded, and with batch 2."""
    # (preset, band table, whether fewer apply passes run): at 64 latent columns a 7-row band
    # is not a whole number of 128-pixel tiles, so the latent-resolution convs stay unfolded
    # there (the next stage's 14-row band folds)
    cases = ((preset(3), None, True), (preset(3), (0, 31, 64, 96, 128), True),
             (preset(2).with_size(batch=2), None, True), (preset(2).with_size(batch=2), (0, 7, 20, 33, 64), None))
    for cfg, starts, folds in cases:
        dec, _ = make_decoder(cfg)
        z = make_latent(cfg)
        b = z.shape[0]
        ws = dec.workspace(b, 1, cfg.latent_h, cfg.latent_w, 4)
        starts = starts or cfg.band_starts
        dec.set_norm_fold(False)
        vaep.profile_begin(dec)
        y0, rc, _ = gpu_decode(dec, cfg, z, starts, ws)
        r0 = vaep.profile_end(dec)
        assert rc == 0
        dec.set_norm_fold(True)
        vaep.profile_begin(dec)
        y1, rc, _ = gpu_decode(dec, cfg, z, starts, ws)
        r1 = vaep.profile_end(dec)
        assert rc == 0
        assert torch.equal(y0, y1), (cfg.name, starts)
        gn0 = sum(r["n_kernels"] for r in r0 if r["step"] == L.STEP_GROUPNORM)
        gn1 = sum(r["n_kernels"] for r in r1 if r["step"] == L.STEP_GROUPNORM)
        assert folds is None or (gn1 < gn0) == folds, (cfg.name, starts, gn0, gn1)   # applies folded away
        dec.close()


def test_halo_poison_gives_the_same_decode(gpu_lib):
    """With every halo slot of a band buffer filled with NaN before the layer that writes
    it (vaep_model_set_halo_poison), a decode gives the same bits as without: each halo row
    a layer reads came from its neighbour's push in that decode, and no slot past the image
    edge is read.  One-band, uneven and one-row band tables; width bands; the full-size
    1024^2, batch-4 and video presets; the folded GroupNorm apply; the tile decode."""
    def width_decode(dec, cfg, latent, starts):
        lat = to_dev(latent, cfg.dtype)
        out = torch.empty(cfg.output_shape(latent.shape[0], 1, *latent.shape[-2:]), dtype=torch.float32,
                          device="cuda")
        ws = dec.workspace(latent.shape[0], 1, *latent.shape[-2:], len(starts) - 1)
        rc, info = dec.decode_sharded(lat, "width", len(starts) - 1, out, ws, starts)
        torch.cuda.synchronize()
        return out, rc, info

    cases = [(preset(1), (0, 8), "height", False), (preset(1), (0, 3, 8), "height", False),
             (preset(1), tuple(range(9)), "height", False), (preset(1), (0, 3, 8), "width", False),
             (preset(2).with_size(batch=2), (0, 7, 20, 33, 64), "width", False),
             (preset(3), None, "height", False), (preset(3), (0, 1, 2, 64, 127, 128), "height", False),
             (preset(3), None, "height", True), (preset(4), None, "height", False),
             (preset(5), None, "height", False), (preset(5), (0, 1, 29, 30, 60), "height", False)]
    for cfg, starts, axis, fold in cases:
        dec, _ = make_decoder(cfg)
        z = make_latent(cfg)
        starts = starts or cfg.band_starts
        dec.set_norm_fold(fold)
        outs = []
        for poison in (False, True):
            dec.set_halo_poison(poison)
            if axis == "height":
                y, rc, info = gpu_decode(dec, cfg, z, starts)
            else:
                y, rc, info = width_decode(dec, cfg, z, starts)
            assert rc == 0 and info.bands_used == len(starts) - 1
            outs.append((y, info.n_launches))
        (y0, n0), (y1, n1) = outs
        what = (cfg.name, starts, axis, fold)
        assert n1 > n0, what                      # the fills ran
        assert not torch.isnan(y1).any().item(), what
        assert torch.equal(y0, y1), what
        dec.close()
        del outs, y0, y1
    # the tile decode (full tiles in one batch, clipped edge tiles batched per size) on the
    # same switch
    cfg = preset(2).with_size(latent_h=20, latent_w=14)
    dec, _ = make_decoder(cfg)
    z = to_dev(make_latent(cfg), cfg.dtype)
    ws = dec.tiled_workspace(1, 1, 20, 14, 8, 6)
    ys = []
    for poison in (False, True):
        dec.set_halo_poison(poison)
        y = torch.empty(cfg.output_shape(), dtype=torch.float32, device="cuda")
        assert dec.decode_tiled(z, 8, 6, y, ws) == 0
        torch.cuda.synchronize()
        ys.append(y)
    assert not torch.isnan(ys[1]).any().item() and torch.equal(ys[0], ys[1])
    dec.close()


def test_2048_single_band_decode_equals_band_decode(gpu_lib):
    """A 2048 x 2048 decode (256 x 256 latent, the 1024^2 model) as one band: its last
    stages' band buffers exceed 2 GiB (up to 4.3 GB of fp32 stream), beyond a buffer
    resource's range, which the conv kernels never span (each tile addresses its own rows).
    It equals the four-band decode bit for bit."""
    cfg = preset(3).with_size(latent_h=256, latent_w=256, band_starts=(0, 62, 128, 192, 256))
    dec, _ = make_decoder(cfg)
    z = make_latent(cfg)
    y1, rc, _ = gpu_decode(dec, cfg, z, (0, 256))
    assert rc == 0
    y4, rc, info = gpu_decode(dec, cfg, z, cfg.band_starts)
    assert rc == 0 and info.bands_used == 4
    assert list(y1.shape) == [1, 3, 2048, 2048]
    assert torch.isfinite(y1).all()
    assert torch.equal(y1, y4)
    dec.close()


def test_video_band_decode_is_bit_identical_to_full(gpu_lib):
    # the video decoder's causal convs, RMSNorm, temporal upsample and per-frame attention
    # (d = 384: two key halves per query block, merged) compute each element identically
    # on any band table
    cfg = preset(5).with_size(frames=3, latent_h=9, latent_w=12, band_starts=(0, 9))
    dec, _ = make_decoder(cfg, affine="random")
    z = make_latent(cfg)
    ws = dec.workspace(1, 3, 9, 12, 9)
    full, rc, _ = gpu_decode(dec, cfg, z, (0, 9), ws)
    assert rc == 0
    for starts in [(0, 4, 9), (0, 1, 2, 5, 9), tuple(range(10))]:
        y, rc, _ = gpu_decode(dec, cfg, z, starts, ws)
        assert rc == 0 and torch.equal(y, full), starts
    dec.close()


@pytest.mark.parametrize("shape", [(10, 12), (12, 20), (9, 16)])
def test_band_decode_is_bit_identical_to_full(gpu_lib, shape):
    # convs and attention compute each element identically on any band table, and the
    # GroupNorm statistics come from a tiling no band boundary can split: every band
    # table decodes to exactly the full-image result
    h, w = shape
    cfg = preset(3).with_size(latent_h=h, latent_w=w, band_starts=(0, h))
    dec, _ = make_decoder(cfg, affine="random")
    z = make_latent(cfg)
    ws = dec.workspace(1, 1, h, w, h)
    full, _, _ = gpu_decode(dec, cfg, z, (0, h), ws)
    for starts in [(0, 3, h), (0, 1, h), (0, h - 1, h), (0, 2, 5, 7, h), tuple(range(h + 1))]:
        y, rc, _ = gpu_decode(dec, cfg, z, starts, ws)
        assert rc == 0 and torch.equal(y, full), starts
    dec.close()
