"""The band decode that allocates nothing (vaep_decode_bands_noalloc), through the C ABI.

Its workspace is the library's static device scratch; it must return exactly what
vaep_decode_bands returns with a caller workspace (the same kernels on the same inputs),
on two calls in a row whose second is smaller (the scratch keeps the first call's
contents), and reject a decode larger than the scratch before enqueuing anything.
"""
import pytest
import torch

from spatially_sharded_conv_amd import _lib as L
from synth import make_latent, preset
from tests._util import to_dev
from tests.test_gpu_decode import make_decoder

pytestmark = pytest.mark.gpu


def _pair(dec, cfg, z, starts):
    lat = to_dev(z, cfg.dtype)
    b = z.shape[0]
    t = z.shape[2] if z.dim() == 5 else 1
    h, w = z.shape[-2:]
    shape = cfg.output_shape(b, t, h, w)
    ref = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = dec.workspace(b, t, h, w, len(starts) - 1)
    rc, info = dec.decode_bands(lat, starts, ref, ws)
    assert rc == 0
    got = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    rc2, info2 = dec.decode_bands_noalloc(lat, starts, got)
    torch.cuda.synchronize()
    assert rc2 == 0 and info2.bands_used == info.bands_used and info2.n_launches == info.n_launches
    assert info2.workspace_bytes == info.workspace_bytes <= L.load().vaep_noalloc_scratch_bytes()
    return got, ref


@pytest.mark.parametrize("cfg_id", [3, 5])
def test_noalloc_equals_the_workspace_decode(gpu_lib, cfg_id):
    if cfg_id == 3:
        cfg = preset(3).with_size(latent_h=12, latent_w=10, band_starts=(0, 5, 12))
        small = dict(latent_h=7, latent_w=6)
        tables = [(0, 5, 12), (0, 2, 3, 7)]
    else:
        cfg = preset(5).with_size(frames=2, latent_h=5, latent_w=6, band_starts=(0, 2, 5))
        small = dict(latent_h=3, latent_w=4)
        tables = [(0, 2, 5), (0, 1, 3)]
    dec, _ = make_decoder(cfg, affine="random")
    # first call: the larger decode; second: a smaller one on the same scratch
    z1 = make_latent(cfg)
    got, ref = _pair(dec, cfg, z1, tables[0])
    assert torch.equal(got, ref)
    cfg2 = cfg.with_size(**small, band_starts=tables[1])
    z2 = make_latent(cfg2)
    got, ref = _pair(dec, cfg2, z2, tables[1])
    assert torch.equal(got, ref)
    dec.close()


def test_noalloc_rejects_a_decode_larger_than_the_scratch(gpu_lib):
    cfg = preset(3).with_size(latent_h=64, latent_w=64, band_starts=(0, 64))
    dec, _ = make_decoder(cfg)
    lat = to_dev(make_latent(cfg), cfg.dtype)
    need = dec.workspace_bytes(1, 1, 64, 64, 1)
    assert need > L.load().vaep_noalloc_scratch_bytes()
    out = torch.full(cfg.output_shape(), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(L.VaepError) as e:
        dec.decode_bands_noalloc(lat, (0, 64), out)
    assert e.value.code == L.VAEP_ERR_WORKSPACE and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    dec.close()
