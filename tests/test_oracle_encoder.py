"""Pins of the oracle's encoder and tiled encode (CPU only), each against something other
than the oracle's own code: brute-force loops, a closed form built from torch.nn.functional
routines under degenerate weights, and the tile merge's geometry."""
import itertools

import pytest
import torch
import torch.nn.functional as F

from oracle import Precision, downsample_conv, encode_full, encode_tiled
from synth import encoder_param_specs, make_encoder_params, make_image, preset

F64 = torch.float64


def test_downsample_conv_matches_brute_force():
    """y[h][w] = b + sum W[dy][dx] x[2h+dy][2w+dx], rows/columns past the bottom/right edge zero,
    no padding at the top/left -- evaluated element by element."""
    g = torch.Generator().manual_seed(7)
    x = torch.randn(2, 3, 1, 6, 8, generator=g, dtype=F64)
    w = torch.randn(4, 3, 1, 3, 3, generator=g, dtype=F64)
    b = torch.randn(4, generator=g, dtype=F64)
    y = downsample_conv(x, w, b, lambda t: t)
    assert y.shape == (2, 4, 1, 3, 4)
    for n, o, h, c in itertools.product(range(2), range(4), range(3), range(4)):
        s = float(b[o])
        for i, dy, dx in itertools.product(range(3), range(3), range(3)):
            r, q = 2 * h + dy, 2 * c + dx
            if r < 6 and q < 8:
                s += float(w[o, i, 0, dy, dx]) * float(x[n, i, 0, r, q])
        assert abs(float(y[n, o, 0, h, c]) - s) < 1e-12


def _skeleton(cfg):
    """Encoder weights under which every resnet and the attention are identities (zero conv /
    projection weights and biases; shortcuts embed the input channels first), every downsample
    keeps pixel (2h, 2w) (a delta at tap (0, 0), identity over channels)."""
    p = make_encoder_params(cfg, affine="random")
    for name, t in p.items():
        if (".conv1." in name or ".conv2." in name or name.startswith("mid.attn.out.")):
            p[name] = torch.zeros_like(t)
        elif name.endswith(".shortcut.weight"):
            e = torch.zeros_like(t)
            for k in range(t.shape[1]):
                e[k, k, 0, 0] = 1.0
            p[name] = e
        elif name.endswith(".shortcut.bias") or (".downsample." in name and name.endswith(".bias")):
            p[name] = torch.zeros_like(t)
        elif ".downsample." in name and name.endswith(".weight"):
            d = torch.zeros_like(t)
            for k in range(t.shape[0]):
                d[k, k, 0, 0] = 1.0
            p[name] = d
    return p


@pytest.mark.parametrize("i", [1, 2])
def test_encoder_skeleton_closed_form(i):
    """With identity blocks the encoder is quant_conv(conv_out(SiLU(GN(x)))) with x = conv_in(image)
    subsampled by 2 per down stage and zero-extended to the widest channel count -- built here
    from F.conv2d / F.group_norm / F.silu.  Pins the down stages' placement and count, the
    channel growth, the stride-2 sampling phase, and the tail order (norm, SiLU, conv_out,
    quant_conv)."""
    cfg = preset(i).with_size(latent_h=4, latent_w=6) if i == 2 else preset(i)
    p = _skeleton(cfg)
    img = make_image(cfg, batch=1, latent_h=cfg.latent_h, latent_w=cfg.latent_w)
    got = encode_full(cfg, p, img, Precision("f32"))
    d = {k: v.to(F64) for k, v in p.items()}
    x = F.conv2d(img.to(F64), d["conv_in.weight"], d["conv_in.bias"], padding=1)
    for _ in range(cfg.n_stages - 1):
        x = x[:, :, ::2, ::2]
    top = cfg.stage_channels[0]
    x = torch.cat([x, torch.zeros(x.shape[0], top - x.shape[1], *x.shape[2:], dtype=F64)], dim=1)
    x = F.silu(F.group_norm(x, cfg.norm_groups, d["norm_out.weight"], d["norm_out.bias"], eps=cfg.eps))
    x = F.conv2d(x, d["conv_out.weight"], d["conv_out.bias"], padding=1)
    ref = F.conv2d(x, d["quant_conv.weight"], d["quant_conv.bias"])
    assert got.shape == ref.shape == cfg.moments_shape(1, cfg.latent_h, cfg.latent_w)
    err = (got.to(F64) - ref).abs().max().item()
    assert err < 1e-4 * (1 + ref.abs().max().item()), err


def test_tiled_encode_with_one_covering_tile_is_the_full_encode():
    cfg = preset(1)
    p = make_encoder_params(cfg, affine="random")
    img = make_image(cfg)
    full = encode_full(cfg, p, img)
    assert torch.equal(encode_tiled(cfg, p, img, cfg.latent_h, cfg.latent_h), full)
    assert torch.equal(encode_tiled(cfg, p, img, 2 * cfg.latent_h, 3 * cfg.latent_h // 2), full)


def test_tiled_encode_merge_geometry():
    """Tiles of 4 latent rows every 3: the first tile's first 3 x 3 latent block is never
    blended and equals that tile's own encode; the block starting at latent (3, 3) blends the
    upper and left neighbours over 1 row / column, and its inner 2 x 2 is tile (1, 1)'s own
    encode; the result is cropped to the latent size."""
    cfg = preset(1)
    up = 2 ** (cfg.n_stages - 1)
    p = make_encoder_params(cfg, affine="random")
    img = make_image(cfg)
    got = encode_tiled(cfg, p, img, 4, 3)
    assert got.shape == cfg.moments_shape()
    t00 = encode_full(cfg, p, img[:, :, :4 * up, :4 * up].contiguous())
    assert torch.equal(got[:, :, :3, :3], t00[:, :, :3, :3])
    t11 = encode_full(cfg, p, img[:, :, 3 * up:7 * up, 3 * up:7 * up].contiguous())
    assert torch.equal(got[:, :, 4:6, 4:6], t11[:, :, 1:3, 1:3])
    # row 3 of the output is tile (1, 0)'s row 0 cross-faded with weight 1 from tile (0, 0)'s last row
    t10 = encode_full(cfg, p, img[:, :, 3 * up:7 * up, :4 * up].contiguous())
    assert torch.allclose(got[:, :, 3, 1:3], t00[:, :, 3, 1:3].to(F64).to(torch.float32), atol=0, rtol=0)
    assert not torch.equal(t10[:, :, 0, 1:3], t00[:, :, 3, 1:3])


def test_encoder_parameter_list_mirrors_the_decoder():
    """Down stages over the reversed decoder widths with one resnet fewer, a downsample after
    every stage but the last, 2 z output channels and a 1x1 quant_conv."""
    for i in (1, 2, 3, 4):
        cfg = preset(i)
        specs = {s.name: s.shape for s in encoder_param_specs(cfg)}
        widths = tuple(reversed(cfg.stage_channels))
        assert specs["conv_in.weight"] == (widths[0], 3, 3, 3)
        assert sum(1 for n in specs if n.endswith(".downsample.weight")) == cfg.n_stages - 1
        for s, c in enumerate(widths):
            assert f"down{s}.res{cfg.encoder_resnets - 1}.conv2.weight" in specs
            assert f"down{s}.res{cfg.encoder_resnets}.conv2.weight" not in specs
            assert specs[f"down{s}.res0.conv2.weight"] == (c, c, 3, 3)
        assert specs["conv_out.weight"] == (2 * cfg.z_channels, widths[-1], 3, 3)
        assert specs["quant_conv.weight"] == (2 * cfg.z_channels, 2 * cfg.z_channels, 1, 1)
    with pytest.raises(ValueError):
        encoder_param_specs(preset(5))


def test_encoder_resnet_probes():
    """Identity blocks plus two probes, against a closed form:
    * every resnet's conv2 bias is a distinct seeded vector, so each adds its own constant at
      its place (a missing, extra or misplaced resnet changes the sum or its channel range);
    * stage 0's last resnet gets gamma2 = 0 and a conv2 that reads only tap (2, 2), so it
      adds silu(beta2) everywhere but on the stage's last row and column; the stride-2 sampling
      keeps even rows and columns only, so that zero edge survives only if the resnet ran
      after the downsample (it must not: stage 0's downsample follows its resnets)."""
    cfg = preset(1)
    p = _skeleton(cfg)
    g = torch.Generator().manual_seed(11)
    res_bias = {}
    for name in list(p):
        if name.endswith(".conv2.bias"):
            res_bias[name[: -len(".conv2.bias")]] = torch.randn(p[name].shape, generator=g)
            p[name] = res_bias[name[: -len(".conv2.bias")]].clone()
    probe = f"down0.res{cfg.encoder_resnets - 1}"
    c0 = p[probe + ".conv2.weight"].shape[0]
    w = torch.zeros_like(p[probe + ".conv2.weight"])
    for k in range(c0):
        w[k, k, 2, 2] = 1.0
    p[probe + ".conv2.weight"] = w
    p[probe + ".norm2.weight"] = torch.zeros(c0)
    beta = torch.randn(c0, generator=g)
    p[probe + ".norm2.bias"] = beta
    img = make_image(cfg)
    got = encode_full(cfg, p, img, Precision("f32")).to(F64)

    d = {k: v.to(F64) for k, v in p.items()}
    x = F.conv2d(img.to(F64), d["conv_in.weight"], d["conv_in.bias"], padding=1)
    widths = tuple(reversed(cfg.stage_channels))
    for s, c in enumerate(widths):
        for j in range(cfg.encoder_resnets):
            name = f"down{s}.res{j}"
            if x.shape[1] < c:
                x = torch.cat([x, torch.zeros(x.shape[0], c - x.shape[1], *x.shape[2:], dtype=F64)], dim=1)
            x = x + res_bias[name].to(F64).view(1, -1, 1, 1)
            if name == probe:
                pat = torch.zeros_like(x[:1])
                pat[:, :, :-1, :-1] = F.silu(beta.to(F64)).view(1, -1, 1, 1)
                x = x + pat
        if s < len(widths) - 1:
            x = x[:, :, ::2, ::2]
    for name in ("mid.res0", "mid.res1"):
        x = x + res_bias[name].to(F64).view(1, -1, 1, 1)
    x = F.silu(F.group_norm(x, cfg.norm_groups, d["norm_out.weight"], d["norm_out.bias"], eps=cfg.eps))
    x = F.conv2d(x, d["conv_out.weight"], d["conv_out.bias"], padding=1)
    ref = F.conv2d(x, d["quant_conv.weight"], d["quant_conv.bias"])
    err = (got - ref).abs().max().item()
    assert err < 1e-4 * (1 + ref.abs().max().item()), err
