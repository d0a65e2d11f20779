"""Pins of the oracle's decoder wiring (CPU only).

The pages name the decoders ("AutoencoderKL, 2D CNN" and "Wan, causal 3D CNN"
in the feature page's model table) but print none of their blocks, so the
block order and channel plan are a reading (conv_in -> mid resnet, attention,
resnet -> up stages -> norm -> SiLU -> conv_out; resnet = conv(SiLU(N(x)))
twice plus the identity or a 1x1 shortcut; a nearest-2x + 3x3 conv after every
stage but the last; Wan: causal 3x3x3 convs, channel RMSNorm, per-frame
attention and a causal temporal upsample in the first two stages).  These tests
pin the oracle's graph to that reading with degenerate weights whose decode has
a closed form built from ``torch.nn.functional`` primitives:

* skeleton: every resnet and attention weight and bias zero, each 1x1 shortcut
  the selection of its first ``co`` input channels, each upsample conv a centre
  tap identity, each time conv an identity on the current frame for both
  halves.  Every block is then the identity (or nearest-2x, or a frame
  repeat), and the decode collapses to conv_out(SiLU(N(up^k(conv_in(z))))).
* one live block (or two, for an order): that block keeps seeded random
  weights, the rest is skeleton; the expected decode is the skeleton chain
  with the block's own definition at its place in the block list below.
* Wan frame labels: latent frame t carries a one-hot channel t; the decoded
  frames carry labels 0,1,1,1,1,2,2,2,2,... (T: 5 -> 9 -> 17).

A planted mistake in the oracle's wiring (checked at the end of this file by
patching the oracle, on the CPU) makes these tests fail.
"""
import functools
import math

import pytest
import torch
import torch.nn.functional as F

import oracle.decoder as odec
from oracle import Precision, decode_bands, decode_full
from synth import make_latent, make_params, preset

F64 = torch.float64

# Block lists of the reading, in decode order: (kind, name).  Written out by hand per
# decoder so that a reader can check them against the reading above.
KL_TINY = [("resnet", "mid.res0"), ("attn", "mid.attn"), ("resnet", "mid.res1"),
           ("resnet", "up0.res0"), ("resnet", "up0.res1"), ("up", "up0.upsample"),
           ("resnet", "up1.res0"), ("resnet", "up1.res1")]
KL_FLUX = [("resnet", "mid.res0"), ("attn", "mid.attn"), ("resnet", "mid.res1")]
for _i in range(4):
    KL_FLUX += [("resnet", f"up{_i}.res{_j}") for _j in range(3)]
    if _i < 3:
        KL_FLUX.append(("up", f"up{_i}.upsample"))
WAN = [("resnet", "mid.res0"), ("attn", "mid.attn"), ("resnet", "mid.res1"),
       ("resnet", "up0.res0"), ("resnet", "up0.res1"), ("time", "up0.time_conv"), ("up", "up0.upsample"),
       ("resnet", "up1.res0"), ("resnet", "up1.res1"), ("time", "up1.time_conv"), ("up", "up1.upsample"),
       ("resnet", "up2.res0"), ("resnet", "up2.res1"), ("up", "up2.upsample"),
       ("resnet", "up3.res0"), ("resnet", "up3.res1")]


# ---------------------------------------------------------------- degenerate weights

def _identity_taps(co, ci, kernel, tap):
    """Weight [co, ci, *kernel] that copies input channel c to output channel c (c < min) at ``tap``."""
    w = torch.zeros((co, ci) + tuple(kernel))
    for c in range(min(co, ci)):
        w[(c, c) + tuple(tap)] = 1.0
    return w


_SUBLAYERS = {"conv1", "conv2", "norm1", "norm2", "shortcut", "q", "k", "v", "out", "norm"}


def _block_of(name):
    """'mid.res0.conv1.weight' -> 'mid.res0'; 'up0.upsample.bias' -> 'up0.upsample'."""
    parts = name.split(".")[:-1]
    if len(parts) > 1 and parts[-1] in _SUBLAYERS:
        parts = parts[:-1]
    return ".".join(parts)


@functools.lru_cache(maxsize=4)
def _random_params(cfg):
    return make_params(cfg, affine="random")


def skeleton_params(cfg, live=()):
    """Seeded random parameters (random affine terms too); blocks not in ``live`` made degenerate."""
    p = {k: v.clone() for k, v in _random_params(cfg).items()}
    for name in list(p):
        block = _block_of(name)
        if block in live or block in ("conv_in", "norm_out", "conv_out"):
            continue
        t = p[name]
        if ".conv1." in name or ".conv2." in name or name.startswith("mid.attn.") and ".norm." not in name:
            p[name] = torch.zeros_like(t)
        elif ".shortcut." in name:
            p[name] = (torch.zeros_like(t) if name.endswith("bias")
                       else _identity_taps(t.shape[0], t.shape[1], t.shape[2:], (0,) * (t.dim() - 2)))
        elif name.endswith("upsample.weight"):
            p[name] = _identity_taps(t.shape[0], t.shape[1], (3, 3), (1, 1))
        elif name.endswith("upsample.bias") or name.endswith("time_conv.bias"):
            p[name] = torch.zeros_like(t)
        elif name.endswith("time_conv.weight"):
            c = t.shape[1]
            w = torch.zeros_like(t)
            for k in range(c):      # both halves copy the current frame (the last causal tap)
                w[k, k, 2, 0, 0] = 1.0
                w[c + k, k, 2, 0, 0] = 1.0
            p[name] = w
    return p


# ---------------------------------------------------------------- the reading, in F primitives

class Ref:
    """Each block of the reading written with torch.nn.functional primitives (float64)."""

    def __init__(self, cfg, p):
        self.cfg = cfg
        self.p = {k: v.to(F64) for k, v in p.items()}
        self.video = cfg.is_video

    # --- operators
    def conv3(self, x, name):
        w, b = self.p[name + ".weight"], self.p[name + ".bias"]
        if self.video:      # causal: two zero frames in front, 1 zero row / column each side
            return F.conv3d(F.pad(x, (1, 1, 1, 1, 2, 0)), w, b)
        return F.conv2d(x, w, b, padding=1)

    def conv1(self, x, name):
        w, b = self.p[name + ".weight"], self.p[name + ".bias"]
        return F.conv3d(x, w, b) if self.video else F.conv2d(x, w, b)

    def norm(self, x, name, act):
        if self.video:
            y = F.rms_norm(x.movedim(1, -1), (x.shape[1],), self.p[name + ".weight"],
                           self.cfg.eps).movedim(-1, 1)
        else:
            y = F.group_norm(x, self.cfg.norm_groups, self.p[name + ".weight"], self.p[name + ".bias"],
                             self.cfg.eps)
        return F.silu(y) if act else y

    def frames(self, x):
        """[B, C, (T,) H, W] -> list of [B, C, H, W] images (one per frame)."""
        return [x[:, :, t] for t in range(x.shape[2])] if self.video else [x]

    def unframes(self, imgs):
        return torch.stack(imgs, dim=2) if self.video else imgs[0]

    # --- blocks, live
    def resnet(self, x, pre):
        h = self.conv3(self.norm(x, pre + ".norm1", True), pre + ".conv1")
        h = self.conv3(self.norm(h, pre + ".norm2", True), pre + ".conv2")
        sc = self.conv1(x, pre + ".shortcut") if pre + ".shortcut.weight" in self.p else x
        return h + sc

    def attn(self, x, pre):
        h = self.norm(x, pre + ".norm", False)
        out = []
        for xi, hi in zip(self.frames(x), self.frames(h)):
            b, c, hh, ww = xi.shape
            tok = hi.flatten(2).transpose(1, 2)                       # [B, HW, C]
            q, k, v = (F.linear(tok, self.p[f"{pre}.{s}.weight"], self.p[f"{pre}.{s}.bias"]) for s in "qkv")
            o = F.scaled_dot_product_attention(q[:, None], k[:, None], v[:, None])[:, 0]
            y = F.linear(o, self.p[pre + ".out.weight"], self.p[pre + ".out.bias"])
            out.append(xi + y.transpose(1, 2).reshape(b, c, hh, ww))
        return self.unframes(out)

    def up(self, x, pre):
        imgs = [F.conv2d(F.interpolate(xi, scale_factor=2, mode="nearest"), self.p[pre + ".weight"],
                         self.p[pre + ".bias"], padding=1) for xi in self.frames(x)]
        return self.unframes(imgs)

    def time(self, x, pre):
        c = x.shape[1]
        z = F.conv3d(F.pad(x, (0, 0, 0, 0, 2, 0)), self.p[pre + ".weight"], self.p[pre + ".bias"])
        pairs = torch.stack([z[:, :c, 1:], z[:, c:, 1:]], dim=3).flatten(2, 3)   # z1a z1b z2a z2b ...
        return torch.cat([x[:, :, :1], pairs], dim=2)

    # --- blocks, degenerate (skeleton)
    @staticmethod
    def skel(kind, x, co):
        if kind == "resnet":
            return x[:, :co]                               # identity / first-co-channel shortcut
        if kind == "attn":
            return x
        if kind == "up":
            if x.dim() == 5:
                return x.repeat_interleave(2, dim=3).repeat_interleave(2, dim=4)
            return F.interpolate(x, scale_factor=2, mode="nearest")
        if kind == "time":                                 # frames x0, x1, x1, x2, x2, ...
            idx = [0] + [t for t in range(1, x.shape[2]) for _ in range(2)]
            return x[:, :, idx]
        raise ValueError(kind)

    def decode(self, z, blocks, live):
        x = z.to(F64)
        if not self.video:
            x = x[:, :, 0] if x.dim() == 5 else x
        x = self.conv3(x, "conv_in")
        for kind, name in blocks:
            if name in live:
                x = getattr(self, kind)(x, name)
            else:
                co = self.p[name + ".conv2.weight"].shape[0] if kind == "resnet" else x.shape[1]
                x = self.skel(kind, x, co)
        x = self.conv3(self.norm(x, "norm_out", True), "conv_out")
        return x


def _err(a, b):
    d = a.double() - b.double()
    return d.abs().max().item(), (d.norm() / b.double().norm()).item()


def wiring_error(cfg, blocks, live):
    p = skeleton_params(cfg, live)
    z = make_latent(cfg)
    got = decode_full(cfg, p, z, Precision("f32"))
    want = Ref(cfg, p).decode(z, blocks, set(live))
    assert got.shape == want.shape, (got.shape, want.shape)
    return _err(got, want)


# fp32 storage between operators, float64 sums: the oracle agrees with the float64
# composition to float32 rounding of each stored tensor.
BAR = 1e-5

CFG_TINY = preset(1)
CFG_FLUX = preset(3).with_size(latent_h=4, latent_w=3, band_starts=(0, 1, 4))
CFG_WAN = preset(5).with_size(frames=3, latent_h=3, latent_w=4, band_starts=(0, 1, 3))


@pytest.mark.parametrize("cfg,blocks", [(CFG_TINY, KL_TINY), (CFG_FLUX, KL_FLUX), (CFG_WAN, WAN)],
                         ids=["kl-tiny", "kl-flux", "wan"])
def test_skeleton_collapses_to_the_trunk(cfg, blocks):
    """Every block degenerate: decode = conv_out(SiLU(N(up^k(conv_in(z)))))."""
    ma, rl = wiring_error(cfg, blocks, live=())
    assert rl <= BAR, (ma, rl)
    # and that trunk is not trivially zero
    p = skeleton_params(cfg)
    assert decode_full(cfg, p, make_latent(cfg), Precision("f32")).abs().max() > 1e-2


@pytest.mark.parametrize("name", [n for _, n in KL_TINY])
def test_one_live_block_kl_tiny(name):
    ma, rl = wiring_error(CFG_TINY, KL_TINY, live=(name,))
    assert rl <= BAR, (name, ma, rl)


@pytest.mark.parametrize("name", ["mid.attn", "up0.res0", "up1.upsample", "up2.res0", "up3.res0",
                                  "up3.res2"])
def test_one_live_block_kl_flux(name):
    ma, rl = wiring_error(CFG_FLUX, KL_FLUX, live=(name,))
    assert rl <= BAR, (name, ma, rl)


@pytest.mark.parametrize("live", [("mid.res0",), ("mid.attn",), ("up0.res1",), ("up0.time_conv",),
                                  ("up0.upsample",), ("up2.res0",), ("up3.res1",),
                                  ("up0.res1", "up0.time_conv"), ("up1.res1", "up1.time_conv"),
                                  ("up1.time_conv", "up1.upsample", "up2.res0")])
def test_live_blocks_wan(live):
    ma, rl = wiring_error(CFG_WAN, WAN, live=live)
    assert rl <= BAR, (live, ma, rl)


def test_all_blocks_live_kl_tiny():
    """Every block live: the oracle equals the composition of the per-block definitions."""
    ma, rl = wiring_error(CFG_TINY, KL_TINY, live=tuple(n for _, n in KL_TINY))
    assert rl <= BAR, (ma, rl)


def test_residual_bias_reaches_the_tail():
    """One nonzero conv2 bias, all else degenerate: the block adds that constant to its input."""
    cfg = CFG_TINY
    p = skeleton_params(cfg)
    bias = torch.linspace(-1.0, 1.0, p["up0.res1.conv2.bias"].numel())
    p["up0.res1.conv2.bias"] = bias
    z = make_latent(cfg)
    got = decode_full(cfg, p, z, Precision("f32"))
    ref = Ref(cfg, p)
    x = ref.conv3(z.to(F64), "conv_in") + bias.to(F64).view(1, -1, 1, 1)
    x = F.interpolate(x, scale_factor=2, mode="nearest")[:, :32]
    want = ref.conv3(ref.norm(x, "norm_out", True), "conv_out")
    assert _err(got, want)[1] <= BAR


def test_wan_frame_labels():
    """Latent frame t one-hot in channel t: decoded frames carry 0,1,1,1,1,2,2,2,2,... (5 -> 9 -> 17)."""
    cfg = preset(5).with_size(frames=5, latent_h=2, latent_w=2, band_starts=(0, 2))
    p = skeleton_params(cfg)
    c_top = cfg.top_channels
    p["conv_in.weight"] = _identity_taps(c_top, cfg.z_channels, (3, 3, 3), (2, 1, 1))
    p["conv_in.bias"] = torch.zeros(c_top)
    p["norm_out.weight"] = torch.ones_like(p["norm_out.weight"])
    w = torch.zeros_like(p["conv_out.weight"])
    w[0, :16, 2, 1, 1] = torch.arange(1, 17, dtype=torch.float32)   # output channel 0 = label + 1
    p["conv_out.weight"] = w
    p["conv_out.bias"] = torch.zeros(3)
    z = torch.zeros(cfg.latent_shape())
    for t in range(5):
        z[:, t, t] = 1.0
    y = decode_full(cfg, p, z, Precision("f32"))
    assert y.shape == (1, 3, 17, 16, 16)
    c_out = p["norm_out.weight"].numel()
    unit = 1.0 / math.sqrt(1.0 / c_out + cfg.eps)          # RMSNorm of a one-hot vector
    unit = unit / (1.0 + math.exp(-unit))                   # SiLU
    labels = y[0, 0] / unit - 1.0
    assert (labels - labels.round()).abs().max() < 1e-4
    want = [0] + [1 + (f - 1) // 4 for f in range(1, 17)]
    assert labels.round().flatten(1).min(dim=1).values.tolist() == want
    assert labels.round().flatten(1).max(dim=1).values.tolist() == want
    assert y[0, 1:].abs().max() == 0


def test_band_decode_of_a_live_block():
    """The band-mode graph carries the same wiring (uneven bands, attention live)."""
    cfg = CFG_FLUX
    p = skeleton_params(cfg, live=("mid.attn", "up1.upsample"))
    z = make_latent(cfg)
    got = decode_bands(cfg, p, z, cfg.band_starts, Precision("f32"))
    want = Ref(cfg, p).decode(z, KL_FLUX, {"mid.attn", "up1.upsample"})
    assert _err(got, want)[1] <= BAR


# ---------------------------------------------------------------- planted mistakes

def _resnet_no_silu2(o, p, prefix, x):
    h = o.norm(x, p, prefix + ".norm1", act=True)
    h = o.conv(h, p[prefix + ".conv1.weight"], p[prefix + ".conv1.bias"])
    h = o.norm(h, p, prefix + ".norm2", act=False)
    sc = o.conv(x, p[prefix + ".shortcut.weight"], p[prefix + ".shortcut.bias"]) \
        if prefix + ".shortcut.weight" in p else x
    return o.conv(h, p[prefix + ".conv2.weight"], p[prefix + ".conv2.bias"], residual=sc)


def _resnet_shortcut_of_h(o, p, prefix, x):
    h = o.norm(x, p, prefix + ".norm1", act=True)
    h = o.conv(h, p[prefix + ".conv1.weight"], p[prefix + ".conv1.bias"])
    sc = o.conv(x, p[prefix + ".shortcut.weight"], p[prefix + ".shortcut.bias"]) \
        if prefix + ".shortcut.weight" in p else h
    h = o.norm(h, p, prefix + ".norm2", act=True)
    return o.conv(h, p[prefix + ".conv2.weight"], p[prefix + ".conv2.bias"], residual=sc)


def _resnet_no_residual(o, p, prefix, x):
    h = o.norm(x, p, prefix + ".norm1", act=True)
    h = o.conv(h, p[prefix + ".conv1.weight"], p[prefix + ".conv1.bias"])
    h = o.norm(h, p, prefix + ".norm2", act=True)
    if prefix + ".shortcut.weight" in p:
        return o.conv(h, p[prefix + ".conv2.weight"], p[prefix + ".conv2.bias"],
                      residual=o.conv(x, p[prefix + ".shortcut.weight"], p[prefix + ".shortcut.bias"]))
    return o.conv(h, p[prefix + ".conv2.weight"], p[prefix + ".conv2.bias"])


@pytest.mark.parametrize("mistake", ["no_silu2", "shortcut_of_h", "no_residual", "upsample_before_resnets",
                                     "tail_without_silu", "time_after_upsample_stage"])
def test_planted_wiring_mistakes_are_caught(monkeypatch, mistake):
    """Each plausible wiring slip, planted in the oracle, fails one of the pins above."""
    graph = odec._graph
    if mistake == "no_silu2":
        monkeypatch.setattr(odec, "_resnet", _resnet_no_silu2)
    elif mistake == "shortcut_of_h":
        monkeypatch.setattr(odec, "_resnet", _resnet_shortcut_of_h)
    elif mistake == "no_residual":
        monkeypatch.setattr(odec, "_resnet", _resnet_no_residual)
    elif mistake == "upsample_before_resnets":
        def g(o, cfg, p, latent):
            x = o.conv(o.enter(latent), p["conv_in.weight"], p["conv_in.bias"])
            x = odec._resnet(o, p, "mid.res0", x)
            x = o.attention(x, p)
            x = odec._resnet(o, p, "mid.res1", x)
            for i in range(cfg.n_stages):
                if cfg.stage_upsamples(i):
                    x = o.conv(o.upsample(x), p[f"up{i}.upsample.weight"], p[f"up{i}.upsample.bias"],
                               causal=False)
                for j in range(cfg.resnets_per_stage):
                    x = odec._resnet(o, p, f"up{i}.res{j}", x)
            x = o.norm(x, p, "norm_out", act=True)
            return o.leave(o.conv(x, p["conv_out.weight"], p["conv_out.bias"]))
        monkeypatch.setattr(odec, "_graph", g)
    elif mistake == "tail_without_silu":
        def g(o, cfg, p, latent):
            orig = o.norm
            o.norm = lambda x, p_, prefix, act: orig(x, p_, prefix, act and prefix != "norm_out")
            return graph(o, cfg, p, latent)
        monkeypatch.setattr(odec, "_graph", g)
    elif mistake == "time_after_upsample_stage":
        # the temporal upsample one stage late (stages 1 and 2 instead of 0 and 1)
        def g(o, cfg, p, latent):
            x = o.conv(o.enter(latent), p["conv_in.weight"], p["conv_in.bias"])
            x = odec._resnet(o, p, "mid.res0", x)
            x = o.attention(x, p)
            x = odec._resnet(o, p, "mid.res1", x)
            for i in range(cfg.n_stages):
                for j in range(cfg.resnets_per_stage):
                    x = odec._resnet(o, p, f"up{i}.res{j}", x)
                if cfg.is_video and i in (1, 2):
                    k = i - 1
                    x = o.temporal_upsample(x, p[f"up{k}.time_conv.weight"], p[f"up{k}.time_conv.bias"])
                if cfg.stage_upsamples(i):
                    x = o.conv(o.upsample(x), p[f"up{i}.upsample.weight"], p[f"up{i}.upsample.bias"],
                               causal=False)
            x = o.norm(x, p, "norm_out", act=True)
            return o.leave(o.conv(x, p["conv_out.weight"], p["conv_out.bias"]))
        monkeypatch.setattr(odec, "_graph", g)

    caught = []
    if mistake == "time_after_upsample_stage":
        cases = [(CFG_WAN, WAN, ("up0.res1", "up0.time_conv")), (CFG_WAN, WAN, ("up1.res1", "up1.time_conv"))]
    else:
        cases = [(CFG_TINY, KL_TINY, ())] + [(CFG_TINY, KL_TINY, (n,)) for _, n in KL_TINY]
    for cfg, blocks, live in cases:
        try:
            caught.append(wiring_error(cfg, blocks, live)[1] > BAR)
        except (AssertionError, RuntimeError):
            caught.append(True)      # a shape mismatch is caught too
    assert any(caught), mistake
