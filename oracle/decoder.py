"""Decoder graphs of the oracle: plain full-image forward and a separate band mode.

The decoder structure (a reading of "AutoencoderKL, 2D CNN" and "Wan, causal
3D CNN" in the feature page's model table; the pages do not print the
blocks):

* ``conv_in`` -> mid block (resnet, single-head attention, resnet) -> up
  stages -> norm_out -> SiLU -> ``conv_out`` (3 channels).
* resnet(ci -> co): h = conv3(SiLU(N1(x))); h = conv3(SiLU(N2(h)));
  y = h + (x if ci == co else conv1x1(x)).
* up stage i: ``resnets_per_stage`` resnets (the first changes channels);
  video stages below ``temporal_up_stages`` add a causal temporal upsample;
  every stage but the last ends with nearest-2x followed by a 3x3 conv
  (per frame for video).
* N is GroupNorm for 2-D decoders and channel RMSNorm for the video decoder;
  2-D attention spans the whole image, video attention spans one frame.

``decode_full`` is the plain whole-tensor forward.  ``decode_bands`` runs the
same graph on disjoint latent row bands (or column bands: the width-sharded
mode) as the pages describe: band rows double with every upsample, convs read
kernel-radius halo rows from the neighbouring bands' buffers, GroupNorm merges
local moments with element-count weights, attention uses the band's Q against
K/V concatenated from all bands, and everything else stays local.  The final
output is the bands' rows (columns) stacked in order (the leader gather).
``choose_axis`` is the per-request ``auto`` policy of the strategy page.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Sequence

import torch

from . import ops

F64 = torch.float64


@dataclass(frozen=True)
class Precision:
    """Rounding of materialised tensors.

    ``storage='f32'``: every tensor is float32.  ``storage='bf16'``: the
    operands of the matrix products -- normalised activations (norm and SiLU
    outputs) and the attention Q, K, V and attention output -- are rounded to
    bfloat16 (round to nearest even); every convolution / projection output
    (the residual stream, conv1 outputs, shortcuts, the decoded image) stays
    float32, i.e. it is the float32 accumulation itself.  Weights and the latent
    arrive bf16-rounded from the generator.
    """
    storage: str = "f32"

    def finish(self, x: torch.Tensor, kind: str = "operand") -> torch.Tensor:
        """Round a float64 result: kind 'operand' (bf16 when storage is bf16) or 'acc' (float32)."""
        y = x.to(torch.float32)
        if self.storage == "bf16" and kind == "operand":
            y = y.to(torch.bfloat16).to(torch.float32)
        return y

    def acc(self, x: torch.Tensor) -> torch.Tensor:
        return self.finish(x, "acc")


def _as5d(w: torch.Tensor) -> torch.Tensor:
    """2-D conv weight [Co, Ci, kh, kw] -> [Co, Ci, 1, kh, kw]."""
    return w if w.dim() == 5 else w.unsqueeze(2)


def _tokens(x: torch.Tensor, n: int, t: int) -> torch.Tensor:
    """Tokens of image n, frame t in row-major (h, w) order: [H*W, C]."""
    return x[n, :, t].reshape(x.shape[1], -1).T


class _Ops:
    def __init__(self, cfg, prec: Precision):
        self.cfg = cfg
        self.prec = prec
        self.video = cfg.is_video
        self.fin = prec.finish       # operands of matrix products
        self.acc = prec.acc          # conv / projection outputs


class FullOps(_Ops):
    """Whole-image operators."""

    def conv(self, x, w, b, causal=None, residual=None):
        causal = self.video and w.dim() == 5 if causal is None else causal
        return ops.conv_full(x, _as5d(w), b, causal, self.acc, residual)

    def norm(self, x, p, prefix, act):
        if self.video:
            return self.fin(ops.rmsnorm(x, p[prefix + ".weight"], self.cfg.eps, act))
        _, mean, var = ops.groupnorm_moments(x, self.cfg.norm_groups)
        return self.fin(ops.groupnorm_apply(x, mean, var, p[prefix + ".weight"],
                                            p[prefix + ".bias"], self.cfg.eps, act))

    def attention(self, x, p):
        h = self.norm(x, p, "mid.attn.norm", act=False)
        c = x.shape[1]
        y = torch.empty_like(x)
        for n in range(x.shape[0]):
            for t in range(x.shape[2]):
                tok = _tokens(h, n, t).to(F64)
                q, k, v = (self.fin(tok @ p[f"mid.attn.{s}.weight"].to(F64).T
                                    + p[f"mid.attn.{s}.bias"].to(F64)) for s in "qkv")
                o = self.fin(ops.attention_rows(q, k, v, 1.0 / math.sqrt(c)))
                proj = o.to(F64) @ p["mid.attn.out.weight"].to(F64).T + p["mid.attn.out.bias"].to(F64)
                res = _tokens(x, n, t).to(F64) + proj
                y[n, :, t] = self.acc(res).T.reshape(c, x.shape[3], x.shape[4])
        return y

    def upsample(self, x):
        return ops.upsample_nearest2x(x)

    def temporal_upsample(self, x, w, b):
        z = ops.conv_full(x, w, b, True, self.acc)
        return ops.temporal_upsample_interleave(x, z)

    def enter(self, z):
        return z.unsqueeze(2) if z.dim() == 4 else z

    def leave(self, y):
        return y[:, :, 0] if not self.video else y


class BandOps(_Ops):
    """Per-band operators; an activation is the list of band tensors in band order.

    ``axis`` 3 cuts latent rows (height bands), 4 cuts latent columns (width
    bands); every other rule is the same on either axis.
    """

    def __init__(self, cfg, prec, starts: Sequence[int], axis: int = 3):
        super().__init__(cfg, prec)
        assert axis in (3, 4)
        self.starts = list(starts)
        self.axis = axis

    def conv(self, xb, w, b, causal=None, residual=None):
        causal = self.video and w.dim() == 5 if causal is None else causal
        w5 = _as5d(w)
        return [ops.conv_band(xb, i, w5, b, causal, self.acc,
                              None if residual is None else residual[i], axis=self.axis)
                for i in range(len(xb))]

    def norm(self, xb, p, prefix, act):
        if self.video:   # channel-only normalisation: local to each band
            return [self.fin(ops.rmsnorm(x, p[prefix + ".weight"], self.cfg.eps, act)) for x in xb]
        local = [ops.groupnorm_moments(x, self.cfg.norm_groups) for x in xb]
        mean, var = ops.merge_moments([l[0] for l in local], [l[1] for l in local],
                                      [l[2] for l in local])
        return [self.fin(ops.groupnorm_apply(x, mean, var, p[prefix + ".weight"],
                                             p[prefix + ".bias"], self.cfg.eps, act)) for x in xb]

    def attention(self, xb, p):
        hb = self.norm(xb, p, "mid.attn.norm", act=False)
        c = xb[0].shape[1]
        outs = [torch.empty_like(x) for x in xb]
        for n in range(xb[0].shape[0]):
            for t in range(xb[0].shape[2]):
                qs, ks, vs = [], [], []
                for h in hb:     # local projections on each band
                    tok = _tokens(h, n, t).to(F64)
                    q, k, v = (self.fin(tok @ p[f"mid.attn.{s}.weight"].to(F64).T
                                        + p[f"mid.attn.{s}.bias"].to(F64)) for s in "qkv")
                    qs.append(q)
                    ks.append(k)
                    vs.append(v)
                k_all = torch.cat(ks, dim=0)   # the gathered global K/V, bands in band order
                v_all = torch.cat(vs, dim=0)
                for i, x in enumerate(xb):
                    o = self.fin(ops.attention_rows(qs[i], k_all, v_all, 1.0 / math.sqrt(c)))
                    proj = (o.to(F64) @ p["mid.attn.out.weight"].to(F64).T
                            + p["mid.attn.out.bias"].to(F64))
                    res = _tokens(x, n, t).to(F64) + proj
                    outs[i][n, :, t] = self.acc(res).T.reshape(c, x.shape[3], x.shape[4])
        return outs

    def upsample(self, xb):
        return [ops.upsample_nearest2x(x) for x in xb]

    def temporal_upsample(self, xb, w, b):
        out = []
        for x in xb:    # the whole time axis lives on every band and the kernel is 1x1 in space
            z = ops.conv_band([x], 0, w, b, True, self.acc)
            out.append(ops.temporal_upsample_interleave(x, z))
        return out

    def enter(self, z):
        z5 = z.unsqueeze(2) if z.dim() == 4 else z
        s = self.starts
        return [z5.narrow(self.axis, s[i], s[i + 1] - s[i]).contiguous() for i in range(len(s) - 1)]

    def leave(self, yb):
        y = torch.cat(yb, dim=self.axis)
        return y[:, :, 0] if not self.video else y


def _resnet(o, p, prefix, x):
    h = o.norm(x, p, prefix + ".norm1", act=True)
    h = o.conv(h, p[prefix + ".conv1.weight"], p[prefix + ".conv1.bias"])
    h = o.norm(h, p, prefix + ".norm2", act=True)
    if prefix + ".shortcut.weight" in p:
        sc = o.conv(x, p[prefix + ".shortcut.weight"], p[prefix + ".shortcut.bias"])
    else:
        sc = x
    return o.conv(h, p[prefix + ".conv2.weight"], p[prefix + ".conv2.bias"], residual=sc)


def _graph(o: _Ops, cfg, p: Dict[str, torch.Tensor], latent: torch.Tensor):
    x = o.enter(latent)
    x = o.conv(x, p["conv_in.weight"], p["conv_in.bias"])
    x = _resnet(o, p, "mid.res0", x)
    x = o.attention(x, p)
    x = _resnet(o, p, "mid.res1", x)
    for i in range(cfg.n_stages):
        for j in range(cfg.resnets_per_stage):
            x = _resnet(o, p, f"up{i}.res{j}", x)
        if cfg.stage_time_upsamples(i):
            x = o.temporal_upsample(x, p[f"up{i}.time_conv.weight"], p[f"up{i}.time_conv.bias"])
        if cfg.stage_upsamples(i):
            x = o.upsample(x)
            x = o.conv(x, p[f"up{i}.upsample.weight"], p[f"up{i}.upsample.bias"], causal=False)
    x = o.norm(x, p, "norm_out", act=True)
    x = o.conv(x, p["conv_out.weight"], p["conv_out.bias"])
    return o.leave(x)


def decode_full(cfg, params: Dict[str, torch.Tensor], latent: torch.Tensor,
                prec: Precision = None) -> torch.Tensor:
    """Plain full-image decode of ``latent`` (float32 tensor) -> float32 output."""
    prec = prec or Precision(cfg.dtype)
    with torch.no_grad():
        return _graph(FullOps(cfg, prec), cfg, params, latent)


def decode_bands(cfg, params: Dict[str, torch.Tensor], latent: torch.Tensor,
                 starts: Sequence[int], prec: Precision = None, axis: str = "height") -> torch.Tensor:
    """Band-mode decode on latent bands [starts[i], starts[i+1]) of the given axis.

    ``axis="height"`` cuts latent rows, ``axis="width"`` latent columns.
    """
    prec = prec or Precision(cfg.dtype)
    dim = {"height": 3, "width": 4}[axis]
    s = list(starts)
    assert s[0] == 0 and s[-1] == latent.shape[dim - 5] and all(a < b for a, b in zip(s, s[1:]))
    with torch.no_grad():
        return _graph(BandOps(cfg, prec, s, dim), cfg, params, latent)


def choose_axis(latent_h: int, latent_w: int, n_shards: int) -> str:
    """The ``auto`` strategy of the Wan spatial-shard decode, per request.

    Strategy page, "Strategy Selection Contract" (the ``auto`` row: tile when
    ineligible) and the Wan spatial-shard notes: auto takes the longer axis
    that can cover every shard, width winning ties; when neither axis can
    cover the shards it uses the tile decode.  A shard needs at least one
    latent row (the kernel radius at the latent level), so an axis covers
    ``n_shards`` when its length is at least ``n_shards``.  One shard is the
    plain dense decode (a reading: there is nothing to shard).  Returns
    "height", "width", "tile" or "dense".
    """
    assert n_shards >= 1
    if n_shards == 1:
        return "dense"
    cover_h, cover_w = latent_h >= n_shards, latent_w >= n_shards
    if cover_w and (latent_w >= latent_h or not cover_h):
        return "width"
    if cover_h:
        return "height"
    return "tile"


# Tile geometry of the tile strategy (a reading: the strategy page names the tile
# attributes but not their values): latent tiles of 32 rows and columns every 24.
AUTO_TILE, AUTO_TILE_STRIDE = 32, 24


def even_starts(length: int, n_shards: int) -> List[int]:
    """Shard boundaries splitting ``length`` into n nearly equal parts, larger parts first."""
    q, r = divmod(length, n_shards)
    starts = [0]
    for i in range(n_shards):
        starts.append(starts[-1] + q + (1 if i < r else 0))
    return starts


def decode_auto(cfg, params: Dict[str, torch.Tensor], latent: torch.Tensor, n_shards: int,
                prec: Precision = None):
    """Decode with the strategy ``choose_axis`` picks (even shards, or the tile decode);
    returns (output, strategy)."""
    from .tiled import decode_tiled
    h, w = latent.shape[-2:]
    axis = choose_axis(h, w, n_shards)
    if axis == "dense":
        return decode_full(cfg, params, latent, prec), axis
    if axis == "tile":
        return decode_tiled(cfg, params, latent, AUTO_TILE, AUTO_TILE_STRIDE, prec), axis
    starts = even_starts(h if axis == "height" else w, n_shards)
    return decode_bands(cfg, params, latent, starts, prec, axis), axis
