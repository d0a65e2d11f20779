"""Python face of the C ABI: same names, torch tensors for device memory and streams.

Every function here only marshals arguments; all computation runs in libvaep.so.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib as L

TORCH_DTYPE = {L.DTYPE_F32: torch.float32, L.DTYPE_BF16: torch.bfloat16}


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _starts(row_starts: Sequence[int]):
    arr = (C.c_int32 * len(row_starts))(*[int(v) for v in row_starts])
    return arr


def _dev(t: torch.Tensor, dtype, name):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t


def version() -> str:
    return L.load().vaep_version().decode()


def config_preset(i: int) -> L.VaepConfig:
    c = L.VaepConfig()
    L.check(L.load().vaep_config_preset(i, C.byref(c)))
    return c


def make_config(family: str, dtype: str, z_channels: int, stage_channels: Sequence[int],
                resnets_per_stage: int, norm_groups: int, temporal_up_stages: int = 0,
                eps: float = 1e-6) -> L.VaepConfig:
    c = L.VaepConfig()
    c.family = {"kl2d": L.FAMILY_KL2D, "wan3d": L.FAMILY_WAN3D}[family]
    c.dtype = {"f32": L.DTYPE_F32, "bf16": L.DTYPE_BF16}[dtype]
    c.z_channels = z_channels
    c.n_stages = len(stage_channels)
    for i, ch in enumerate(stage_channels):
        c.stage_channels[i] = ch
    c.resnets_per_stage = resnets_per_stage
    c.norm_groups = norm_groups
    c.temporal_up_stages = temporal_up_stages
    c.eps = eps
    return c


def param_info(cfg: L.VaepConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    lib = L.load()
    n = L.check(lib.vaep_param_count(C.byref(cfg)))
    out = []
    for j in range(n):
        name = C.create_string_buffer(128)
        shape = (C.c_int64 * 5)()
        nd = C.c_int()
        L.check(lib.vaep_param_info(C.byref(cfg), j, name, 128, shape, C.byref(nd)))
        out.append((name.value.decode(), tuple(shape[i] for i in range(nd.value))))
    return out


class Decoder:
    """A vaep_model: weights repacked into library-owned device memory."""

    def __init__(self, cfg: L.VaepConfig, params: Sequence[torch.Tensor], stream=None):
        self.cfg = cfg
        self.dtype = TORCH_DTYPE[cfg.dtype]
        lib = L.load()
        for t in params:
            _dev(t, self.dtype, "parameter")
        arr = (C.c_void_p * len(params))(*[t.data_ptr() for t in params])
        h = C.c_void_p()
        L.check(lib.vaep_model_create(C.byref(cfg), arr, len(params), _stream(stream), C.byref(h)))
        self._h = h

    def set_norm_fold(self, on: bool):
        """Fold the resnet GroupNorm apply into the conv operand load where the kernel supports
        it (vaep_model_set_norm_fold); the decoded output is the same."""
        L.check(L.load().vaep_model_set_norm_fold(self._h, 1 if on else 0))

    def set_halo_poison(self, on: bool):
        """Debug mode: every halo slot of a band buffer is filled with NaN before the layer
        that writes the buffer runs (vaep_model_set_halo_poison)."""
        L.check(L.load().vaep_model_set_halo_poison(self._h, 1 if on else 0))

    def close(self):
        if getattr(self, "_h", None):
            L.check(L.load().vaep_model_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, batch, frames, latent_h, latent_w, n_bands) -> int:
        n = C.c_size_t()
        L.check(L.load().vaep_workspace_bytes(self._h, batch, frames, latent_h, latent_w, n_bands,
                                              C.byref(n)))
        return n.value

    def workspace(self, batch, frames, latent_h, latent_w, n_bands, device="cuda") -> torch.Tensor:
        return torch.empty(self.workspace_bytes(batch, frames, latent_h, latent_w, n_bands),
                           dtype=torch.uint8, device=device)

    @staticmethod
    def _dims(latent):
        if latent.dim() == 4:
            b, _, h, w = latent.shape
            return b, 1, h, w
        b, _, t, h, w = latent.shape
        return b, t, h, w

    def decode_full(self, latent, out, ws, stream=None) -> int:
        b, t, h, w = self._dims(latent)
        _dev(latent, self.dtype, "latent")
        _dev(out, torch.float32, "out")
        return L.check(L.load().vaep_decode_full(self._h, _p(latent), b, t, h, w, _p(out), _p(ws),
                                                 ws.numel(), _stream(stream)))

    def decode_bands(self, latent, row_starts, out, ws, stream=None):
        b, t, h, w = self._dims(latent)
        _dev(latent, self.dtype, "latent")
        _dev(out, torch.float32, "out")
        info = L.VaepDecodeInfo()
        rc = L.check(L.load().vaep_decode_bands(self._h, _p(latent), b, t, h, w, _starts(row_starts),
                                                len(row_starts) - 1, _p(out), _p(ws), ws.numel(),
                                                _stream(stream), C.byref(info)))
        return rc, info

    def decode_bands_noalloc(self, latent, row_starts, out, stream=None):
        """decode_bands with the library's static scratch as workspace (allocates nothing)."""
        b, t, h, w = self._dims(latent)
        _dev(latent, self.dtype, "latent")
        _dev(out, torch.float32, "out")
        info = L.VaepDecodeInfo()
        rc = L.check(L.load().vaep_decode_bands_noalloc(self._h, _p(latent), b, t, h, w, _starts(row_starts),
                                                        len(row_starts) - 1, _p(out), _stream(stream),
                                                        C.byref(info)))
        return rc, info

    def decode_sharded(self, latent, axis: str, n_shards: int, out, ws, starts=None, stream=None):
        """axis: 'height', 'width', 'tile' or 'auto'; starts: shard boundaries along the axis or None."""
        b, t, h, w = self._dims(latent)
        _dev(latent, self.dtype, "latent")
        _dev(out, torch.float32, "out")
        code = AXES[axis]
        info = L.VaepDecodeInfo()
        st = None
        if starts is not None:
            assert len(starts) == n_shards + 1
            st = _starts(starts)
        rc = L.check(L.load().vaep_decode_sharded(self._h, _p(latent), b, t, h, w, code, st, n_shards,
                                                  _p(out), _p(ws), ws.numel(), _stream(stream),
                                                  C.byref(info)))
        return rc, info


    def sharded_workspace(self, batch, frames, latent_h, latent_w, n_shards, device="cuda") -> torch.Tensor:
        """Workspace for every outcome of decode_sharded, the tile fallback included."""
        n = C.c_size_t()
        L.check(L.load().vaep_sharded_workspace_bytes(self._h, batch, frames, latent_h, latent_w, n_shards,
                                                      C.byref(n)))
        return torch.empty(n.value, dtype=torch.uint8, device=device)

    def tiled_workspace(self, batch, frames, latent_h, latent_w, tile, stride, device="cuda") -> torch.Tensor:
        n = C.c_size_t()
        L.check(L.load().vaep_tiled_workspace_bytes(self._h, batch, frames, latent_h, latent_w, tile, stride,
                                                    C.byref(n)))
        return torch.empty(n.value, dtype=torch.uint8, device=device)

    def decode_tiled(self, latent, tile: int, stride: int, out, ws, stream=None) -> int:
        """Tiled decode with overlap blending (the comparison baseline of the sharded decode)."""
        b, t, h, w = self._dims(latent)
        _dev(latent, self.dtype, "latent")
        _dev(out, torch.float32, "out")
        return L.check(L.load().vaep_decode_tiled(self._h, _p(latent), b, t, h, w, tile, stride, _p(out), _p(ws),
                                                  ws.numel(), _stream(stream)))


def encoder_param_info(cfg: L.VaepConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """Canonical (name, shape) list of the encoder of a 2-D config (vaep_encoder_param_info)."""
    lib = L.load()
    n = L.check(lib.vaep_encoder_param_count(C.byref(cfg)))
    out = []
    for j in range(n):
        name = C.create_string_buffer(128)
        shape = (C.c_int64 * 5)()
        nd = C.c_int()
        L.check(lib.vaep_encoder_param_info(C.byref(cfg), j, name, 128, shape, C.byref(nd)))
        out.append((name.value.decode(), tuple(shape[i] for i in range(nd.value))))
    return out


class Encoder:
    """A vaep_encoder (the tiled encode of a 2-D config): weights repacked into library-owned
    device memory."""

    def __init__(self, cfg: L.VaepConfig, params: Sequence[torch.Tensor], stream=None):
        self.cfg = cfg
        self.dtype = TORCH_DTYPE[cfg.dtype]
        lib = L.load()
        for t in params:
            _dev(t, self.dtype, "parameter")
        arr = (C.c_void_p * len(params))(*[t.data_ptr() for t in params])
        h = C.c_void_p()
        L.check(lib.vaep_encoder_create(C.byref(cfg), arr, len(params), _stream(stream), C.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            L.check(L.load().vaep_encoder_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, batch, height, width, tile, stride, device="cuda") -> torch.Tensor:
        n = C.c_size_t()
        L.check(L.load().vaep_encode_tiled_workspace_bytes(self._h, batch, height, width, tile, stride,
                                                           C.byref(n)))
        return torch.empty(n.value, dtype=torch.uint8, device=device)

    def encode_tiled(self, image, tile: int, stride: int, out, ws, stream=None):
        """image (B, 3, H, W) in the config's dtype -> out (B, 2 z, H / up, W / up) fp32; returns
        (status, info)."""
        if image.dim() != 4 or image.shape[1] != 3:
            raise ValueError("image must be (batch, 3, height, width)")
        b, _, h, w = image.shape
        _dev(image, self.dtype, "image")
        _dev(out, torch.float32, "out")
        info = L.VaepDecodeInfo()
        rc = L.check(L.load().vaep_encode_tiled(self._h, _p(image), b, h, w, tile, stride, _p(out), _p(ws),
                                                ws.numel(), _stream(stream), C.byref(info)))
        return rc, info


AXES = {"auto": L.AXIS_AUTO, "height": L.AXIS_HEIGHT, "width": L.AXIS_WIDTH, "tile": L.AXIS_TILE}
AXIS_NAMES = {L.AXIS_HEIGHT: "height", L.AXIS_WIDTH: "width", L.AXIS_DENSE: "dense", L.AXIS_TILE: "tile"}


def select_axis(latent_h: int, latent_w: int, n_shards: int) -> str:
    """The library's per-request axis policy: 'height', 'width', 'tile' or 'dense'."""
    a = C.c_int32()
    L.check(L.load().vaep_select_axis(latent_h, latent_w, n_shards, C.byref(a)), allow_warning=False)
    return AXIS_NAMES[a.value]


def profile_begin(dec: "Decoder", max_launches: int = 4096):
    L.check(L.load().vaep_profile_begin(dec._h, max_launches))


def profile_end(dec: "Decoder"):
    """Per-launch records (list of dicts) of the decodes since profile_begin."""
    cap = 1 << 16
    arr = (L.VaepProfileEntry * cap)()
    n = C.c_int()
    L.check(L.load().vaep_profile_end(dec._h, arr, cap, C.byref(n)))
    keys = [f[0] for f in L.VaepProfileEntry._fields_]
    return [{k: getattr(arr[i], k) for k in keys} for i in range(min(n.value, cap))]


def groupnorm_merge(local_mean: torch.Tensor, local_var: torch.Tensor, counts: torch.Tensor,
                    stream=None):
    """vaep_groupnorm_merge on [n_shards, n_stats] device tensors -> (mean, var)."""
    _dev(local_mean, torch.float32, "local_mean")
    _dev(local_var, torch.float32, "local_var")
    _dev(counts, torch.int64, "counts")
    n_shards, n_stats = local_mean.shape
    mean = torch.empty(n_stats, dtype=torch.float32, device=local_mean.device)
    var = torch.empty_like(mean)
    L.check(L.load().vaep_groupnorm_merge(n_shards, n_stats, _p(local_mean), _p(local_var), _p(counts),
                                          _p(mean), _p(var), _stream(stream)))
    return mean, var


def _dt(t: torch.Tensor) -> int:
    return {torch.float32: L.DTYPE_F32, torch.bfloat16: L.DTYPE_BF16}[t.dtype]


def _bchw(x):
    if x.dim() == 4:
        b, c, h, w = x.shape
        return b, 1, c, h, w
    b, c, t, h, w = x.shape
    return b, t, c, h, w


def _run_step(fn, args_before_ws, stream, device):
    """Call a vaep_step_* twice: size query, then the real call with a torch workspace."""
    need = C.c_size_t()
    L.check(fn(*args_before_ws, None, 0, C.byref(need), _stream(stream)))
    ws = torch.empty(max(1, need.value), dtype=torch.uint8, device=device)
    L.check(fn(*args_before_ws, _p(ws), ws.numel(), None, _stream(stream)))
    return ws


def step_conv(x, weight, bias, row_starts, *, causal=False, upsample=False, residual=None, stream=None):
    """Conv step; the compute dtype is the weight's, x may be fp32 or that dtype; y is fp32."""
    b, t, cin, h, w = _bchw(x)
    cout = weight.shape[0]
    k = weight.shape[2:]
    kt, kh, kw = (1,) + tuple(k) if len(k) == 2 else tuple(k)
    ho, wo = (2 * h, 2 * w) if upsample else (h, w)
    shape = (b, cout, ho, wo) if x.dim() == 4 else (b, cout, t, ho, wo)
    y = torch.empty(shape, dtype=torch.float32, device=x.device)
    lib = L.load()
    _run_step(lib.vaep_step_conv,
              (_dt(weight), _dt(x), _p(x), b, t, cin, h, w, _p(weight), _p(bias), cout, kt, kh, kw, int(causal),
               int(upsample), _p(residual), _starts(row_starts), len(row_starts) - 1, _p(y)),
              stream, x.device)
    return y


def step_groupnorm(x, groups, eps, gamma, beta, row_starts, *, act=True, out_dtype=torch.bfloat16,
                   stream=None):
    """GroupNorm step on an fp32 x; y in out_dtype (the compute dtype)."""
    b, t, c, h, w = _bchw(x)
    nb = len(row_starts) - 1
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    moments = torch.empty((3, nb, b * t * groups), dtype=torch.float32, device=x.device)
    merged = torch.empty((2, b * t * groups), dtype=torch.float32, device=x.device)
    _run_step(L.load().vaep_step_groupnorm,
              (_dt(y), _p(x), b, t, c, h, w, groups, C.c_float(eps), _p(gamma), _p(beta), int(act),
               _starts(row_starts), nb, _p(y), _p(moments), _p(merged)),
              stream, x.device)
    return y, moments, merged


def step_rmsnorm(x, eps, gamma, row_starts, *, act=True, out_dtype=torch.bfloat16, stream=None):
    """RMSNorm step on an fp32 x; y in out_dtype (the compute dtype)."""
    b, t, c, h, w = _bchw(x)
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _run_step(L.load().vaep_step_rmsnorm,
              (_dt(y), _p(x), b, t, c, h, w, C.c_float(eps), _p(gamma), int(act), _starts(row_starts),
               len(row_starts) - 1, _p(y)),
              stream, x.device)
    return y


def step_attention(x, groups, eps, norm_gamma, norm_beta, wq, bq, wk, bk, wv, bv, wo, bo, row_starts,
                   *, stream=None):
    b, t, c, h, w = _bchw(x)
    y = torch.empty_like(x)
    _run_step(L.load().vaep_step_attention,
              (_dt(wq), _p(x), b, t, c, h, w, groups, C.c_float(eps), _p(norm_gamma), _p(norm_beta),
               _p(wq), _p(bq), _p(wk), _p(bk), _p(wv), _p(bv), _p(wo), _p(bo), _starts(row_starts),
               len(row_starts) - 1, _p(y)),
              stream, x.device)
    return y


def step_temporal_upsample(x, weight, bias, row_starts, *, stream=None):
    b, t, c, h, w = _bchw(x)
    y = torch.empty((b, c, 2 * t - 1, h, w), dtype=torch.float32, device=x.device)
    _run_step(L.load().vaep_step_temporal_upsample,
              (_dt(weight), _p(x), b, t, c, h, w, _p(weight), _p(bias), _starts(row_starts),
               len(row_starts) - 1, _p(y)),
              stream, x.device)
    return y
