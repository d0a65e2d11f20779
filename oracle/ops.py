"""Per-operator definitions of the decode, written out in float64.

Every tensor is 5-D ``[N, C, T, H, W]`` (2-D images use T = 1).  Each
function evaluates the plain definition of its operator; where the method's
pages fix a formula it is cited beside the function.  Library routines used
as steps: ``torch.matmul`` / ``addmm_`` (a dense matrix product), ``exp``,
``sqrt``, elementwise arithmetic and ``cat``/indexing.  Nothing is fused or
reordered beyond what the definitions state.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence, Tuple

import torch

F64 = torch.float64
# Upper bound on the float64 elements of one staged operand slice; bounds memory only.
_CHUNK_ELEMS = 1 << 24


def conv_padded(xp: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor],
                finish: Callable[[torch.Tensor], torch.Tensor],
                residual: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Valid cross-correlation of an already padded input.

    ``y[n,o,t,h,w] = bias[o] + sum_{i,dt,dy,dx} W[o,i,dt,dy,dx] * xp[n,i,t+dt,h+dy,w+dx]``
    (+ ``residual[n,o,t,h,w]`` when given), accumulated in float64 and handed
    to ``finish`` (the storage rounding) once per output chunk.

    xp: [N, Ci, Tp, Hp, Wp]; w: [Co, Ci, kt, kh, kw]; returns [N, Co, To, Ho, Wo]
    with To = Tp-kt+1, Ho = Hp-kh+1, Wo = Wp-kw+1.
    """
    n_img, ci, tp, hp, wp = xp.shape
    co, ci2, kt, kh, kw = w.shape
    assert ci == ci2, (ci, ci2)
    to, ho, wo = tp - kt + 1, hp - kh + 1, wp - kw + 1
    y = None
    taps = [(dt, dy, dx, w[:, :, dt, dy, dx].to(F64).contiguous())
            for dt in range(kt) for dy in range(kh) for dx in range(kw)]
    bias = torch.zeros(co, dtype=F64) if b is None else b.to(F64)
    rows = max(1, min(ho, _CHUNK_ELEMS // max(1, ci * wo)))
    for n in range(n_img):
        for t in range(to):
            for h0 in range(0, ho, rows):
                h1 = min(ho, h0 + rows)
                acc = bias[:, None].expand(co, (h1 - h0) * wo).clone()
                for dt, dy, dx, wt in taps:
                    xs = xp[n, :, t + dt, h0 + dy:h1 + dy, dx:dx + wo].to(F64).reshape(ci, -1)
                    acc.addmm_(wt, xs)
                acc = acc.view(co, h1 - h0, wo)
                if residual is not None:
                    acc = acc + residual[n, :, t, h0:h1, :].to(F64)
                out = finish(acc)
                if y is None:
                    y = torch.empty((n_img, co, to, ho, wo), dtype=out.dtype)
                y[n, :, t, h0:h1, :] = out
    return y


def _pad_tw(x: torch.Tensor, t_front: int, pw: int) -> torch.Tensor:
    """Zero frames in front (causal time padding) and zero columns at both W edges."""
    if t_front == 0 and pw == 0:
        return x
    return torch.nn.functional.pad(x, (pw, pw, 0, 0, t_front, 0))


def conv_full(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], causal: bool,
              finish, residual=None) -> torch.Tensor:
    """Full-image conv with 'same' zero padding on H and W; causal front padding in time.

    Centered odd kernels, stride 1, dilation 1: the pad is (k-1)/2 on each
    spatial side.  In time the causal conv pads kt-1 zero frames in front and
    none behind (the Wan-style causal 3-D convolution).
    """
    _, _, kt, kh, kw = w.shape
    ph, pw = (kh - 1) // 2, (kw - 1) // 2
    pt = (kt - 1) if causal else 0
    assert causal or kt == 1
    xp = _pad_tw(x, pt, pw)
    if ph:
        xp = torch.nn.functional.pad(xp, (0, 0, ph, ph))
    return conv_padded(xp, w, b, finish, residual)


def conv_band(bands: Sequence[torch.Tensor], i: int, w: torch.Tensor, b: Optional[torch.Tensor],
              causal: bool, finish, residual=None, axis: int = 3) -> torch.Tensor:
    """Conv of band i: its own rows plus kernel-radius halo rows from the neighbours.

    The feature page's conv section: each conv fetches the boundary rows it
    needs from the adjacent shards; padding is used only at the outer edges
    of the whole image; a shard keeps only the output rows it owns.  The
    validation page's operator table says the same (kernel-radius rows, zero
    padding only at the global image edges).

    ``axis`` is the dimension the bands cut: 3 (height, row bands) or 4
    (width, column bands -- the width-sharded mode of the Wan page's strategy
    table).  Along the cut axis the halo comes from the neighbour bands;
    along the other spatial axis and in time the padding is the plain zero /
    causal padding of ``conv_full``.
    """
    assert axis in (3, 4)
    _, _, kt, kh, kw = w.shape
    ph, pw = (kh - 1) // 2, (kw - 1) // 2
    pt = (kt - 1) if causal else 0
    halo = ph if axis == 3 else pw
    x = bands[i]

    def zeros():
        shape = list(x.shape)
        shape[axis] = halo
        return torch.zeros(shape, dtype=x.dtype)

    parts = []
    if halo:
        if i > 0:
            before = bands[i - 1]
            assert before.shape[axis] >= halo, "neighbour band thinner than the halo"
            parts.append(before.narrow(axis, before.shape[axis] - halo, halo))
        else:
            parts.append(zeros())
    parts.append(x)
    if halo:
        if i + 1 < len(bands):
            after = bands[i + 1]
            assert after.shape[axis] >= halo, "neighbour band thinner than the halo"
            parts.append(after.narrow(axis, 0, halo))
        else:
            parts.append(zeros())
    xc = torch.cat(parts, dim=axis)
    if axis == 3:
        xp = _pad_tw(xc, pt, pw)
    else:   # zero rows at both H edges, causal zero frames in front
        xp = torch.nn.functional.pad(xc, (0, 0, ph, ph, pt, 0)) if (ph or pt) else xc
    return conv_padded(xp, w, b, finish, residual)


def groupnorm_moments(x: torch.Tensor, groups: int) -> Tuple[int, torch.Tensor, torch.Tensor]:
    """Element count, mean and population variance per (sample, group), two-pass.

    mean = sum(x) / n; var = sum((x - mean)^2) / n over the group's channels and
    every position of the tensor.  Returns (n, mean[N, G], var[N, G]).
    """
    n_img, c = x.shape[:2]
    assert c % groups == 0
    count = (c // groups) * x[0, 0].numel()
    mean = torch.empty((n_img, groups), dtype=F64)
    var = torch.empty((n_img, groups), dtype=F64)
    for n in range(n_img):
        xg = x[n].to(F64).reshape(groups, -1)
        m = xg.sum(dim=1) / count
        mean[n] = m
        var[n] = ((xg - m[:, None]) ** 2).sum(dim=1) / count
    return count, mean, var


def merge_moments(counts: Sequence[int], means: Sequence[torch.Tensor],
                  variances: Sequence[torch.Tensor]) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge per-shard central moments with actual element-count weights.

    Feature page, GroupNorm section (and the formula under the validation
    page's operator table): with w_i the shard's share of the elements,
    mean = sum_i w_i * mean_i and var = sum_i w_i * (var_i + (mean_i - mean)^2).
    A shard with zero elements gets weight zero.
    """
    total = float(sum(counts))
    assert total > 0
    mean = torch.zeros_like(means[0], dtype=F64)
    for n_i, m_i in zip(counts, means):
        mean = mean + (n_i / total) * m_i.to(F64)
    var = torch.zeros_like(means[0], dtype=F64)
    for n_i, m_i, v_i in zip(counts, means, variances):
        var = var + (n_i / total) * (v_i.to(F64) + (m_i.to(F64) - mean) ** 2)
    return mean, var


def silu(x: torch.Tensor) -> torch.Tensor:
    """SiLU(x) = x / (1 + e^{-x})."""
    return x / (1.0 + torch.exp(-x))


def groupnorm_apply(x: torch.Tensor, mean: torch.Tensor, var: torch.Tensor,
                    gamma: torch.Tensor, beta: torch.Tensor, eps: float, act: bool) -> torch.Tensor:
    """y = (x - mean_g) / sqrt(var_g + eps) * gamma_c + beta_c, then SiLU if ``act``.

    mean/var: [N, G] statistics of the whole image (float64).  Returns float64.
    """
    n_img, c = x.shape[:2]
    groups = mean.shape[1]
    cg = c // groups
    m = mean.repeat_interleave(cg, dim=1).view(n_img, c, 1, 1, 1)
    r = (1.0 / torch.sqrt(var + eps)).repeat_interleave(cg, dim=1).view(n_img, c, 1, 1, 1)
    y = (x.to(F64) - m) * r * gamma.to(F64).view(1, c, 1, 1, 1) + beta.to(F64).view(1, c, 1, 1, 1)
    return silu(y) if act else y


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, act: bool) -> torch.Tensor:
    """Channel RMSNorm per position: y_c = gamma_c * x_c / sqrt(mean_c x^2 + eps) (+ SiLU)."""
    xd = x.to(F64)
    ms = (xd * xd).mean(dim=1, keepdim=True)
    y = xd / torch.sqrt(ms + eps) * gamma.to(F64).view(1, -1, 1, 1, 1)
    return silu(y) if act else y


def attention_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                   q_chunk: int = 1024) -> torch.Tensor:
    """Single-head softmax attention O = softmax(q k^T * scale) v, float64.

    q: [Nq, C]; k, v: [Nk, C].  The softmax subtracts the row maximum before
    exponentiating.  Query rows are processed in independent chunks.
    """
    kd = k.to(F64)
    vd = v.to(F64)
    out = torch.empty((q.shape[0], v.shape[1]), dtype=F64)
    for r0 in range(0, q.shape[0], q_chunk):
        s = (q[r0:r0 + q_chunk].to(F64) @ kd.T) * scale
        s = s - s.max(dim=1, keepdim=True).values
        p = torch.exp(s)
        p = p / p.sum(dim=1, keepdim=True)
        out[r0:r0 + q_chunk] = p @ vd
    return out


def downsample_conv(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], finish) -> torch.Tensor:
    """Stride-2 3x3 convolution of the encoder's down stages (2-D, T = 1).

    The input is zero-padded by one row at the bottom and one column at the right
    (none at the top or left), and
    ``y[n,o,0,h,w] = bias[o] + sum_{i,dy,dx} W[o,i,0,dy,dx] * xp[n,i,0,2h+dy,2w+dx]``
    for h < H/2, w < W/2 (H and W even), accumulated in float64, then ``finish``.
    """
    n_img, ci, t, hh, ww = x.shape
    co, ci2, kt, kh, kw = w.shape
    assert ci == ci2 and t == 1 and kt == 1 and kh == 3 and kw == 3 and hh % 2 == 0 and ww % 2 == 0
    ho, wo = hh // 2, ww // 2
    xp = torch.nn.functional.pad(x.to(F64), (0, 1, 0, 1))
    y = torch.zeros((n_img, co, 1, ho, wo), dtype=F64)
    if b is not None:
        y += b.to(F64).view(1, co, 1, 1, 1)
    for dy in range(3):
        for dx in range(3):
            xs = xp[:, :, :, dy:dy + 2 * ho:2, dx:dx + 2 * wo:2]            # [N, Ci, 1, Ho, Wo]
            wt = w[:, :, 0, dy, dx].to(F64)                                # [Co, Ci]
            y += torch.matmul(wt, xs.reshape(n_img, ci, -1)).view(n_img, co, 1, ho, wo)
    return finish(y)


def upsample_nearest2x(x: torch.Tensor) -> torch.Tensor:
    """u[..., y, x] = v[..., floor(y/2), floor(x/2)] on H and W."""
    return x.repeat_interleave(2, dim=3).repeat_interleave(2, dim=4)


def temporal_upsample_interleave(x: torch.Tensor, z: torch.Tensor) -> torch.Tensor:
    """Causal temporal upsample, frame layout.

    z is the causal (3,1,1) time conv C -> 2C of x.  Frame 0 passes through;
    for t >= 1 the first C channels of z[t] become frame 2t-1 and the last C
    become frame 2t, so T frames become 2T-1.
    """
    n_img, c, t = x.shape[:3]
    assert z.shape[1] == 2 * c and z.shape[2] == t
    out = torch.empty((n_img, c, 2 * t - 1) + tuple(x.shape[3:]), dtype=x.dtype)
    out[:, :, 0] = x[:, :, 0]
    for s in range(1, t):
        out[:, :, 2 * s - 1] = z[:, :c, s]
        out[:, :, 2 * s] = z[:, c:, s]
    return out
