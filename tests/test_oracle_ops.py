"""Pins of the oracle's per-operator definitions (CPU only).

Each test checks an oracle function against something other than itself:
hand-worked closed forms, golden fixtures from the pages' formula, brute
force on tiny inputs, or a special case that reduces to a PyTorch library
routine (an independent implementation of the same textbook operator).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ops
from oracle.decoder import Precision

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64
fin32 = Precision("f32").finish


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=F64) * scale


# ----------------------------------------------------------------------------- conv

def test_conv_ones_closed_form():
    want = np.loadtxt(os.path.join(GOLDEN, "conv3x3_ones_4x5.txt"))
    x = torch.ones(1, 1, 1, 4, 5)
    w = torch.ones(1, 1, 1, 3, 3)
    y = ops.conv_full(x, w, None, False, fin32)
    assert torch.equal(y[0, 0, 0], torch.from_numpy(want).float())


def test_conv_impulse_gives_flipped_kernel():
    # cross-correlation: an impulse at (r, c) puts W[dy, dx] at output (r+1-dy, c+1-dx)
    w = torch.arange(1, 10, dtype=torch.float32).view(1, 1, 1, 3, 3)
    x = torch.zeros(1, 1, 1, 5, 5)
    x[0, 0, 0, 2, 2] = 1.0
    y = ops.conv_full(x, w, None, False, fin32)[0, 0, 0]
    assert torch.equal(y[1:4, 1:4], torch.flip(w[0, 0, 0], dims=(0, 1)))
    assert y.sum().item() == w.sum().item()


def test_conv_brute_force_tiny():
    x = _rand((2, 3, 1, 4, 5), 1).float()
    w = _rand((4, 3, 1, 3, 3), 2).float()
    b = _rand((4,), 3).float()
    y = ops.conv_full(x, w, b, False, lambda a: a.to(F64))
    for n in range(2):
        for o in range(4):
            for h in range(4):
                for c in range(5):
                    s = float(b[o])
                    for i in range(3):
                        for dy in range(3):
                            for dx in range(3):
                                hh, cc = h + dy - 1, c + dx - 1
                                if 0 <= hh < 4 and 0 <= cc < 5:
                                    s += float(w[o, i, 0, dy, dx]) * float(x[n, i, 0, hh, cc])
                    assert abs(float(y[n, o, 0, h, c]) - s) < 1e-12


@pytest.mark.parametrize("k", [1, 3])
def test_conv2d_matches_library(k):
    x = _rand((2, 5, 1, 9, 7), 4).float()
    w = _rand((6, 5, 1, k, k), 5).float()
    b = _rand((6,), 6).float()
    r = _rand((2, 6, 1, 9, 7), 7).float()
    y = ops.conv_full(x, w, b, False, lambda a: a.to(F64), residual=r)
    ref = F.conv2d(x[:, :, 0].double(), w[:, :, 0].double(), b.double(), padding=(k - 1) // 2) + r[:, :, 0]
    assert torch.allclose(y[:, :, 0], ref, atol=1e-12, rtol=0)


def test_causal_conv3d_matches_library_with_front_padding():
    x = _rand((1, 3, 4, 5, 6), 8).float()
    w = _rand((2, 3, 3, 3, 3), 9).float()
    b = _rand((2,), 10).float()
    y = ops.conv_full(x, w, b, True, lambda a: a.to(F64))
    xp = F.pad(x.double(), (1, 1, 1, 1, 2, 0))
    ref = F.conv3d(xp, w.double(), b.double())
    assert y.shape == x.shape[:1] + (2,) + x.shape[2:]
    assert torch.allclose(y, ref, atol=1e-12, rtol=0)


def test_causal_conv_ones_frame_counts():
    # all-ones input and kernel: frames 0, 1, >=2 see 1, 2, 3 input frames
    x = torch.ones(1, 1, 5, 3, 3)
    w = torch.ones(1, 1, 3, 1, 1)
    y = ops.conv_full(x, w, None, True, fin32)
    assert y[0, 0, :, 1, 1].tolist() == [1.0, 2.0, 3.0, 3.0, 3.0]


def test_causal_conv_impulse_reaches_only_later_frames():
    x = torch.zeros(1, 1, 6, 3, 3)
    x[0, 0, 2, 1, 1] = 1.0
    w = torch.ones(1, 1, 3, 3, 3)
    y = ops.conv_full(x, w, None, True, fin32)
    touched = (y[0, 0].abs().sum(dim=(1, 2)) > 0).tolist()
    assert touched == [False, False, True, True, True, False]


def test_conv_band_equals_full_bitwise():
    x = _rand((2, 4, 3, 10, 7), 11).float()
    w = _rand((5, 4, 3, 3, 3), 12).float()
    b = _rand((5,), 13).float()
    full = ops.conv_full(x, w, b, True, fin32)
    starts = [0, 1, 4, 5, 10]
    bands = [x[:, :, :, s:e].contiguous() for s, e in zip(starts, starts[1:])]
    parts = [ops.conv_band(bands, i, w, b, True, fin32) for i in range(len(bands))]
    assert torch.equal(torch.cat(parts, dim=3), full)


def test_conv_width_band_equals_full():
    # column bands (the width-sharded mode): halo columns from the neighbours, zero rows
    # at the H edges; uneven bands including 1-column bands
    x = _rand((2, 4, 3, 7, 10), 21).float()
    w = _rand((5, 4, 3, 3, 3), 22).float()
    b = _rand((5,), 23).float()
    r = _rand((2, 5, 3, 7, 10), 24).float()
    for causal, wk in ((True, w), (False, w[:, :, 2:])):
        full = ops.conv_full(x, wk, b, causal, fin32, r)
        starts = [0, 1, 4, 5, 10]
        bands = [x[:, :, :, :, s:e].contiguous() for s, e in zip(starts, starts[1:])]
        parts = [ops.conv_band(bands, i, wk, b, causal, fin32, r[..., s:e], axis=4)
                 for i, (s, e) in enumerate(zip(starts, starts[1:]))]
        y = torch.cat(parts, dim=4)
        assert y.shape == full.shape
        assert (y - full).abs().max().item() <= 1e-6 * full.abs().max().item()


def test_conv_linearity():
    x1 = _rand((1, 3, 1, 6, 6), 14).float()
    x2 = _rand((1, 3, 1, 6, 6), 15).float()
    w = _rand((2, 3, 1, 3, 3), 16).float()
    f = lambda a: a.to(F64)
    y = ops.conv_full(x1 + x2, w, None, False, f)
    y12 = ops.conv_full(x1, w, None, False, f) + ops.conv_full(x2, w, None, False, f)
    assert torch.allclose(y, y12, atol=1e-5)


# ----------------------------------------------------------------------------- GroupNorm

def _golden_merge():
    cases = []
    with open(os.path.join(GOLDEN, "groupnorm_merge_example.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("|")
            shards = [[float(v) for v in s.split()] for s in lhs.split(";")]
            m, v = (float(t) for t in rhs.split())
            cases.append((shards, m, v))
    return cases


def test_merge_golden_worked_examples():
    cases = _golden_merge()
    assert len(cases) == 3
    for shards, m_want, v_want in cases:
        counts, means, vars_ = [], [], []
        for s in shards:
            t = torch.tensor(s, dtype=torch.float32).view(1, 1, 1, 1, -1)
            n, m, v = ops.groupnorm_moments(t, 1)
            counts.append(n)
            means.append(m)
            vars_.append(v)
        mean, var = ops.merge_moments(counts, means, vars_)
        assert abs(mean.item() - m_want) < 1e-12 and abs(var.item() - v_want) < 1e-12


def test_moments_closed_form_arange():
    n = 1000
    x = torch.arange(n, dtype=torch.float32).view(1, 1, 1, 1, n)
    cnt, m, v = ops.groupnorm_moments(x, 1)
    assert cnt == n
    assert m.item() == (n - 1) / 2
    assert abs(v.item() - (n * n - 1) / 12) < 1e-9


def test_merge_identity_random_uneven_splits():
    x = _rand((2, 8, 1, 37, 9), 20, 3.0).float() + 5.0
    _, m_full, v_full = ops.groupnorm_moments(x, 4)
    for starts in ([0, 1, 37], [0, 5, 6, 20, 37], [0, 36, 37]):
        parts = [ops.groupnorm_moments(x[:, :, :, s:e], 4) for s, e in zip(starts, starts[1:])]
        m, v = ops.merge_moments([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
        assert torch.allclose(m, m_full, rtol=1e-12, atol=0)
        assert torch.allclose(v, v_full, rtol=1e-12, atol=0)


def test_merge_large_offset_is_stable():
    # 1e4 + N(0,1): E[x^2]-E[x]^2 in fp32 loses the variance; the central-moment merge does not
    x = (torch.randn(1, 1, 1, 64, 64, generator=torch.Generator().manual_seed(3)) + 1e4).float()
    exact = x.double().var(unbiased=False).item()
    parts = [ops.groupnorm_moments(x[:, :, :, s:e], 1) for s, e in ((0, 9), (9, 40), (40, 64))]
    _, v = ops.merge_moments([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
    assert abs(v.item() - exact) / exact < 1e-9
    xs = x.float().flatten()
    naive = (xs * xs).mean() - xs.mean() ** 2
    assert abs(naive.item() - exact) / exact > 1e-2   # the failure the merge avoids


def test_merge_zero_count_shard_has_no_weight():
    m, v = ops.merge_moments([0, 4], [torch.tensor([100.0]), torch.tensor([2.0])],
                             [torch.tensor([50.0]), torch.tensor([3.0])])
    assert m.item() == 2.0 and v.item() == 3.0


def test_groupnorm_matches_library_with_affine():
    x = _rand((3, 12, 1, 5, 7), 21).float()
    g = _rand((12,), 22).float()
    b = _rand((12,), 23).float()
    _, m, v = ops.groupnorm_moments(x, 4)
    y = ops.groupnorm_apply(x, m, v, g, b, 1e-6, act=False)
    ref = F.group_norm(x[:, :, 0].double(), 4, g.double(), b.double(), eps=1e-6)
    assert torch.allclose(y[:, :, 0], ref, atol=1e-10, rtol=0)
    ya = ops.groupnorm_apply(x, m, v, g, b, 1e-6, act=True)
    assert torch.allclose(ya[:, :, 0], F.silu(ref), atol=1e-10, rtol=0)


def test_groupnorm_constant_input_gives_beta():
    x = torch.full((1, 4, 1, 3, 3), 7.25)
    _, m, v = ops.groupnorm_moments(x, 2)
    beta = torch.tensor([0.5, -1.0, 2.0, 3.0])
    y = ops.groupnorm_apply(x, m, v, torch.ones(4), beta, 1e-6, act=False)
    assert torch.allclose(y, beta.double().view(1, 4, 1, 1, 1).expand_as(y), atol=0)


# ----------------------------------------------------------------------------- pointwise

def test_silu_identities_and_library():
    x = torch.linspace(-30, 30, 601, dtype=F64)
    s = ops.silu(x)
    assert ops.silu(torch.zeros(1, dtype=F64)).item() == 0.0
    assert torch.allclose(s - ops.silu(-x), x, atol=1e-12)
    assert torch.allclose(s, F.silu(x), atol=1e-14)


def test_rmsnorm_constant_vector():
    a, eps = 0.3, 1e-6
    x = torch.full((1, 8, 1, 1, 1), a)
    g = torch.linspace(0.5, 2.0, 8)
    y = ops.rmsnorm(x, g, eps, act=False)
    want = a / math.sqrt(a * a + eps) * g.double()
    assert torch.allclose(y.view(-1), want, atol=1e-12)


def test_rmsnorm_matches_library():
    x = _rand((2, 6, 3, 4, 5), 30).float()
    g = _rand((6,), 31).float()
    y = ops.rmsnorm(x, g, 1e-6, act=True)
    xm = x.double().movedim(1, -1)
    ref = F.silu(F.rms_norm(xm, (6,), g.double(), eps=1e-6)).movedim(-1, 1)
    assert torch.allclose(y, ref, atol=1e-10)


def test_upsample_index_map():
    x = torch.arange(2 * 3 * 4, dtype=torch.float32).view(1, 2, 1, 3, 4)
    u = ops.upsample_nearest2x(x)
    for y in range(6):
        for c in range(8):
            assert torch.equal(u[0, :, 0, y, c], x[0, :, 0, y // 2, c // 2])
    ref = F.interpolate(x[:, :, 0], scale_factor=2, mode="nearest")
    assert torch.equal(u[:, :, 0], ref)


def test_temporal_interleave_frame_map():
    n, c, t = 1, 2, 4
    x = torch.arange(t, dtype=torch.float32).view(1, 1, t, 1, 1).expand(n, c, t, 1, 1).contiguous()
    z = torch.zeros(n, 2 * c, t, 1, 1)
    for s in range(t):
        z[:, :c, s] = 100 + s      # first half of z[s]
        z[:, c:, s] = 200 + s      # second half
    out = ops.temporal_upsample_interleave(x, z)
    assert out[0, 0, :, 0, 0].tolist() == [0, 101, 201, 102, 202, 103, 203]


# ----------------------------------------------------------------------------- attention

def test_attention_equal_logits_gives_mean_of_v():
    q = torch.zeros(3, 4, dtype=F64)
    k = _rand((7, 4), 40)
    v = _rand((7, 4), 41)
    o = ops.attention_rows(q, k, v, 0.5)
    assert torch.allclose(o, v.mean(dim=0, keepdim=True).expand(3, 4), atol=1e-14)


def test_attention_dominant_logit_selects_row():
    k = torch.eye(5, dtype=F64)
    q = torch.zeros(1, 5, dtype=F64)
    q[0, 3] = 200.0
    v = _rand((5, 5), 42)
    o = ops.attention_rows(q, k, v, 1.0)
    assert torch.allclose(o[0], v[3], atol=1e-12)


def test_attention_single_key_returns_v():
    o = ops.attention_rows(_rand((4, 3), 43), _rand((1, 3), 44), torch.tensor([[1.0, -2.0, 3.0]], dtype=F64), 0.1)
    assert torch.allclose(o, torch.tensor([[1.0, -2.0, 3.0]], dtype=F64).expand(4, 3))


def test_attention_matches_library_and_rows_are_independent():
    q = _rand((50, 16), 45)
    k = _rand((70, 16), 46)
    v = _rand((70, 16), 47)
    o = ops.attention_rows(q, k, v, 0.25, q_chunk=7)
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], scale=0.25)[0]
    assert torch.allclose(o, ref, atol=1e-12)
    sub = ops.attention_rows(q[11:29], k, v, 0.25)
    assert torch.allclose(sub, o[11:29], atol=1e-14)
