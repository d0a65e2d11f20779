"""Per-step parity of the HIP kernels against the oracle, through the C ABI.

Shapes span several workgroup tiles with ragged tails, uneven and one-row
bands, and channel counts that are not multiples of the output tile.  Inputs are
seeded; the oracle evaluates each step's definition in float64 on the same
values and rounds to the storage type once.
"""
import math

import pytest
import torch

import spatially_sharded_conv_amd as vaep
from oracle import ops
from oracle.decoder import Precision
from tests._util import assert_close, seeded, to_dev

pytestmark = pytest.mark.gpu

# A step whose output is a normalised operand: the GPU and the oracle both round it to
# the compute dtype once.  Conv outputs are fp32 accumulations of exact products.
STEP_TOL = {"bf16": (2e-2, 4e-3), "f32": (1e-4, 1e-5)}
ACC_TOL = (1e-4, 1e-5)


def _op(x, dtype):
    """The matrix-core operand the GPU forms from a stored tensor."""
    return Precision(dtype).finish(x.double(), "operand")


def _x5(x):
    return x if x.dim() == 5 else x.unsqueeze(2)


def _conv_ref(x, w, b, causal, res, dtype, upsample=False, x_exact=False):
    # bf16 operands load as they are; fp32 sources are split into hi + lo parts on the GPU,
    # which carries them to ~2^-17 relative: the reference uses them unrounded
    x5 = _x5(x if x_exact else _op(x, dtype))
    if upsample:
        x5 = ops.upsample_nearest2x(x5)
    w5 = w if w.dim() == 5 else w.unsqueeze(2)
    r5 = None if res is None else _x5(res)
    y = ops.conv_full(x5, w5, b, causal, Precision(dtype).acc, r5)
    return y if x.dim() == 5 else y[:, :, 0]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", [
    # (B, cin, cout, H, W, starts, with_residual)
    (2, 64, 96, 13, 37, (0, 1, 6, 13), True),
    (1, 32, 128, 16, 16, (0, 16), False),
    (1, 128, 256, 9, 70, (0, 4, 5, 9), True),
    # 96 input channels (not a multiple of 64): the tile kernel's 32-channel K steps,
    # three per tap, ragged bands and a one-row band
    (2, 96, 128, 11, 29, (0, 3, 4, 11), True),
])
def test_conv3x3_step(gpu_lib, dtype, case):
    B, cin, cout, H, W, starts, with_res = case
    x = seeded((B, cin, H, W), 11, dtype=dtype)
    w = seeded((cout, cin, 3, 3), 12, 1 / math.sqrt(cin * 9), dtype=dtype)
    b = seeded((cout,), 13, 0.1, dtype=dtype)
    r = seeded((B, cout, H, W), 14, dtype="f32") if with_res else None
    ref = _conv_ref(x, w, b, False, r, dtype)
    got = vaep.step_conv(to_dev(x, dtype), to_dev(w, dtype), to_dev(b, dtype), starts,
                         residual=None if r is None else r.cuda())
    assert got.dtype == torch.float32
    assert_close(got, ref, *ACC_TOL, what=f"conv3x3 {case}")


@pytest.mark.parametrize("cin", [64, 96])
def test_conv3x3_step_wide_tiles(gpu_lib, cin):
    # enough 256-pixel tiles for the 256-channel output tiles of the wide kernel (ragged
    # rows, a one-row band, residual); 96 input channels: each tap's second 64-channel
    # step half empty
    B, cout, H, W, starts = 1, 256, 130, 1030, (0, 40, 41, 130)
    x = seeded((B, cin, H, W), 15, dtype="bf16")
    w = seeded((cout, cin, 3, 3), 16, 1 / math.sqrt(cin * 9), dtype="bf16")
    b = seeded((cout,), 17, 0.1, dtype="bf16")
    r = seeded((B, cout, H, W), 18, dtype="f32")
    ref = _conv_ref(x, w, b, False, r, "bf16")
    got = vaep.step_conv(to_dev(x, "bf16"), to_dev(w, "bf16"), to_dev(b, "bf16"), starts, residual=r.cuda())
    assert_close(got, ref, *ACC_TOL, what=f"conv3x3 wide tiles, cin {cin}")


@pytest.mark.parametrize("case", [
    # (B, cin, cout, H, W, starts): 128 x (4 x 128) tiles; 256 x (4 x 64) tiles
    (1, 128, 128, 1030, 256, (0, 5, 6, 261, 517, 1030)),
    (1, 64, 256, 516, 256, (0, 1, 130, 131, 387, 516)),
])
def test_conv3x3_halo_tiles(gpu_lib, case):
    """The halo-tile kernel (pixel operand staged once per 32-channel block, 4-row tiles
    aligned to global rows and clipped at band edges): residual, uneven and one-row bands,
    bit-identical on every band table."""
    B, cin, cout, H, W, starts = case
    x = seeded((B, cin, H, W), 41, dtype="bf16")
    w = seeded((cout, cin, 3, 3), 42, 1 / math.sqrt(cin * 9), dtype="bf16")
    b = seeded((cout,), 43, 0.1, dtype="bf16")
    r = seeded((B, cout, H, W), 44, dtype="f32")
    ref = _conv_ref(x, w, b, False, r, "bf16")
    xd, wd, bd, rd = to_dev(x, "bf16"), to_dev(w, "bf16"), to_dev(b, "bf16"), r.cuda()
    got = vaep.step_conv(xd, wd, bd, starts, residual=rd)
    assert_close(got, ref, *ACC_TOL, what=f"conv3x3 halo tiles {case}")
    one = vaep.step_conv(xd, wd, bd, (0, H), residual=rd)
    assert torch.equal(got, one)


def test_conv_step_single_band_above_2gib(gpu_lib):
    """One band whose buffer exceeds a buffer resource's 2 GiB range: 2048 x 2048 pixels of
    256 bf16 channels (2.15 GB with the halo rows).  The conv kernels address only the rows
    each tile reads, so the single band runs; it equals the two-band run bit for bit, and
    sampled outputs (corners, edges, the band seam) match the float64 definition."""
    cin, cout, H, W = 256, 128, 2048, 2048
    gen = torch.Generator(device="cuda").manual_seed(261)
    x = torch.randn((1, cin, H, W), generator=gen, device="cuda").to(torch.bfloat16)
    w = seeded((cout, cin, 3, 3), 262, 1 / math.sqrt(cin * 9), dtype="bf16")
    b = seeded((cout,), 263, 0.1, dtype="bf16")
    wd, bd = to_dev(w, "bf16"), to_dev(b, "bf16")
    one = vaep.step_conv(x, wd, bd, (0, H))
    two = vaep.step_conv(x, wd, bd, (0, 1000, H))
    assert torch.equal(one, two)
    pts = [(0, 0), (0, W - 1), (H - 1, 0), (H - 1, W - 1), (999, 5), (1000, 7), (1000, W - 1), (517, 0)]
    g2 = torch.Generator().manual_seed(264)
    pts += [(int(h), int(c)) for h, c in zip(torch.randint(0, H, (24,), generator=g2),
                                              torch.randint(0, W, (24,), generator=g2))]
    xp = torch.nn.functional.pad(x[0].float(), (1, 1, 1, 1))       # zero padding at the image edges
    wdb = w.double()
    got, ref = [], []
    for h, c in pts:
        patch = xp[:, h:h + 3, c:c + 3].cpu().double()                # rows h-1..h+1, columns c-1..c+1
        ref.append((wdb * patch).sum(dim=(1, 2, 3)) + b.double())
        got.append(one[0, :, h, c].cpu().double())
    assert_close(torch.stack(got), torch.stack(ref), *ACC_TOL, what="2048^2 single-band conv, sampled pixels")


def test_upsample_conv_from_fp32_wide_tiles(gpu_lib):
    # sub-pixel upsample conv with 256-channel output tiles
    x = seeded((1, 64, 130, 260), 27, dtype="f32")
    w = seeded((256, 64, 3, 3), 28, 1 / math.sqrt(64 * 9), dtype="bf16")
    b = seeded((256,), 29, 0.1, dtype="bf16")
    ref = _conv_ref(x, w, b, False, None, "bf16", upsample=True, x_exact=True)
    got = vaep.step_conv(x.cuda(), to_dev(w, "bf16"), to_dev(b, "bf16"), (0, 64, 65, 130), upsample=True)
    assert got.shape == (1, 256, 260, 520)
    _assert_subpixel_close(got, x, w, ref, "sub-pixel upsample conv, wide tiles")


@pytest.mark.parametrize("kind", ["3x3_res_cout96", "1x1_cout128", "3x3x3_causal_cout128"])
def test_conv_128x512_tiles(gpu_lib, kind):
    # 128-channel output tiles over 512 pixels (8 waves): enough pixels that the layer fills
    # the CUs with them, rows that are not a multiple of 512 (tiles straddle rows), a one-row
    # band, a ragged channel tile (96 of 128), and a second band table that must give the
    # same bits
    video = kind.startswith("3x3x3")
    cout = 96 if "cout96" in kind else 128
    ks = 1 if kind.startswith("1x1") else 3
    shape = (1, 64, 4, 130, 520) if video else (1, 64, 260, 1030)
    H = shape[-2]
    x = seeded(shape, 51, dtype="bf16")
    wshape = (cout, 64, 3, 3, 3) if video else (cout, 64, ks, ks)
    w = seeded(wshape, 52, 1 / math.sqrt(64 * ks * ks * (3 if video else 1)), dtype="bf16")
    b = seeded((cout,), 53, 0.1, dtype="bf16")
    r = seeded((shape[0], cout) + shape[2:], 54, dtype="f32") if kind.startswith("3x3_res") else None
    ref = _conv_ref(x, w, b, video, r, "bf16")
    args = (to_dev(x, "bf16"), to_dev(w, "bf16"), to_dev(b, "bf16"))
    res = None if r is None else r.cuda()
    got = vaep.step_conv(*args, (0, 77, 78, H), causal=video, residual=res)
    assert_close(got, ref, *ACC_TOL, what=f"conv {kind}, 128x512 tiles")
    again = vaep.step_conv(*args, (0, H // 2, H), causal=video, residual=res)
    assert torch.equal(again, got)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv1x1_step(gpu_lib, dtype):
    x = seeded((2, 192, 7, 45), 21, dtype=dtype)
    w = seeded((96, 192, 1, 1), 22, 1 / math.sqrt(192), dtype=dtype)
    b = seeded((96,), 23, 0.1, dtype=dtype)
    ref = _conv_ref(x, w, b, False, None, dtype)
    got = vaep.step_conv(to_dev(x, dtype), to_dev(w, dtype), to_dev(b, dtype), (0, 3, 7))
    assert_close(got, ref, *ACC_TOL, what="conv1x1")


def _assert_subpixel_close(got, x, w, ref, what):
    # The sub-pixel upsample conv of an fp32 operand forms x_hi * w_hi in bf16 and its two
    # correction products, 2^-9 of the product each, in fp8 (operand parts e5m2, rounding
    # 2^-3; weight parts e4m3, 2^-4): every output lies within 2^-10 of sum |w| |x| over
    # its taps of the exact result, fp32 accumulation included (bf16 operands alone would
    # allow 2^-8).
    bound = _conv_ref(x.abs(), w.abs(), torch.zeros(w.shape[0]), False, None, "f32", upsample=True,
                      x_exact=True).double()
    err = (got.cpu().double() - ref.double()).abs()
    worst = (err / (bound * 2.0 ** -10 + 1e-6)).max().item()
    assert worst <= 1.0, f"{what}: error reaches {worst:.3f} of the bound"


def test_conv_from_fp32_source(gpu_lib):
    # shortcut / upsample convs read the fp32 residual stream (hi + lo bf16 passes)
    x = seeded((1, 64, 9, 21), 24, dtype="f32")
    w = seeded((128, 64, 3, 3), 25, 1 / math.sqrt(64 * 9), dtype="bf16")
    b = seeded((128,), 26, 0.1, dtype="bf16")
    ref = _conv_ref(x, w, b, False, None, "bf16", x_exact=True)
    got = vaep.step_conv(x.cuda(), to_dev(w, "bf16"), to_dev(b, "bf16"), (0, 2, 9))
    assert_close(got, ref, *ACC_TOL, what="conv from fp32 source")
    ref_up = _conv_ref(x, w, b, False, None, "bf16", upsample=True, x_exact=True)
    got_up = vaep.step_conv(x.cuda(), to_dev(w, "bf16"), to_dev(b, "bf16"), (0, 2, 9), upsample=True)
    _assert_subpixel_close(got_up, x, w, ref_up, "upsample conv from fp32 source")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_upsample_conv_step(gpu_lib, dtype):
    x = seeded((1, 64, 6, 11), 31, dtype=dtype)
    w = seeded((64, 64, 3, 3), 32, 1 / math.sqrt(64 * 9), dtype=dtype)
    b = seeded((64,), 33, 0.1, dtype=dtype)
    starts = (0, 1, 2, 6)
    ref = _conv_ref(x, w, b, False, None, dtype, upsample=True)
    got = vaep.step_conv(to_dev(x, dtype), to_dev(w, dtype), to_dev(b, dtype), starts, upsample=True)
    assert got.shape == (1, 64, 12, 22)
    assert_close(got, ref, *ACC_TOL, what="upsample conv")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cin", [32, 64, 96])
def test_causal_conv3d_step(gpu_lib, dtype, cin):
    x = seeded((1, cin, 4, 9, 11), 41, dtype=dtype)
    w = seeded((64, cin, 3, 3, 3), 42, 1 / math.sqrt(cin * 27), dtype=dtype)
    b = seeded((64,), 43, 0.1, dtype=dtype)
    r = seeded((1, 64, 4, 9, 11), 44, dtype="f32")
    ref = _conv_ref(x, w, b, True, r, dtype)
    got = vaep.step_conv(to_dev(x, dtype), to_dev(w, dtype), to_dev(b, dtype), (0, 4, 9), causal=True,
                         residual=r.cuda())
    assert_close(got, ref, *ACC_TOL, what="causal conv3d")


@pytest.mark.parametrize("cin", [64, 96])
def test_causal_conv3d_step_wide_tiles(gpu_lib, cin):
    # causal 3x3x3 conv on 256-channel output tiles of the wide kernel (96 input channels:
    # half-empty second channel step per tap)
    x = seeded((1, cin, 4, 130, 260), 45, dtype="bf16")
    w = seeded((256, cin, 3, 3, 3), 46, 1 / math.sqrt(cin * 27), dtype="bf16")
    b = seeded((256,), 47, 0.1, dtype="bf16")
    r = seeded((1, 256, 4, 130, 260), 48, dtype="f32")
    ref = _conv_ref(x, w, b, True, r, "bf16")
    got = vaep.step_conv(to_dev(x, "bf16"), to_dev(w, "bf16"), to_dev(b, "bf16"), (0, 61, 62, 130), causal=True,
                         residual=r.cuda())
    assert_close(got, ref, *ACC_TOL, what=f"causal conv3d, wide tiles, cin {cin}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_groupnorm_step(gpu_lib, dtype):
    B, C, H, W, G = 2, 128, 11, 19, 32
    starts = (0, 2, 5, 11)
    x = seeded((B, C, H, W), 51, 2.0, offset=3.0, dtype="f32")
    g = seeded((C,), 52, 0.25, offset=1.0, dtype="f32")
    be = seeded((C,), 53, 0.1, dtype="f32")
    x5 = _x5(x)
    _, m, v = ops.groupnorm_moments(x5, G)
    ref = Precision(dtype).finish(ops.groupnorm_apply(x5, m, v, g, be, 1e-6, act=True))[:, :, 0]
    odt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y, moments, merged = vaep.step_groupnorm(x.cuda(), G, 1e-6, g.cuda(), be.cuda(), starts, out_dtype=odt)
    assert_close(y, ref, *STEP_TOL[dtype], what="groupnorm")
    # merged statistics and every band's local moments against the two-pass definition
    assert_close(merged[0].view(B, G), m, 1e-4, 1e-5, "merged mean")
    assert_close(merged[1].view(B, G), v, 1e-3, 1e-5, "merged var")
    for i, (s, e) in enumerate(zip(starts, starts[1:])):
        cnt, mi, vi = ops.groupnorm_moments(x5[:, :, :, s:e], G)
        assert torch.all(moments[0, i].cpu() == cnt)
        assert_close(moments[1, i].view(B, G), mi, 1e-4, 1e-5, f"band {i} mean")
        assert_close(moments[2, i].view(B, G), vi, 1e-3, 1e-5, f"band {i} var")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm_step(gpu_lib, dtype):
    x = seeded((1, 96, 3, 7, 10), 61, 1.5, dtype="f32")
    g = seeded((96,), 62, 0.25, offset=1.0, dtype="f32")
    ref = Precision(dtype).finish(ops.rmsnorm(x, g, 1e-6, act=True))
    odt = torch.bfloat16 if dtype == "bf16" else torch.float32
    got = vaep.step_rmsnorm(x.cuda(), 1e-6, g.cuda(), (0, 1, 7), out_dtype=odt)
    assert_close(got, ref, *STEP_TOL[dtype], what="rmsnorm")


def _attn_ref(x, groups, g, be, wq, bq, wk, bk, wv, bv, wo, bo, dtype):
    fin = Precision(dtype).finish
    x5 = _x5(x)
    if groups:
        _, m, v = ops.groupnorm_moments(x5, groups)
        h = fin(ops.groupnorm_apply(x5, m, v, g, be, 1e-6, act=False))
    else:
        h = fin(ops.rmsnorm(x5, g, 1e-6, act=False))
    c = x5.shape[1]
    y = torch.empty_like(x5)
    for n in range(x5.shape[0]):
        for t in range(x5.shape[2]):
            tok = h[n, :, t].reshape(c, -1).T.double()
            q = fin(tok @ wq.double().T + bq.double())
            k = fin(tok @ wk.double().T + bk.double())
            v_ = fin(tok @ wv.double().T + bv.double())
            o = fin(ops.attention_rows(q, k, v_, 1 / math.sqrt(c)))
            out = x5[n, :, t].reshape(c, -1).T.double() + o.double() @ wo.double().T + bo.double()
            y[n, :, t] = Precision(dtype).acc(out).T.reshape(c, x5.shape[3], x5.shape[4])
    return y if x.dim() == 5 else y[:, :, 0]


@pytest.mark.parametrize("case", [
    ("bf16", 512, 32, (1, 8, 25), (0, 3, 8)),          # 200 tokens: ragged key and query tiles
    ("bf16", 384, 0, (2, 6, 10), (0, 1, 6)),           # per-frame span, RMSNorm pre-norm
    ("bf16", 384, 0, (2, 8, 13), (0, 3, 8)),           # 104 tokens a frame: a ragged last key tile
    ("bf16", 256, 32, (1, 16, 32), (0, 5, 16)),         # 512 tokens, 64-channel wave slices
    ("bf16", 128, 32, (1, 12, 20), (0, 12)),            # 240 tokens, 32-channel wave slices
    ("f32", 64, 8, (1, 8, 8), (0, 3, 8)),
])
def test_attention_step(gpu_lib, case):
    dtype, C, G, (T, H, W), starts = case
    video = G == 0
    shape = (1, C, T, H, W) if video else (1, C, H, W)
    x = seeded(shape, 71, dtype="f32")
    g = seeded((C,), 72, 0.25, offset=1.0, dtype="f32")
    be = seeded((C,), 73, 0.1, dtype="f32")
    ws = [seeded((C, C), 74 + i, 1 / math.sqrt(C), dtype=dtype) for i in range(4)]
    bs = [seeded((C,), 80 + i, 0.1, dtype=dtype) for i in range(4)]
    ref = _attn_ref(x, G, g, be, ws[0], bs[0], ws[1], bs[1], ws[2], bs[2], ws[3], bs[3], dtype)
    dev = [to_dev(t, dtype) for t in ws + bs]
    got = vaep.step_attention(x.cuda(), G, 1e-6, g.cuda(), be.cuda(), dev[0], dev[4], dev[1],
                              dev[5], dev[2], dev[6], dev[3], dev[7], starts)
    assert_close(got, ref, *STEP_TOL[dtype], what=f"attention {case}")


def test_attention_step_d512_full_grid(gpu_lib):
    """d = 512 over 128 x 128 tokens on uneven bands: 256 blocks of 64 queries fill the CUs,
    so the one-workgroup-per-CU form runs (the 200-token case above runs the 32-query form).
    Sampled query rows of every band, first and last tokens included, against the float64
    reference; the output does not depend on the band table."""
    C, G, H, W = 512, 32, 128, 128
    starts = (0, 31, 64, 96, 128)
    x = seeded((1, C, H, W), 241, dtype="f32")
    g = seeded((C,), 242, 0.25, offset=1.0, dtype="f32")
    be = seeded((C,), 243, 0.1, dtype="f32")
    ws = [seeded((C, C), 244 + i, 1 / math.sqrt(C), dtype="bf16") for i in range(4)]
    bs = [seeded((C,), 250 + i, 0.1, dtype="bf16") for i in range(4)]
    dev = [to_dev(t, "bf16") for t in ws + bs]
    xd, gd, bed = x.cuda(), g.cuda(), be.cuda()
    got = vaep.step_attention(xd, G, 1e-6, gd, bed, dev[0], dev[4], dev[1], dev[5], dev[2], dev[6],
                              dev[3], dev[7], starts)
    whole = vaep.step_attention(xd, G, 1e-6, gd, bed, dev[0], dev[4], dev[1], dev[5], dev[2], dev[6],
                                dev[3], dev[7], (0, H))
    assert torch.equal(got, whole)
    # float64 reference of the sampled query rows (same rounding points as _attn_ref)
    fin = Precision("bf16").finish
    x5 = x[:, :, None]
    _, m, v = ops.groupnorm_moments(x5, G)
    h = fin(ops.groupnorm_apply(x5, m, v, g, be, 1e-6, act=False))
    tok = h[0, :, 0].reshape(C, -1).T.double()
    q = fin(tok @ ws[0].double().T + bs[0].double())
    k = fin(tok @ ws[1].double().T + bs[1].double())
    v_ = fin(tok @ ws[2].double().T + bs[2].double())
    gen = torch.Generator().manual_seed(245)
    rows = torch.cat([torch.tensor([0, H * W - 1] + [s * W for s in starts[1:-1]] + [s * W - 1 for s in starts[1:-1]]),
                      torch.randint(0, H * W, (184,), generator=gen)])
    o = fin(ops.attention_rows(q[rows], k, v_, 1 / math.sqrt(C)))
    xr = x[0].reshape(C, -1).T.double()[rows]
    out = xr + o.double() @ ws[3].double().T + bs[3].double()
    ref = Precision("bf16").acc(out)
    sel = got[0].reshape(C, -1).T[rows].cpu()
    assert_close(sel, ref, *STEP_TOL["bf16"], what="attention d=512, 16384 tokens, sampled rows")
    # The attention branch alone (output minus the residual input) against attention computed
    # exactly on the same bf16 Q, K and V: its rounding is one bf16 rounding of O plus P's
    # bf16 rounding averaged over 16384 keys, so rel-L2 stays below 2^-9.
    branch = sel.double() - xr
    assert_close(branch, o.double() @ ws[3].double().T + bs[3].double(), 1.0, 2.0 ** -9,
                 what="attention d=512 branch, 16384 tokens", log=True)


def test_attention_step_d384_video_whole_key_range(gpu_lib):
    """d = 384 per-frame attention over 3 frames of 64 x 96 tokens: 144 blocks of 128
    queries, enough that the keys are not split in halves.  Sampled query rows of every frame
    and band against the float64 reference; the output does not depend on the band table."""
    C, T, H, W = 384, 3, 64, 96
    starts = (0, 21, 40, 64)
    x = seeded((1, C, T, H, W), 261, dtype="f32")
    g = seeded((C,), 262, 0.25, offset=1.0, dtype="f32")
    be = seeded((C,), 263, 0.1, dtype="f32")
    ws = [seeded((C, C), 264 + i, 1 / math.sqrt(C), dtype="bf16") for i in range(4)]
    bs = [seeded((C,), 270 + i, 0.1, dtype="bf16") for i in range(4)]
    dev = [to_dev(t, "bf16") for t in ws + bs]
    xd, gd, bed = x.cuda(), g.cuda(), be.cuda()
    args = (dev[0], dev[4], dev[1], dev[5], dev[2], dev[6], dev[3], dev[7])
    got = vaep.step_attention(xd, 0, 1e-6, gd, bed, *args, starts)
    whole = vaep.step_attention(xd, 0, 1e-6, gd, bed, *args, (0, H))
    assert torch.equal(got, whole)
    fin = Precision("bf16").finish
    h = fin(ops.rmsnorm(x, g, 1e-6, act=False))
    gen = torch.Generator().manual_seed(275)
    for t in range(T):
        tok = h[0, :, t].reshape(C, -1).T.double()
        q = fin(tok @ ws[0].double().T + bs[0].double())
        k = fin(tok @ ws[1].double().T + bs[1].double())
        v_ = fin(tok @ ws[2].double().T + bs[2].double())
        rows = torch.cat([torch.tensor([0, H * W - 1] + [s * W for s in starts[1:-1]] + [s * W - 1 for s in starts[1:-1]]),
                          torch.randint(0, H * W, (60,), generator=gen)])
        o = fin(ops.attention_rows(q[rows], k, v_, 1 / math.sqrt(C)))
        out = x[0, :, t].reshape(C, -1).T.double()[rows] + o.double() @ ws[3].double().T + bs[3].double()
        ref = Precision("bf16").acc(out)
        sel = got[0, :, t].reshape(C, -1).T[rows].cpu()
        assert_close(sel, ref, *STEP_TOL["bf16"], what=f"attention d=384, frame {t}, sampled rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_temporal_upsample_step(gpu_lib, dtype):
    C = 64
    x = seeded((1, C, 3, 5, 6), 91, dtype="f32")
    w = seeded((2 * C, C, 3, 1, 1), 92, 1 / math.sqrt(3 * C), dtype=dtype)
    b = seeded((2 * C,), 93, 0.1, dtype=dtype)
    z = ops.conv_full(x, w, b, True, Precision(dtype).acc)     # fp32 source: hi + lo passes
    ref = ops.temporal_upsample_interleave(x, z)
    got = vaep.step_temporal_upsample(x.cuda(), to_dev(w, dtype), to_dev(b, dtype), (0, 2, 5))
    assert got.shape == (1, C, 5, 5, 6)
    assert_close(got, ref, *ACC_TOL, what="temporal upsample")


def test_groupnorm_merge_entry_point(gpu_lib):
    from synth.gen import uniform_draws
    n_shards, n_stats = 5, 37
    mean = seeded((n_shards, n_stats), 101, 3.0, dtype="f32")
    var = seeded((n_shards, n_stats), 102, 1.0, dtype="f32").abs()
    counts = torch.from_numpy((uniform_draws(103, n_shards * n_stats) * 1000).astype("int64")).view(n_shards, n_stats)
    counts[2, 5] = 0
    counts[:, 7] = 0
    # reference per statistic (column): counts differ per column
    m_ref = torch.zeros(n_stats, dtype=torch.float64)
    v_ref = torch.zeros(n_stats, dtype=torch.float64)
    for s in range(n_stats):
        cs = [int(counts[i, s]) for i in range(n_shards)]
        if sum(cs) == 0:
            continue
        m, v = ops.merge_moments(cs, [mean[i, s:s + 1] for i in range(n_shards)],
                                 [var[i, s:s + 1] for i in range(n_shards)])
        m_ref[s], v_ref[s] = m.item(), v.item()
    gm, gv = vaep.groupnorm_merge(mean.cuda(), var.cuda(), counts.cuda())
    assert_close(gm, m_ref, 1e-5, 1e-6, "merged mean")
    assert_close(gv, v_ref, 1e-5, 1e-6, "merged var")
    assert gm[7].item() == 0.0 and gv[7].item() == 0.0


# ----------------------------------------------------------------------------- band invariance
# Every step computes each output element with the same arithmetic whatever the band
# table: convs and attention read the same operands in the same order, and GroupNorm
# merges fp64 band moments rounded once to fp32.  Partitions must give bit-equal results.
PARTITIONS = [(0, 10), (0, 3, 10), (0, 1, 5, 9, 10), (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10)]


@pytest.mark.parametrize("kind", ["conv3", "conv3_f32src", "upconv_f32src", "conv1_f32src", "conv333"])
def test_conv_band_invariance(gpu_lib, kind):
    video = kind == "conv333"
    shape = (1, 64, 3, 10, 12) if video else (1, 64, 10, 12)
    src = "f32" if "f32src" in kind else "bf16"
    x = to_dev(seeded(shape, 201, dtype=src), src)
    k = (64, 64, 3, 3, 3) if video else ((64, 64, 1, 1) if kind == "conv1_f32src" else (64, 64, 3, 3))
    w = to_dev(seeded(k, 202, 0.05), "bf16")
    b = to_dev(seeded((64,), 203, 0.1), "bf16")
    outs = [vaep.step_conv(x, w, b, p, causal=video, upsample=kind.startswith("up")) for p in PARTITIONS]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_groupnorm_band_invariance(gpu_lib):
    x = seeded((2, 512, 10, 12), 211, 3.0, offset=0.5, dtype="f32").cuda()
    g = seeded((512,), 212, 0.25, offset=1.0, dtype="f32").cuda()
    be = seeded((512,), 213, 0.1, dtype="f32").cuda()
    outs = [vaep.step_groupnorm(x, 32, 1e-6, g, be, p)[0] for p in PARTITIONS]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("G", [32, 0])
def test_attention_band_invariance(gpu_lib, G):
    C = 512 if G else 384
    x = seeded((1, C, 10, 12), 221, dtype="f32").cuda()
    g = seeded((C,), 222, 0.25, offset=1.0, dtype="f32").cuda()
    be = seeded((C,), 223, 0.1, dtype="f32").cuda()
    ws = [to_dev(seeded((C, C), 224 + i, 1 / math.sqrt(C)), "bf16") for i in range(4)]
    bs = [to_dev(seeded((C,), 230 + i, 0.1), "bf16") for i in range(4)]
    outs = [vaep.step_attention(x, G, 1e-6, g, be, ws[0], bs[0], ws[1], bs[1], ws[2], bs[2], ws[3], bs[3], p)
            for p in PARTITIONS]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
