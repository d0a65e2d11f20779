"""Shared helpers of the test-suite: seeded inputs and the parity bar."""
import numpy as np
import torch

from synth.gen import normal_draws, round_bf16

# Parity bar for a whole decode: bf16 max-abs 2e-2 and rel-L2 1e-2; fp32 1e-4 for both.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
# Whole decodes are compared with the oracle's exact decode (fp32 storage, fp64 math).
# A bf16-rounding oracle is a second, independent bf16 rounding sequence: its distance
# to the HIP path is about sqrt(2) times either one's distance to the exact decode.
REFERENCE_PRECISION = "f32"
# Band decode vs full decode on the GPU.
BAND_VS_FULL_REL = 1e-3


def seeded(shape, seed, scale=1.0, offset=0.0, dtype="bf16"):
    """CPU fp32 tensor of seeded normals (bf16-representable when dtype is bf16)."""
    n = int(np.prod(shape))
    t = torch.from_numpy((normal_draws(seed, n) * scale + offset).astype(np.float32).reshape(shape))
    return round_bf16(t) if dtype == "bf16" else t


def to_dev(t, dtype):
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda().contiguous()


def errors(got, ref):
    g = got.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert torch.isfinite(g).all(), "non-finite output"
    d = g - r
    return d.abs().max().item(), (d.norm() / max(r.norm().item(), 1e-30)).item()


# Measured parity figures of the session, printed in pytest's terminal summary
# (tests/conftest.py) so that the margins to the bar are visible in the run's log.
PARITY_LOG = []


def record(what, max_abs, rel_l2, bar_abs=None, bar_rel=None):
    PARITY_LOG.append((what, max_abs, rel_l2, bar_abs, bar_rel))


def assert_close(got, ref, max_abs, rel_l2, what="", log=False):
    ma, rl = errors(got, ref)
    if log:
        record(what, ma, rl, max_abs, rel_l2)
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max-abs {ma:.3e} (bar {max_abs}), rel-L2 {rl:.3e} (bar {rel_l2})"
    return ma, rl
