"""Write oracle outputs of the full-size presets to tests/golden/.

Runs only the CPU oracle (``oracle.decode_full`` with float32 storage and
float64 arithmetic: the exact decode the bf16 path approximates) on the seeded
latents and weights of ``synth`` and stores, per preset:

* ``cfg{i}_oracle_samples.npy``: the decoded values at ``N_SAMPLES`` flat
  positions drawn from ``numpy.random.default_rng(SAMPLE_SEED + cfg)``;
* ``cfg{i}_oracle_summary.json``: whole-tensor summary statistics;
* ``cfg3_oracle_full.npy``: the whole 1x3x1024x1024 output of the 1024^2 preset;
* ``cfg{4,5}_oracle_rows.npz``: every output row within ``ROW_MARGIN`` rows of
  each band boundary of the preset's band table and of the image's top and
  bottom edges (``rows``: the row indices, ``values``: ``[B, 3, (T,) rows, W]``);
  the validation page's correctness tests compare full tensors including the
  boundary rows;
* with ``--full``: the whole outputs of presets 4 and 5 (50 MB and 81 MB) under
  ``tests/golden/full/``, which is not committed.

GPU parity tests at full size compare the HIP decode against these.

Usage: python tests/golden/make_full_size_golden.py [--full] [cfg ...]   (default 3 4 5)
Takes about 2, 8 and 10 minutes for presets 3, 4 and 5 on 8 cores.
"""
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import decode_full, Precision  # noqa: E402
from synth import make_latent, make_params, preset  # noqa: E402

N_SAMPLES = 32768
SAMPLE_SEED = 20260901
ROW_MARGIN = 8
HERE = os.path.dirname(os.path.abspath(__file__))
FULL_DIR = os.path.join(HERE, "full")


def sample_positions(cfg_id: int, numel: int) -> np.ndarray:
    return np.random.default_rng(SAMPLE_SEED + cfg_id).integers(0, numel, N_SAMPLES)


def boundary_rows(cfg) -> np.ndarray:
    """Output rows within ROW_MARGIN of each interior band boundary and of the two image edges."""
    scale = cfg.output_shape()[-2] // cfg.latent_h
    height = cfg.output_shape()[-2]
    rows = set(range(ROW_MARGIN)) | set(range(height - ROW_MARGIN, height))
    for s in cfg.band_starts[1:-1]:
        rows |= set(range(scale * s - ROW_MARGIN, scale * s + ROW_MARGIN))
    return np.array(sorted(r for r in rows if 0 <= r < height), dtype=np.int64)


def main(ids, full):
    for i in ids:
        cfg = preset(i)
        t0 = time.time()
        y = decode_full(cfg, make_params(cfg), make_latent(cfg), Precision("f32"))
        dt = time.time() - t0
        flat = y.reshape(-1).numpy()
        pos = sample_positions(i, flat.size)
        np.save(os.path.join(HERE, f"cfg{i}_oracle_samples.npy"), flat[pos].astype(np.float32))
        if i == 3:
            np.save(os.path.join(HERE, "cfg3_oracle_full.npy"), y.numpy().astype(np.float32))
        else:
            rows = boundary_rows(cfg)
            np.savez(os.path.join(HERE, f"cfg{i}_oracle_rows.npz"), rows=rows,
                     values=y.numpy()[..., rows, :].astype(np.float32))
            if full:
                os.makedirs(FULL_DIR, exist_ok=True)
                np.save(os.path.join(FULL_DIR, f"cfg{i}_oracle_full.npy"), y.numpy().astype(np.float32))
        meta = {
            "config": cfg.name, "oracle_storage": "f32", "shape": list(y.shape), "n_samples": N_SAMPLES,
            "sample_seed": SAMPLE_SEED + i, "oracle_seconds": round(dt, 1),
            "torch_threads": torch.get_num_threads(),
            "mean": float(y.double().mean()), "std": float(y.double().std()),
            "absmax": float(y.abs().max()), "l2": float(y.double().norm()),
            "channel_mean": [float(v) for v in y.double().mean(dim=[d for d in range(y.dim()) if d != 1])],
        }
        with open(os.path.join(HERE, f"cfg{i}_oracle_summary.json"), "w") as fh:
            json.dump(meta, fh, indent=1)
        print(f"cfg{i}: {dt:.1f} s  {meta}", flush=True)
        del y


if __name__ == "__main__":
    args = sys.argv[1:]
    want_full = "--full" in args
    main([int(a) for a in args if a != "--full"] or [3, 4, 5], want_full)
