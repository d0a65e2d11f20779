"""Write sampled oracle outputs of the full-size presets to tests/golden/.

Runs only the CPU oracle (``oracle.decode_full`` with float32 storage and
float64 arithmetic: the exact decode the bf16 path approximates) on the seeded
latents and weights of ``synth`` and stores the decoded values at
``N_SAMPLES`` flat positions drawn from ``numpy.random.default_rng(SAMPLE_SEED
+ cfg)``, plus whole-tensor summary statistics.  GPU parity tests at full size
compare the HIP decode at the same positions.

Usage: python tests/golden/make_full_size_golden.py [cfg ...]   (default 3 4 5)
Takes tens of minutes on 8 cores for configs 4 and 5.
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
HERE = os.path.dirname(os.path.abspath(__file__))


def sample_positions(cfg_id: int, numel: int) -> np.ndarray:
    return np.random.default_rng(SAMPLE_SEED + cfg_id).integers(0, numel, N_SAMPLES)


def main(ids):
    for i in ids:
        cfg = preset(i)
        t0 = time.time()
        y = decode_full(cfg, make_params(cfg), make_latent(cfg), Precision("f32"))
        dt = time.time() - t0
        flat = y.reshape(-1).numpy()
        pos = sample_positions(i, flat.size)
        np.save(os.path.join(HERE, f"cfg{i}_oracle_samples.npy"), flat[pos].astype(np.float32))
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
    main([int(a) for a in sys.argv[1:]] or [3, 4, 5])
