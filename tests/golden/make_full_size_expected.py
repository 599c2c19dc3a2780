"""Write oracle expectations for the full-size workloads (calls only oracle/ and the seeded inputs).

For each of the standard, stress and high-resolution workloads this runs the
fp64 oracle on the whole target and stores, per sample, the per-modality L2
norms, the loss, and J and gbar on a fixed random sample of rows (48 video
and 24 audio rows).  Usage: python tests/golden/make_full_size_expected.py [names...]
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from joint_video_audio_trigflow_amd import inputs  # noqa: E402

OUT = os.path.dirname(os.path.abspath(__file__))
ROWS_V, ROWS_A = 48, 24


def sample_rows(cfg):
    rng = np.random.default_rng(7)
    rv = np.stack([np.sort(rng.choice(cfg.Nv, ROWS_V, replace=False)) for _ in range(cfg.B)])
    ra = np.stack([np.sort(rng.choice(cfg.Na, ROWS_A, replace=False)) for _ in range(cfg.B)])
    return rv, ra


def main(names):
    for name in names:
        cfg = inputs.CONFIGS[name]
        t0 = time.time()
        p = inputs.make_problem(cfg)
        res = oracle.scm_target(p)
        rv, ra = sample_rows(cfg)
        b = np.arange(cfg.B)[:, None]
        np.savez_compressed(
            os.path.join(OUT, f"expected_{name}.npz"),
            rows_v=rv, rows_a=ra,
            J_v=res["J_v"][b, rv].astype(np.float32), J_a=res["J_a"][b, ra].astype(np.float32),
            gbar_v=res["gbar_v"][b, rv].astype(np.float32), gbar_a=res["gbar_a"][b, ra].astype(np.float32),
            norms=res["norms"], loss=res["loss"], t=res["t"])
        print(f"{name}: {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["standard", "stress", "high-res"])
