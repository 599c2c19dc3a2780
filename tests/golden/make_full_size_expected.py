"""Write oracle expectations for the full-size workloads (calls only oracle/ and the seeded inputs).

For each of the standard, stress and high-resolution workloads this runs the
fp64 oracle on the whole target and stores, per sample, the per-modality L2
norms, the loss, and J and gbar on a fixed random sample of rows (48 video
and 24 audio rows).  With --storage it also runs the oracle with bf16 rounding
at the points where the GPU path stores bf16 (keys prefixed "st_"), which
measures how sensitive each sample is to that storage precision.
With --dmd it does the same for the joint DMD term (guided teacher, fake-score
block): per sample the residual scales, the loss and Delta on the sampled rows,
into expected_dmd_<name>.npz.
Usage: python tests/golden/make_full_size_expected.py [--storage] [--dmd] [names...]
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


def rows_of(res, cfg, prefix=""):
    rv, ra = sample_rows(cfg)
    b = np.arange(cfg.B)[:, None]
    return {prefix + "J_v": res["J_v"][b, rv].astype(np.float32),
            prefix + "J_a": res["J_a"][b, ra].astype(np.float32),
            prefix + "gbar_v": res["gbar_v"][b, rv].astype(np.float32),
            prefix + "gbar_a": res["gbar_a"][b, ra].astype(np.float32),
            prefix + "norms": res["norms"], prefix + "loss": res["loss"]}


def dmd_rows_of(res, cfg, prefix=""):
    rv, ra = sample_rows(cfg)
    b = np.arange(cfg.B)[:, None]
    return {prefix + "delta_v": res["delta_v"][b, rv].astype(np.float32),
            prefix + "delta_a": res["delta_a"][b, ra].astype(np.float32),
            prefix + "scales": res["scales"], prefix + "loss": res["loss"]}


def main_dmd(names, storage):
    from oracle import scm_oracle
    for name in names:
        cfg = inputs.CONFIGS[name]
        t0 = time.time()
        p = inputs.make_dmd_problem(cfg)
        path = os.path.join(OUT, f"expected_dmd_{name}.npz")
        if os.path.exists(path):
            out = dict(np.load(path))
        else:
            scm_oracle.STORAGE = None
            res = oracle.dmd_target(p)
            rv, ra = sample_rows(cfg)
            out = dict(rows_v=rv, rows_a=ra, t=res["t"], **dmd_rows_of(res, cfg))
        if storage:
            scm_oracle.STORAGE = "bf16"
            out.update(dmd_rows_of(oracle.dmd_target(p), cfg, "st_"))
            scm_oracle.STORAGE = None
        np.savez_compressed(path, **out)
        print(f"dmd {name}: {time.time() - t0:.0f} s", flush=True)


def main(names, storage):
    from oracle import scm_oracle
    for name in names:
        cfg = inputs.CONFIGS[name]
        t0 = time.time()
        p = inputs.make_problem(cfg)
        path = os.path.join(OUT, f"expected_{name}.npz")
        if os.path.exists(path):
            out = dict(np.load(path))
        else:
            scm_oracle.STORAGE = None
            res = oracle.scm_target(p)
            rv, ra = sample_rows(cfg)
            out = dict(rows_v=rv, rows_a=ra, t=res["t"], **rows_of(res, cfg))
        if storage:
            scm_oracle.STORAGE = "bf16"
            out.update(rows_of(oracle.scm_target(p), cfg, "st_"))
            scm_oracle.STORAGE = None
        np.savez_compressed(path, **out)
        print(f"{name}: {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    storage = "--storage" in args
    names = [a for a in args if not a.startswith("--")]
    if "--dmd" in args:
        main_dmd(names or ["standard", "stress", "high-res"], storage)
    else:
        main(names or ["standard", "stress", "high-res"], storage)
