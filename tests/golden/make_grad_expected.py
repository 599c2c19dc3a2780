"""Write oracle expectations for the training backward at full size (calls only
oracle/ and the seeded inputs).

For the standard and high-resolution workloads this runs the fp64 sCM oracle
(for gbar) and the fp64 autograd backward, and stores per student weight: the
gradient's norm, its inner products with four seeded random directions, and
2048 seeded sampled entries; plus the per-sample loss.  The GPU test draws the
same directions and indices from the same seeds.  At high resolution the
attention is evaluated in blocks of query rows recomputed in the backward
(the oracle's query_chunk), since 29k x 29k logits per head do not fit.
Usage: python tests/golden/make_grad_expected.py [names...]
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
WEIGHTS = ("w_in_v", "w_in_a", "w_t", "w_qkv", "w_out_v", "w_out_a")
N_DIR, N_SAMPLE = 4, 2048


def probes(shape, name):
    """Seeded unit directions and sampled flat indices for one weight."""
    rng = np.random.default_rng(700 + WEIGHTS.index(name))
    dirs = rng.standard_normal((N_DIR,) + tuple(shape))
    dirs /= np.sqrt(np.sum(dirs.reshape(N_DIR, -1) ** 2, axis=1)).reshape((N_DIR,) + (1,) * len(shape))
    idx = rng.choice(int(np.prod(shape)), size=min(N_SAMPLE, int(np.prod(shape))), replace=False)
    return dirs, np.sort(idx)


def main(names):
    for name in names:
        cfg = inputs.CONFIGS[name]
        t0 = time.time()
        p = inputs.make_problem(cfg)
        g = oracle.scm_loss_and_grads(p, query_chunk=4096 if cfg.Nv > 10000 else None)
        out = {"t": p["data"]["t"], "loss": g["loss"]}
        for k in WEIGHTS:
            dirs, idx = probes(g[k].shape, k)
            out[f"{k}_norm"] = np.linalg.norm(g[k])
            out[f"{k}_proj"] = np.array([np.sum(g[k] * dv) for dv in dirs])
            out[f"{k}_idx"] = idx
            out[f"{k}_val"] = g[k].reshape(-1)[idx]
        np.savez_compressed(os.path.join(OUT, f"expected_grad_{name}.npz"), **out)
        print(f"grad {name}: {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["standard"])
