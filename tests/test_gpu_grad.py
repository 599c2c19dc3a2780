"""GPU parity of the training backward of the joint sCM loss (t2va_scm_grad,
through the C ABI) against the fp64 oracle (torch float64 autograd with gbar
held constant).

Tolerance: the gradient of every student weight within 2e-2 relative L2, the
bound used for J and gbar: the backward's operands are stored in bf16 (unit
roundoff 2^-9) between its steps and accumulated in fp32, like the forward's.
The target's own outputs must equal t2va_scm_target's bit for bit (same
kernels, same order).
"""
import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2
WEIGHTS = ("w_in_v", "w_in_a", "w_t", "w_qkv", "w_out_v", "w_out_a")

RAGGED = inputs.Config("ragged", B=2, Nv=300, Na=45, Nt=20, Ntv=13, Cv=128, Ca=64, d=256, H=2,
                       in_dtype="bf16", beta=1.5, gamma=0.7, mask_mode="scatter", w_v=0.5, w_a=2.0,
                       index=11)
RAGGED64 = inputs.Config("ragged64", B=1, Nv=130, Na=70, Nt=0, Ntv=0, Cv=64, Ca=64, d=256, H=4,
                         in_dtype="bf16", index=12)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def say(*a):
    print(*a, flush=True)


def run_grad(problem):
    from joint_video_audio_trigflow_amd import _lib
    cfg = problem["cfg"]
    dev = _lib.to_device_problem(problem)
    dt = _lib.DTYPE_BF16 if cfg.in_dtype == "bf16" else _lib.DTYPE_FP32
    op = _lib.ScmGrad(cfg, in_dtype=dt, weight_dtype=dt)
    out, grads = op(dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"],
                    dev["text"], dev["text_mask"], dev["t"])
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in out.items()}, {k: v.cpu().numpy() for k, v in grads.items()},
            dev, dt)


ALLPAD = inputs.Config("allpad", B=2, Nv=96, Na=40, Nt=16, Ntv=0, Cv=64, Ca=64, d=256, H=2,
                       in_dtype="bf16", index=13)
MAXB = inputs.Config("maxbatch", B=64, Nv=64, Na=32, Nt=8, Ntv=5, Cv=64, Ca=64, d=128, H=2,
                     in_dtype="bf16", mask_mode="scatter", index=14)
ONETOK = inputs.Config("onetoken", B=2, Nv=1, Na=1, Nt=3, Ntv=2, Cv=64, Ca=64, d=128, H=1,
                       in_dtype="bf16", index=16)

CASES = [inputs.CONFIGS["tiny"], RAGGED, RAGGED64, inputs.CONFIGS["tiny"].replace(param="rf"),
         RAGGED.replace(param="rf"), inputs.CONFIGS["small"], ALLPAD, MAXB, ONETOK]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name + ("-rf" if c.param == "rf" else ""))
def test_scm_grad_matches_oracle(cfg):
    say(f"scm_grad {cfg.name} param={cfg.param}")
    p = inputs.make_problem(cfg)
    out, grads, dev, dt = run_grad(p)
    res = oracle.scm_target(p)
    ref = oracle.scm_loss_and_grads(p, res)
    errs = {k: rel_l2(grads[k], ref[k]) for k in WEIGHTS}
    say("  rel-L2 per weight:", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert np.all(np.isfinite(grads[k])), k
        assert e <= TOL_GRAD, (cfg.name, k, e)
    # the target's outputs are exactly t2va_scm_target's
    from joint_video_audio_trigflow_amd import _lib
    op = _lib.ScmTarget(cfg, in_dtype=dt, weight_dtype=dt)
    tgt = op(dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"],
             dev["text"], dev["text_mask"], dev["t"])
    torch.cuda.synchronize()
    for k in ("gbar_v", "gbar_a", "norms", "loss"):
        assert np.array_equal(out[k], tgt[k].cpu().numpy()), k


def test_scm_grad_deterministic():
    say("scm_grad determinism")
    p = inputs.make_problem(RAGGED)
    _, g1, _, _ = run_grad(p)
    _, g2, _, _ = run_grad(p)
    for k in WEIGHTS:
        assert np.array_equal(g1[k], g2[k]), k


def test_scm_grad_batch_is_the_sum_over_samples():
    say("scm_grad batch additivity")
    p = inputs.make_problem(RAGGED)
    _, g, _, _ = run_grad(p)
    parts = []
    for b in range(2):
        one = {k: (v[b:b + 1] if isinstance(v, np.ndarray) else v) for k, v in p["data"].items()}
        parts.append(run_grad(dict(p, cfg=RAGGED.replace(B=1), data=one))[1])
    for k in WEIGHTS:
        # fp32 sums in a different order: equal to rounding
        assert rel_l2(g[k], parts[0][k] + parts[1][k]) < 1e-3, k
