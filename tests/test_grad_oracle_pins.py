"""Pins of the fp64 oracle for the training backward of the joint sCM loss.

* The student's torch forward used for the gradient equals the sCM oracle's
  x0-prediction of the student (dual-number numpy code, an independent route).
* Central finite differences of the loss as a function of each student
  weight, sum_m w_m ||F(W) - F(W0) - gbar||^2 with gbar fixed (the loss the
  pages define with sg(F) = F(W0)), match the gradient's directional
  derivative along random directions; with the x0-prediction block and through
  the TrigFlow wrapper.
* A planted mistake (the sign of gbar flipped in the loss) fails the FD pin.
* The gradient of a batch is the sum of the per-sample gradients.
"""
import math

import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs

WEIGHTS = oracle.grad_oracle.WEIGHTS


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module", params=["x0", "rf"])
def tiny_grad(request):
    cfg = inputs.CONFIGS["tiny"].replace(param=request.param)
    p = inputs.make_problem(cfg)
    res = oracle.scm_target(p)
    g = oracle.scm_loss_and_grads(p, res)
    return p, res, g


def test_torch_forward_matches_the_dual_oracle(tiny_grad):
    p, res, _ = tiny_grad
    F = oracle.student_fields(p, p["student"])
    for m in "va":
        assert rel_l2(F[m], res[f"F_S_{m}"]) < 1e-12


def _fd(p, res, name, direction, h, sign=1.0):
    cfg = p["cfg"]
    F0 = oracle.student_fields(p, p["student"])
    vals = []
    for s in (+1, -1):
        W = dict(p["student"])
        W[name] = np.asarray(W[name], np.float64) + s * h * direction
        F = oracle.student_fields(p, W)
        L = 0.0
        for m, w in (("v", cfg.w_v), ("a", cfg.w_a)):
            r = F[m] - F0[m] - sign * res[f"gbar_{m}"]
            L += w * float(np.sum(r * r))
        vals.append(L)
    return (vals[0] - vals[1]) / (2 * h)


@pytest.mark.parametrize("name", WEIGHTS)
def test_gradient_matches_central_differences(tiny_grad, name):
    p, res, g = tiny_grad
    rng = np.random.default_rng(hash(name) % 2**32)
    direction = rng.standard_normal(np.shape(p["student"][name]))
    direction /= np.linalg.norm(direction)
    fd = _fd(p, res, name, direction, 1e-4)
    an = float(np.sum(g[name] * direction))
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3 * np.linalg.norm(g[name])), (name, fd, an)


def test_fd_catches_a_flipped_target_sign(tiny_grad):
    p, res, g = tiny_grad
    rng = np.random.default_rng(9)
    direction = rng.standard_normal(np.shape(p["student"]["w_qkv"]))
    direction /= np.linalg.norm(direction)
    fd = _fd(p, res, "w_qkv", direction, 1e-4, sign=-1.0)
    an = float(np.sum(g["w_qkv"] * direction))
    assert abs(fd - an) > 0.5 * abs(an)


def test_batch_gradient_is_the_sum_over_samples():
    cfg = inputs.Config("pair", B=2, Nv=64, Na=16, Nt=8, Ntv=5, Cv=64, Ca=64, d=128, H=2,
                        in_dtype="fp32", gamma=0.5, mask_mode="scatter", index=21)
    p = inputs.make_problem(cfg)
    g = oracle.scm_loss_and_grads(p)
    parts = []
    for b in range(2):
        one = {k: (v[b:b + 1] if isinstance(v, np.ndarray) else v) for k, v in p["data"].items()}
        parts.append(oracle.scm_loss_and_grads(dict(p, cfg=cfg.replace(B=1), data=one)))
    for k in WEIGHTS:
        assert rel_l2(g[k], parts[0][k] + parts[1][k]) < 1e-12, k
    assert abs(g["loss_sum"] - parts[0]["loss_sum"] - parts[1]["loss_sum"]) < 1e-12


def test_query_chunked_backward_matches_the_plain_one():
    """The chunked, recomputed attention (used at high resolution, where the
    logits do not fit in memory) gives the plain autograd's loss and
    gradients: the same arithmetic, evaluated block by block.  Query blocks of
    17 rows do not divide the 80 queries of the tiny workload."""
    p = inputs.make_problem(inputs.CONFIGS["tiny"])
    ref = oracle.scm_target(p)
    a = oracle.scm_loss_and_grads(p, ref)
    b = oracle.scm_loss_and_grads(p, ref, query_chunk=17)
    assert np.allclose(a["loss"], b["loss"], rtol=1e-13, atol=0)
    for k in oracle.grad_oracle.WEIGHTS:
        assert np.allclose(a[k], b[k], rtol=1e-10, atol=1e-14 * np.max(np.abs(a[k]))), k
