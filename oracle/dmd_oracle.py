"""fp64 CPU oracle for the joint DMD term, the teacher's classifier-free
guidance and the stage-3 objective of TurboT2VA.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path; both consume the same seeded inputs.

What it computes, following "TurboT2VA：分数正则化一致性蒸馏加速 19B 视频音频联合生成"
(robotworld.top Chinese deep read of arXiv 2608.24674; [deep read]):

* Section 4: the student's on-policy paired sample x0_hat = (x0^v, x0^a) is
  perturbed to z_t with the TrigFlow noising of section 3; the per-modality
  DMD direction is the fake-score block's x0-prediction minus the teacher's,
  both taken at (z_t, t, c); the teacher's prediction uses classifier-free
  guidance with its own scale per modality.
* Section 4: the residual-scale normaliser c^m = mean over the modality's
  latent elements of |x0^m - x0_T^m|, the normalised direction
  g^m / (c^m + eps_DMD), the residual Delta^m = x0^m - sg(x0^m - gbar^m), and
  the loss summed (not averaged) over latent elements and weighted by w_m.
* Section 4.1: L_stage3 = lam_sCM L_sCM + lam_DMD L_DMD.
* Section 7: guidance scales 3.0 (video) and 5.0 (audio); equal sCM and DMD
  weights.

Readings where the pages are silent:
* Guidance is the usual affine combination x0_u + s (x0_c - x0_u).  It is the
  same whether applied to x0-predictions, velocities or TrigFlow fields, since
  the weights 1 - s and s sum to one and those parameterisations are affine in
  one another at fixed (z, t).
* The unconditional (null-condition) teacher pass is the same block with every
  text key masked.
* The student's sample is an input; generating it is outside this term.
* eps_DMD defaults to 1e-6, like eps_sCM.
"""
from __future__ import annotations

import numpy as np

from .scm_oracle import block_x0, const, trigflow_noise


def guided(x_cond, x_uncond, scale):
    """Classifier-free guidance: x_u + s (x_c - x_u) ([deep read] section 4; the
    affine form is the standard one, the pages give only the per-modality scales)."""
    x_cond = np.asarray(x_cond, np.float64)
    x_uncond = np.asarray(x_uncond, np.float64)
    return x_uncond + scale * (x_cond - x_uncond)


def teacher_prediction(zv, za, t, text, mask, W, H, cfg_v, cfg_a, param="x0"):
    """The guided teacher x0-prediction for one sample at TrigFlow inputs
    (z, t): a conditional pass with the sample's text mask, an unconditional
    pass with every text key masked, combined with the per-modality scales.
    Returns (x0^v, x0^a, parts) where parts holds the two unguided passes."""
    cv, ca = block_x0(const(zv), const(za), const(t), text, mask, W, H, param)
    null_mask = np.zeros_like(np.asarray(mask))
    uv, ua = block_x0(const(zv), const(za), const(t), text, null_mask, W, H, param)
    parts = dict(cond_v=cv.p, cond_a=ca.p, uncond_v=uv.p, uncond_a=ua.p)
    return guided(cv.p, uv.p, cfg_v), guided(ca.p, ua.p, cfg_a), parts


def residual_scale(x0, x0_T):
    """c = (1/N) sum_i |x0_i - x0_T,i| over all N latent elements of one sample's
    modality ([deep read] section 4, the DMD normaliser)."""
    diff = np.abs(np.asarray(x0, np.float64) - np.asarray(x0_T, np.float64))
    return float(np.sum(diff)) / diff.size


def dmd_sample(cfg, data: dict, teacher: dict, fake: dict, b: int, cfg_v=None, cfg_a=None) -> dict:
    """The joint DMD term for sample ``b``: the guided teacher and fake-score
    predictions at the noised student sample, the direction, its residual-scale
    normalisation, the residual and the sum-reduced weighted loss."""
    cfg_v = cfg.cfg_v if cfg_v is None else cfg_v
    cfg_a = cfg.cfg_a if cfg_a is None else cfg_a
    t = float(data["t"][b])
    text, mask = data["text"][b], data["text_mask"][b]
    x0 = {"v": np.asarray(data["x0_v"][b], np.float64), "a": np.asarray(data["x0_a"][b], np.float64)}
    z_t = {m: trigflow_noise(t, x0[m], data[f"eps_{m}"][b]) for m in "va"}
    param = getattr(cfg, "param", "x0")

    tv, ta, parts = teacher_prediction(z_t["v"], z_t["a"], t, text, mask, teacher, cfg.H, cfg_v, cfg_a,
                                       param)
    fv, fa = block_x0(const(z_t["v"]), const(z_t["a"]), const(t), text, mask, fake, cfg.H, param)
    x0_T = {"v": tv, "a": ta}
    x0_F = {"v": fv.p, "a": fa.p}

    out = dict(t=t, z_t=z_t, x0_T=x0_T, x0_F=x0_F, parts=parts)
    loss = 0.0
    scales = []
    for m, w in (("v", cfg.w_v), ("a", cfg.w_a)):
        g = x0_F[m] - x0_T[m]                          # fake minus teacher prediction
        c = residual_scale(x0[m], x0_T[m])
        gbar = g / (c + cfg.eps_dmd)
        delta = x0[m] - (x0[m] - gbar)                 # x0 - sg(x0 - gbar), in value
        out[f"g_{m}"] = g
        out[f"gbar_{m}"] = gbar
        out[f"delta_{m}"] = delta
        scales.append(c)
        loss += w * float(np.sum(np.square(delta)))     # summed over latent elements
    out["scales"] = np.array(scales)
    out["loss"] = loss
    return out


def dmd_target(problem: dict, cfg_v=None, cfg_a=None) -> dict:
    """The joint DMD term for a whole batch; arrays stacked over the batch."""
    cfg, data = problem["cfg"], problem["data"]
    per = [dmd_sample(cfg, data, problem["teacher"], problem["fake"], b, cfg_v, cfg_a)
           for b in range(cfg.B)]
    res = {}
    for key in ("g_v", "g_a", "gbar_v", "gbar_a", "delta_v", "delta_a"):
        res[key] = np.stack([p[key] for p in per])
    for key in ("z_t", "x0_T", "x0_F"):
        for m in "va":
            res[f"{key}_{m}"] = np.stack([p[key][m] for p in per])
    res["scales"] = np.stack([p["scales"] for p in per])
    res["loss"] = np.array([p["loss"] for p in per])
    res["t"] = np.array([p["t"] for p in per])
    return res


def stage3_loss(loss_scm, loss_dmd, lam_scm, lam_dmd):
    """L_stage3 = lam_sCM L_sCM + lam_DMD L_DMD ([deep read] section 4.1), per sample."""
    return lam_scm * np.asarray(loss_scm, np.float64) + lam_dmd * np.asarray(loss_dmd, np.float64)
