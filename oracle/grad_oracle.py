"""fp64 CPU oracle for the training backward of the joint sCM loss.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path.

What it computes ("TurboT2VA：分数正则化一致性蒸馏加速 19B 视频音频联合生成",
robotworld.top deep read of arXiv 2608.24674, section 3.1: the residual
r = F_theta - sg(F_theta) - gbar and the joint loss sum_m w_m ||r^m||^2;
section 7 trains the student with AdamW on this loss):

* gbar is a constant target: every quantity inside it (the teacher, the JVP
  J, the norms) is under stop-gradient, so the gradient of the loss reaches
  the student's weights only through F_theta's own forward pass, with
  dL/dF_theta^m = 2 w_m r^m = -2 w_m gbar^m in value.
* The gradient is that of sum_b L_b (the batch scalar mean_b L_b is this
  divided by B).

It takes gbar from the sCM oracle, rebuilds the student's primal block in
plain torch float64 operations (the same synthetic block: per-modality input
projections plus the time-embedding linear layer, one joint attention over
video, audio and valid text tokens, per-modality output projections; the
TrigFlow wrapper when the block is a rectified-flow model), forms the loss
with sg as detach, and differentiates it with torch's reverse-mode autograd.
"""
from __future__ import annotations

import math

import numpy as np

from . import scm_oracle

WEIGHTS = ("w_in_v", "w_in_a", "w_t", "w_qkv", "w_out_v", "w_out_a")


def _torch():
    import torch
    return torch


def _attention_rows(q, k, v, dh):
    """softmax(q k^T / sqrt(dh)) v for a block of query rows (one head)."""
    torch = _torch()
    s = (q @ k.T) / math.sqrt(dh)
    return torch.softmax(s, dim=1) @ v


def student_x0_torch(zv, za, t, text, mask, W, H, param="x0", query_chunk=None):
    """The student's x0-predictions as a torch float64 graph of the weights
    ``W`` (dict of tensors); zv, za, text are float64 tensors, t a float.

    ``query_chunk``: evaluate each head's attention over blocks of that many
    query rows and let autograd recompute a block's logits and softmax in the
    backward pass instead of keeping them (torch.utils.checkpoint): the same
    arithmetic, with memory for one block of logits at a time, which the
    high-resolution workload needs (29k x 29k logits per head)."""
    torch = _torch()
    d = W["w_t"].shape[0]
    dh = d // H
    half = d // 2
    if param == "rf":
        cs = math.cos(t) + math.sin(t)
        zv, za, t_in = zv / cs, za / cs, math.sin(t) / cs
    else:
        t_in = t
    omega = 10000.0 ** (-torch.arange(half, dtype=torch.float64) / half)
    e = torch.cat([torch.cos(t_in * omega), torch.sin(t_in * omega)])
    tau = W["w_t"] @ e
    hv = zv @ W["w_in_v"].T + tau
    ha = za @ W["w_in_a"].T + tau
    hc = text[torch.as_tensor(np.asarray(mask) != 0)]
    X = torch.cat([hv, ha, hc])
    Nq = hv.shape[0] + ha.shape[0]
    w_q, w_k, w_v = W["w_qkv"][:d], W["w_qkv"][d:2 * d], W["w_qkv"][2 * d:]
    Q = X[:Nq] @ w_q.T
    K = X @ w_k.T
    V = X @ w_v.T
    outs = []
    for h in range(H):
        sl = slice(h * dh, (h + 1) * dh)
        if query_chunk is None:
            outs.append(_attention_rows(Q[:, sl], K[:, sl], V[:, sl], dh))
        else:
            from torch.utils.checkpoint import checkpoint
            blocks = [checkpoint(_attention_rows, Q[r0:r0 + query_chunk, sl], K[:, sl], V[:, sl], dh,
                                 use_reentrant=False)
                      for r0 in range(0, Nq, query_chunk)]
            outs.append(torch.cat(blocks, dim=0))
    Y = torch.cat(outs, dim=1)
    Nv = hv.shape[0]
    yv = Y[:Nv] @ W["w_out_v"].T
    ya = Y[Nv:] @ W["w_out_a"].T
    if param == "rf":
        return zv - t_in * yv, za - t_in * ya
    return yv, ya


def scm_loss_and_grads(problem: dict, scm_result: dict | None = None, query_chunk=None) -> dict:
    """sum_b L_b of the joint sCM loss with gbar held constant, and its
    gradient with respect to every student weight (float64 arrays shaped like
    the weights).  ``scm_result`` is the sCM oracle's output for the same
    problem (computed here when absent); ``query_chunk`` as in
    student_x0_torch."""
    torch = _torch()
    cfg, data = problem["cfg"], problem["data"]
    param = getattr(cfg, "param", "x0")
    res = scm_oracle.scm_target(problem) if scm_result is None else scm_result
    W = {k: torch.tensor(np.asarray(problem["student"][k], np.float64), requires_grad=True) for k in WEIGHTS}
    total = torch.zeros((), dtype=torch.float64)
    per_sample = []
    for b in range(cfg.B):
        t = float(data["t"][b])
        zt = {m: torch.tensor(res[f"z_t_{m}"][b]) for m in "va"}
        text = torch.tensor(np.asarray(data["text"][b], np.float64))
        xv, xa = student_x0_torch(zt["v"], zt["a"], t, text, data["text_mask"][b], W, cfg.H, param,
                                  query_chunk=query_chunk)
        Lb = torch.zeros((), dtype=torch.float64)
        for m, x0, w in (("v", xv, cfg.w_v), ("a", xa, cfg.w_a)):
            F = (math.cos(t) * zt[m] - x0) / math.sin(t)
            r = F - F.detach() - torch.tensor(res[f"gbar_{m}"][b])
            Lb = Lb + w * torch.sum(r * r)
        per_sample.append(float(Lb.detach()))
        total = total + Lb
    total.backward()
    out = {k: W[k].grad.numpy().copy() for k in WEIGHTS}
    out["loss_sum"] = float(total.detach())
    out["loss"] = np.array(per_sample)
    return out


def student_fields(problem: dict, student: dict) -> dict:
    """F_theta^m = (cos t z_t^m - x0^m)/sin t at the given student weights, per
    sample, in plain float64 (no autograd): {"v": [B, Nv, Cv], "a": [B, Na, Ca]}.
    Finite differences of sum_m w_m ||F(W) - F(W0) - gbar||^2 in W check the
    gradient, since that is the loss as a function of W around W0."""
    torch = _torch()
    cfg, data = problem["cfg"], problem["data"]
    param = getattr(cfg, "param", "x0")
    W = {k: torch.tensor(np.asarray(student[k], np.float64)) for k in WEIGHTS}
    out = {"v": [], "a": []}
    with torch.no_grad():
        for b in range(cfg.B):
            t = float(data["t"][b])
            zt = {m: torch.tensor(scm_oracle.trigflow_noise(t, data[f"z0_{m}"][b], data[f"eps_{m}"][b]))
                  for m in "va"}
            text = torch.tensor(np.asarray(data["text"][b], np.float64))
            xv, xa = student_x0_torch(zt["v"], zt["a"], t, text, data["text_mask"][b], W, cfg.H, param)
            for m, x0 in (("v", xv), ("a", xa)):
                out[m].append(((math.cos(t) * zt[m] - x0) / math.sin(t)).numpy())
    return {m: np.stack(v) for m, v in out.items()}
