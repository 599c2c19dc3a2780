"""Pins of the fp64 DMD / guidance / stage-3 oracle against what the pages and
the mathematics fix, independent of the oracle's own code paths.

* the residual-scale normaliser against its definition on tiny inputs, by
  plain loops, and against special cases that tell a mean of absolute values
  from a sum, an L2 norm or an RMS;
* the guidance reductions (scale 1 = conditional pass, scale 0 = the
  null-condition pass) and the null condition against a block that has no
  text at all;
* an independent implementation of the block with torch's fp64
  scaled_dot_product_attention and a boolean key mask (the oracle removes the
  padded keys instead);
* token duplication: attention is invariant under duplicating every key, so a
  sample whose tokens are all duplicated has the same normaliser and twice the
  loss when the loss is summed over latent elements (a mean would not change);
* the sign of the direction: a descent step on the student's sample moves it
  from the fake-score prediction towards the teacher's;
* fake block = teacher block with unit guidance gives a zero direction;
* the stage-3 mix reductions.
"""
import math

import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module")
def tiny_dmd():
    return inputs.make_dmd_problem(inputs.CONFIGS["tiny"])


@pytest.fixture(scope="module")
def tiny_dmd_result(tiny_dmd):
    return oracle.dmd_sample(tiny_dmd["cfg"], tiny_dmd["data"], tiny_dmd["teacher"], tiny_dmd["fake"], 0)


def test_residual_scale_by_loops_and_special_cases():
    rng = np.random.default_rng(7)
    a, b = rng.standard_normal((5, 3)), rng.standard_normal((5, 3))
    total, count = 0.0, 0
    for i in range(5):
        for j in range(3):
            total += abs(a[i, j] - b[i, j])
            count += 1
    assert abs(oracle.residual_scale(a, b) - total / count) < 1e-15
    # a constant difference delta gives |delta| (a sum would give N |delta|)
    x = rng.standard_normal((4, 8))
    assert abs(oracle.residual_scale(x, x - 0.75) - 0.75) < 1e-15
    # one non-zero difference among N gives |delta|/N (an L2 norm or an RMS would not)
    y = x.copy()
    y[2, 5] += 3.0
    assert abs(oracle.residual_scale(x, y) - 3.0 / 32) < 1e-15


def test_guidance_reductions(tiny_dmd):
    cfg, data = tiny_dmd["cfg"], tiny_dmd["data"]
    z = {m: data[f"x0_{m}"][0] for m in "va"}
    t = float(data["t"][0])
    args = (z["v"], z["a"], t, data["text"][0], data["text_mask"][0], tiny_dmd["teacher"], cfg.H)
    v1, a1, parts = oracle.teacher_prediction(*args, 1.0, 0.0)
    close = lambda a, b: np.max(np.abs(a - b)) < 1e-13
    assert close(v1, parts["cond_v"]) and close(a1, parts["uncond_a"])
    v0, a0, _ = oracle.teacher_prediction(*args, 0.0, 1.0)
    assert close(v0, parts["uncond_v"]) and close(a0, parts["cond_a"])
    # the guided prediction is affine in the scale: three scales on one line
    v3, _, _ = oracle.teacher_prediction(*args, 3.0, 1.0)
    v5, _, _ = oracle.teacher_prediction(*args, 5.0, 1.0)
    assert np.max(np.abs((v5 - v3) - (v3 - v1))) < 1e-12
    # conditioning matters in this block (else every guidance test is void)
    assert rel_l2(parts["cond_v"], parts["uncond_v"]) > 1e-3


def test_null_condition_equals_a_block_without_text(tiny_dmd):
    cfg, data = tiny_dmd["cfg"], tiny_dmd["data"]
    z = {m: data[f"x0_{m}"][0] for m in "va"}
    t = float(data["t"][0])
    _, _, parts = oracle.teacher_prediction(z["v"], z["a"], t, data["text"][0], data["text_mask"][0],
                                            tiny_dmd["teacher"], cfg.H, 3.0, 5.0)
    no_text = np.zeros((0, cfg.d))
    gv, ga = oracle.joint_block(oracle.scm_oracle.const(z["v"]), oracle.scm_oracle.const(z["a"]),
                                oracle.scm_oracle.const(t), no_text, np.zeros(0, np.uint8),
                                tiny_dmd["teacher"], cfg.H)
    assert np.array_equal(parts["uncond_v"], gv.p) and np.array_equal(parts["uncond_a"], ga.p)


def _torch_block(zv, za, t, text, mask, W, H):
    """The synthetic joint block written with torch fp64 library routines and a
    boolean key mask (padded and, for the null condition, all text keys masked)."""
    torch = pytest.importorskip("torch")
    T = lambda a: torch.as_tensor(np.asarray(a, np.float64))
    d = W["w_t"].shape[0]
    half = d // 2
    omega = 10000.0 ** (-torch.arange(half, dtype=torch.float64) / half)
    e = torch.cat([torch.cos(t * omega), torch.sin(t * omega)])
    tau = T(W["w_t"]) @ e
    hv = T(zv) @ T(W["w_in_v"]).T + tau
    ha = T(za) @ T(W["w_in_a"]).T + tau
    X = torch.cat([hv, ha, T(text)])
    Nq, N = hv.shape[0] + ha.shape[0], X.shape[0]
    wq, wk, wv = T(W["w_qkv"]).split(d)
    heads = lambda y: y.reshape(y.shape[0], H, d // H).transpose(0, 1).contiguous()
    q, k, v = heads(X[:Nq] @ wq.T), heads(X @ wk.T), heads(X @ wv.T)
    keep = torch.ones(N, dtype=torch.bool)
    keep[Nq:] = torch.as_tensor(np.asarray(mask) != 0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=keep[None, None, :])
    Y = o.transpose(0, 1).reshape(Nq, d)
    Nv = hv.shape[0]
    return (Y[:Nv] @ T(W["w_out_v"]).T).numpy(), (Y[Nv:] @ T(W["w_out_a"]).T).numpy()


def test_dmd_term_against_independent_torch_block(tiny_dmd, tiny_dmd_result):
    cfg, data = tiny_dmd["cfg"], tiny_dmd["data"]
    t = float(data["t"][0])
    text, mask = data["text"][0], data["text_mask"][0]
    zt = {m: math.cos(t) * data[f"x0_{m}"][0] + math.sin(t) * data[f"eps_{m}"][0] for m in "va"}
    cv, ca = _torch_block(zt["v"], zt["a"], t, text, mask, tiny_dmd["teacher"], cfg.H)
    uv, ua = _torch_block(zt["v"], zt["a"], t, text, np.zeros_like(mask), tiny_dmd["teacher"], cfg.H)
    fv, fa = _torch_block(zt["v"], zt["a"], t, text, mask, tiny_dmd["fake"], cfg.H)
    teach = {"v": uv + cfg.cfg_v * (cv - uv), "a": ua + cfg.cfg_a * (ca - ua)}
    fake = {"v": fv, "a": fa}
    loss = 0.0
    for i, (m, w) in enumerate((("v", cfg.w_v), ("a", cfg.w_a))):
        c = np.mean(np.abs(data[f"x0_{m}"][0] - teach[m]))
        gbar = (fake[m] - teach[m]) / (c + cfg.eps_dmd)
        assert abs(tiny_dmd_result["scales"][i] - c) < 1e-12 * c
        assert rel_l2(tiny_dmd_result[f"x0_T"][m], teach[m]) < 1e-12
        assert rel_l2(tiny_dmd_result[f"delta_{m}"], gbar) < 1e-12
        loss += w * np.sum(gbar ** 2)
    assert abs(tiny_dmd_result["loss"] - loss) < 1e-11 * loss


def test_token_duplication_keeps_the_scale_and_doubles_the_summed_loss(tiny_dmd, tiny_dmd_result):
    cfg, data = tiny_dmd["cfg"], tiny_dmd["data"]
    dup = {}
    for key in ("x0_v", "x0_a", "eps_v", "eps_a", "text", "text_mask"):
        x = data[key][:1]
        dup[key] = np.concatenate([x, x], axis=1)
    dup["t"] = data["t"][:1]
    cfg2 = cfg.replace(Nv=2 * cfg.Nv, Na=2 * cfg.Na, Nt=2 * cfg.Nt, Ntv=2 * cfg.Ntv)
    r2 = oracle.dmd_sample(cfg2, dup, tiny_dmd["teacher"], tiny_dmd["fake"], 0)
    assert np.max(np.abs(r2["scales"] - tiny_dmd_result["scales"])) < 1e-12
    assert abs(r2["loss"] - 2.0 * tiny_dmd_result["loss"]) < 1e-10 * tiny_dmd_result["loss"]
    for m in "va":
        n = tiny_dmd_result[f"delta_{m}"].shape[0]
        assert rel_l2(r2[f"delta_{m}"][:n], tiny_dmd_result[f"delta_{m}"]) < 1e-12
        assert rel_l2(r2[f"delta_{m}"][n:], tiny_dmd_result[f"delta_{m}"]) < 1e-12


def test_descent_moves_the_sample_from_fake_towards_teacher(tiny_dmd_result):
    torch = pytest.importorskip("torch")
    # loss as printed, with sg as detach; its gradient in the student's sample
    for m in "va":
        x0 = torch.zeros(tiny_dmd_result[f"gbar_{m}"].shape, dtype=torch.float64, requires_grad=True)
        gbar = torch.as_tensor(tiny_dmd_result[f"gbar_{m}"])
        delta = x0 - (x0 - gbar).detach()
        (delta ** 2).sum().backward()
        step = -x0.grad.numpy()
        towards_teacher = tiny_dmd_result["x0_T"][m] - tiny_dmd_result["x0_F"][m]
        cos = np.sum(step * towards_teacher) / (np.linalg.norm(step) * np.linalg.norm(towards_teacher))
        assert cos > 0.999


def test_fake_equal_to_teacher_with_unit_guidance_gives_zero(tiny_dmd):
    cfg, data = tiny_dmd["cfg"], tiny_dmd["data"]
    r = oracle.dmd_sample(cfg, data, tiny_dmd["teacher"], tiny_dmd["teacher"], 0, cfg_v=1.0, cfg_a=1.0)
    # u + 1 (c - u) equals c up to one rounding
    assert r["loss"] < 1e-25
    for m in "va":
        assert np.max(np.abs(r[f"g_{m}"])) < 1e-14
    assert np.all(r["scales"] > 0)


def test_teacher_prediction_matches_the_scm_teacher_at_unit_guidance():
    cfg = inputs.CONFIGS["tiny"]
    p = inputs.make_problem(cfg)
    d = p["data"]
    dmd_data = dict(x0_v=d["z0_v"], x0_a=d["z0_a"], eps_v=d["eps_v"], eps_a=d["eps_a"], t=d["t"],
                    text=d["text"], text_mask=d["text_mask"])
    r = oracle.dmd_sample(cfg, dmd_data, p["teacher"], p["student"], 0, cfg_v=1.0, cfg_a=1.0)
    s = oracle.scm_sample(cfg, d, p["teacher"], p["student"], 0)
    for m in "va":
        assert rel_l2(r["x0_T"][m], s["x0_T"][m]) < 1e-14
        assert rel_l2(r["x0_F"][m], s["x0_S_" + m]) < 1e-14


def test_stage3_mix_reductions():
    a, b = np.array([1.5, 2.0]), np.array([7.0, -1.0])
    assert np.array_equal(oracle.stage3_loss(a, b, 1.0, 0.0), a)
    assert np.array_equal(oracle.stage3_loss(a, b, 0.0, 1.0), b)
    assert np.allclose(oracle.stage3_loss(a, b, 1.0, 1.0), [8.5, 1.0], rtol=0, atol=0)
