"""Pins for the fp64 oracle, against what the pages and the mathematics fix.

Each test ties one part of the oracle to something other than itself:
finite differences of its own primal for the JVP, closed forms of special
cases, identities implied by the normalisation and loss definitions, and an
independent library implementation (torch's fp64 attention with torch.func.jvp).
Citations refer to the robotworld.top deep read of TurboT2VA (arXiv 2608.24674),
section 3.1 unless noted.
"""
import math

import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs

TINY = inputs.CONFIGS["tiny"]


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module")
def tiny_problem():
    return inputs.make_problem(TINY)


@pytest.fixture(scope="module")
def tiny_result(tiny_problem):
    return oracle.scm_target(tiny_problem)


# ---------------------------------------------------------------------------
# E1 / E3: noising and fields
# ---------------------------------------------------------------------------
def test_noise_special_cases():
    rng = np.random.default_rng(0)
    z0 = rng.standard_normal((5, 7))
    eps = rng.standard_normal((5, 7))
    t = 0.7
    assert np.array_equal(oracle.trigflow_noise(t, z0, np.zeros_like(eps)), math.cos(t) * z0)
    assert np.array_equal(oracle.trigflow_noise(t, np.zeros_like(z0), eps), math.sin(t) * eps)
    # cos^2 + sin^2 = 1: unit-variance inputs keep unit variance in expectation;
    # exactly, |z_t|^2 = c^2|z0|^2 + s^2|eps|^2 + 2cs<z0,eps>
    zt = oracle.trigflow_noise(t, z0, eps)
    c, s = math.cos(t), math.sin(t)
    lhs = float(np.sum(zt * zt))
    rhs = c * c * np.sum(z0 * z0) + s * s * np.sum(eps * eps) + 2 * c * s * np.sum(z0 * eps)
    assert abs(lhs - rhs) <= 1e-12 * abs(rhs)


@pytest.mark.parametrize("t", [0.01, 0.3, 0.785, 1.2, math.pi / 2 - 0.01])
def test_field_identity_when_prediction_is_clean(t):
    """If x0_hat = z0 then F = cos t eps - sin t z0 exactly (E1 substituted into E3)."""
    rng = np.random.default_rng(1)
    z0 = rng.standard_normal((64, 16))
    eps = rng.standard_normal((64, 16))
    zt = oracle.trigflow_noise(t, z0, eps)
    F = oracle.trigflow_field(t, zt, z0)
    expect = math.cos(t) * eps - math.sin(t) * z0
    assert np.max(np.abs(F - expect)) <= 1e-13 / math.sin(t)


# ---------------------------------------------------------------------------
# E4: the joint JVP against central finite differences of the primal field
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("t_override", [None, 0.06, 1.5])
def test_jvp_matches_central_differences(tiny_problem, t_override):
    cfg, data = tiny_problem["cfg"], dict(tiny_problem["data"])
    if t_override is not None:
        data["t"] = np.array([t_override])
    res = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0)
    t = res["t"]
    zv, za = res["z_t"]["v"], res["z_t"]["a"]
    FTv, FTa = res["F_T"]["v"], res["F_T"]["a"]
    h = 1e-6
    fp = oracle.student_field(cfg, data, tiny_problem["student"], 0, zv + h * FTv, za + h * FTa, t + h)
    fm = oracle.student_field(cfg, data, tiny_problem["student"], 0, zv - h * FTv, za - h * FTa, t - h)
    ct_st = math.cos(t) * math.sin(t)
    for i, m in enumerate("va"):
        fd = ct_st * (fp[i] - fm[i]) / (2 * h)
        assert rel_l2(res[f"J_{m}"], fd) <= 1e-6, (m, rel_l2(res[f"J_{m}"], fd))


def test_fd_catches_a_planted_mistake(tiny_problem):
    """Dropping the time-embedding tangent (a plausible mistake) must fail the FD pin."""
    cfg, data = tiny_problem["cfg"], tiny_problem["data"]
    orig = oracle.scm_oracle.time_embedding

    def no_tangent(t, d):
        e = orig(t, d)
        return oracle.Dual(e.p, np.zeros_like(e.t))

    oracle.scm_oracle.time_embedding = no_tangent
    try:
        res = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0)
    finally:
        oracle.scm_oracle.time_embedding = orig
    t = res["t"]
    zv, za = res["z_t"]["v"], res["z_t"]["a"]
    h = 1e-6
    fp = oracle.student_field(cfg, data, tiny_problem["student"], 0, zv + h * res["F_T"]["v"],
                              za + h * res["F_T"]["a"], t + h)
    fm = oracle.student_field(cfg, data, tiny_problem["student"], 0, zv - h * res["F_T"]["v"],
                              za - h * res["F_T"]["a"], t - h)
    fd = math.cos(t) * math.sin(t) * (fp[0] - fm[0]) / (2 * h)
    assert rel_l2(res["J_v"], fd) > 1e-4


# ---------------------------------------------------------------------------
# E5: the sCM direction
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("t", [0.02, 0.5, 1.0, 1.55])
def test_boost_factor_reductions(t):
    # gamma = 1: cos t / sqrt(1 - sin^2 t) = cos t / |cos t| = 1 on (0, pi/2)
    assert abs(oracle.boost_factor(t, 1.0, 1.0) - 1.0) < 1e-12
    assert abs(oracle.boost_factor(t, 2.5, 1.0) - 2.5) < 1e-12
    # gamma = 0: the factor is beta cos t
    assert abs(oracle.boost_factor(t, 2.0, 0.0) - 2.0 * math.cos(t)) < 1e-15


def test_teacher_equals_student_gamma_one(tiny_problem):
    """theta = T and gamma = 1: g = cos t * dG, whatever beta (derived from E3-E5)."""
    p = dict(tiny_problem)
    p["student"] = p["teacher"]
    for beta in (1.0, 3.0):
        r = oracle.scm_sample(p["cfg"], p["data"], p["teacher"], p["teacher"], 0, beta=beta, gamma=1.0)
        for m in "va":
            expect = math.cos(r["t"]) * r[f"Gdot_{m}"]
            assert rel_l2(r[f"g_{m}"], expect) <= 1e-12


@pytest.mark.parametrize("gamma", [0.0, 1.0])
def test_beta_enters_linearly_with_the_printed_factor(tiny_problem, gamma):
    """g(beta2) - g(beta1) = (beta2 - beta1) f(t, gamma) (x0_S - x0_T)/sin t with
    f(t, 1) = 1 and f(t, 0) = cos t."""
    cfg, data = tiny_problem["cfg"], tiny_problem["data"]
    r1 = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0, beta=1.0, gamma=gamma)
    r2 = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0, beta=2.0, gamma=gamma)
    t = r1["t"]
    f = 1.0 if gamma == 1.0 else math.cos(t)
    for m in "va":
        expect = f * (r1[f"x0_S_{m}"] - r1["x0_T"][m]) / math.sin(t)
        assert rel_l2(r2[f"g_{m}"] - r1[f"g_{m}"], expect) <= 1e-10


def test_gamma_term_sign(tiny_problem):
    """With beta = 0 the only gamma dependence is -gamma cos t sin t z_t."""
    cfg, data = tiny_problem["cfg"], tiny_problem["data"]
    r0 = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0, beta=0.0, gamma=0.0)
    r1 = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0, beta=0.0, gamma=1.0)
    t = r0["t"]
    for m in "va":
        expect = -math.cos(t) * math.sin(t) * r0["z_t"][m]
        assert rel_l2(r1[f"g_{m}"] - r0[f"g_{m}"], expect) <= 1e-12


# ---------------------------------------------------------------------------
# E6-E8: normalisation, residual, loss
# ---------------------------------------------------------------------------
def test_norm_bound_and_loss_identity(tiny_result):
    cfg = TINY
    for b in range(cfg.B):
        L = 0.0
        for i, (m, w) in enumerate((("v", cfg.w_v), ("a", cfg.w_a))):
            n = tiny_result["norms"][b, i]
            gbar = tiny_result[f"gbar_{m}"][b]
            assert abs(n - np.linalg.norm(tiny_result[f"g_{m}"][b])) <= 1e-12 * n
            ng = np.linalg.norm(gbar)
            assert ng < 1.0
            assert abs(ng - n / (n + cfg.eps_scm)) <= 1e-14
            assert np.array_equal(tiny_result[f"r_{m}"][b], -gbar)
            L += w * n * n / (n + cfg.eps_scm) ** 2
        assert abs(tiny_result["loss"][b] - L) <= 1e-13
        assert abs(tiny_result["loss"][b] - (cfg.w_v + cfg.w_a)) <= 1e-4


# ---------------------------------------------------------------------------
# Attention: softmax tangent, uniform-attention closed form, library cross-check
# ---------------------------------------------------------------------------
def test_softmax_tangent_rows_sum_to_zero():
    """With V = 1 and dV = 0, O = 1 and dO = sum_j dP_ij = 0."""
    rng = np.random.default_rng(3)
    q = oracle.Dual(rng.standard_normal((40, 16)), rng.standard_normal((40, 16)))
    k = oracle.Dual(rng.standard_normal((33, 16)) * 3, rng.standard_normal((33, 16)))
    v = oracle.Dual(np.ones((33, 16)), np.zeros((33, 16)))
    o = oracle.attention(q, k, v, chunk=7)
    assert np.max(np.abs(o.p - 1)) < 1e-14
    assert np.max(np.abs(o.t)) < 1e-13


def test_attention_matches_torch_jvp():
    torch = pytest.importorskip("torch")
    from torch.func import jvp
    rng = np.random.default_rng(4)
    B, Nq, Nk, H, dh = 2, 37, 45, 3, 16
    ops = {n: rng.standard_normal((B, Nq if n.startswith("q") else Nk, H, dh))
           for n in ("q", "k", "v", "qd", "kd", "vd")}
    nk = np.array([45, 30], dtype=np.int32)
    o, od, lse = oracle.attention_fwd_jvp(ops["q"], ops["k"], ops["v"], ops["qd"], ops["kd"], ops["vd"], nk)
    for b in range(B):
        n = nk[b]
        T = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))  # [H, N, dh]

        def f(q, k, v):
            return torch.nn.functional.scaled_dot_product_attention(q, k, v)

        prim = (T(ops["q"][b]), T(ops["k"][b, :n]), T(ops["v"][b, :n]))
        tang = (T(ops["qd"][b]), T(ops["kd"][b, :n]), T(ops["vd"][b, :n]))
        out, tout = jvp(f, prim, tang)
        assert np.max(np.abs(out.numpy().transpose(1, 0, 2) - o[b])) < 1e-12
        assert np.max(np.abs(tout.numpy().transpose(1, 0, 2) - od[b])) < 1e-12
        s = torch.einsum("hqd,hkd->hqk", prim[0], prim[1]) / math.sqrt(dh)
        assert np.max(np.abs(torch.logsumexp(s, -1).numpy() - lse[b])) < 1e-12


def _embedding_and_derivative(t, d):
    half = d // 2
    w = 10000.0 ** (-np.arange(half) / half)
    e = np.concatenate([np.cos(w * t), np.sin(w * t)])
    de = np.concatenate([-w * np.sin(w * t), w * np.cos(w * t)])
    return e, de


def test_uniform_attention_closed_form(tiny_problem):
    """W_q = W_k = 0 makes every logit 0: each query averages V over the valid keys.

    Then x0_hat^m_i = mean_j(X_j) W_v^T W_out^m^T for every row i, and its
    tangent averages dX_j = F_T,j W_in^T + de W_t^T (text rows: 0).  J follows
    from differentiating E3: J = -c_t z_t + cos^2 t (F_T - F_S) - cos t dG.
    """
    cfg, data = tiny_problem["cfg"], tiny_problem["data"]
    W = {k: v.copy() for k, v in tiny_problem["student"].items()}
    d = cfg.d
    W["w_qkv"][: 2 * d] = 0.0
    r = oracle.scm_sample(cfg, data, tiny_problem["teacher"], W, 0)
    t = r["t"]
    e, de = _embedding_and_derivative(t, d)
    tau, dtau = W["w_t"] @ e, W["w_t"] @ de
    zv, za = r["z_t"]["v"], r["z_t"]["a"]
    Xv = zv @ W["w_in_v"].T + tau
    Xa = za @ W["w_in_a"].T + tau
    Xc = data["text"][0][data["text_mask"][0].astype(bool)]
    X = np.concatenate([Xv, Xa, Xc])
    dX = np.concatenate([r["F_T"]["v"] @ W["w_in_v"].T + dtau, r["F_T"]["a"] @ W["w_in_a"].T + dtau,
                         np.zeros_like(Xc)])
    wv = W["w_qkv"][2 * d:]
    ybar, dybar = X.mean(0) @ wv.T, dX.mean(0) @ wv.T
    c, s = math.cos(t), math.sin(t)
    for m, z, wo in (("v", zv, W["w_out_v"]), ("a", za, W["w_out_a"])):
        x0 = np.broadcast_to(ybar @ wo.T, z.shape)
        dG = np.broadcast_to(dybar @ wo.T, z.shape)
        F_S = (c * z - x0) / s
        J = -c * s * z + c * c * (r["F_T"][m] - F_S) - c * dG
        assert rel_l2(r[f"x0_S_{m}"], x0) < 1e-13
        assert rel_l2(r[f"Gdot_{m}"], dG) < 1e-12
        assert rel_l2(r[f"J_{m}"], J) < 1e-12


# ---------------------------------------------------------------------------
# Structural invariants of the joint block
# ---------------------------------------------------------------------------
def test_padded_text_values_do_not_matter():
    cfg = TINY.replace(Nt=12, Ntv=5, mask_mode="scatter")
    p = inputs.make_problem(cfg)
    r1 = oracle.scm_target(p)
    data2 = dict(p["data"])
    text2 = data2["text"].copy()
    text2[data2["text_mask"] == 0] = 123.0
    data2["text"] = text2
    r2 = oracle.scm_target(dict(p, data=data2))
    for key in ("J_v", "J_a", "gbar_v", "gbar_a", "loss"):
        assert np.array_equal(r1[key], r2[key])
    # and valid text does matter
    text3 = data2["text"].copy()
    text3[data2["text_mask"] == 1] += 0.5
    data2["text"] = text3
    r3 = oracle.scm_target(dict(p, data=data2))
    assert rel_l2(r3["J_v"], r1["J_v"]) > 1e-6


def test_video_permutation_equivariance(tiny_problem):
    p = tiny_problem
    r1 = oracle.scm_target(p)
    perm = np.random.default_rng(5).permutation(TINY.Nv)
    data2 = dict(p["data"])
    data2["z0_v"] = data2["z0_v"][:, perm]
    data2["eps_v"] = data2["eps_v"][:, perm]
    r2 = oracle.scm_target(dict(p, data=data2))
    assert rel_l2(r2["J_v"], r1["J_v"][:, perm]) < 1e-12
    assert rel_l2(r2["J_a"], r1["J_a"]) < 1e-12
    assert abs(r2["loss"][0] - r1["loss"][0]) < 1e-12


def test_batch_independence():
    cfg = TINY.replace(B=3, Nv=20, Na=6, Nt=5, Ntv=4, mask_mode="scatter", index=7)
    p = inputs.make_problem(cfg)
    r = oracle.scm_target(p)
    for b in range(cfg.B):
        one = {k: (v[b:b + 1] if isinstance(v, np.ndarray) else v) for k, v in p["data"].items()}
        r1 = oracle.scm_target(dict(p, cfg=cfg.replace(B=1), data=one))
        for key in ("J_v", "J_a", "gbar_a", "loss"):
            assert np.array_equal(r[key][b:b + 1], r1[key])


def test_video_tangent_depends_on_audio(tiny_problem):
    """The joint JVP couples modalities: changing audio latents changes J^v."""
    p = tiny_problem
    r1 = oracle.scm_target(p)
    data2 = dict(p["data"])
    data2["z0_a"] = data2["z0_a"] + 0.25
    r2 = oracle.scm_target(dict(p, data=data2))
    assert rel_l2(r2["J_v"], r1["J_v"]) > 1e-4


def test_storage_rounding_mode_is_a_small_perturbation(tiny_problem):
    """STORAGE = "bf16" only rounds stored intermediates: on a well-conditioned
    workload it moves J by about the bf16 unit roundoff, and the default mode is
    untouched by it."""
    from oracle import scm_oracle
    cfg, data = tiny_problem["cfg"], tiny_problem["data"]
    exact = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0)
    scm_oracle.STORAGE = "bf16"
    try:
        st = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0)
    finally:
        scm_oracle.STORAGE = None
    again = oracle.scm_sample(cfg, data, tiny_problem["teacher"], tiny_problem["student"], 0)
    for m in "va":
        e = rel_l2(st[f"J_{m}"], exact[f"J_{m}"])
        assert 1e-5 < e < 1e-2, (m, e)
        assert np.array_equal(again[f"J_{m}"], exact[f"J_{m}"])
    # the rounding helper is round-to-nearest-even bfloat16
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5])
    assert np.array_equal(scm_oracle._bf16(x), np.array([1.0, 1 + 2 * 2.0 ** -7, -2.5]))
