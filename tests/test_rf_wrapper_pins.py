"""Pins of the oracle's TrigFlow -> rectified-flow wrapper (the block as a
velocity model behind the wrapper), independent of the oracle's own code paths.

* closed-form values of the input map and its derivative at t = pi/4, where
  cos t = sin t;
* the wrapper is consistent with both noising processes: TrigFlow's
  z = cos t x0 + sin t eps maps to rectified flow's (1 - t_rf) x0 + t_rf eps,
  so a block that returns the true velocity eps - x0 yields x0 exactly;
* for the exact velocity field of a single data point x0,
  v(z_rf, t_rf) = (z_rf - x0)/t_rf, the wrapped x0-prediction is the constant
  x0, so its JVP through the wrapper must vanish (every chain-rule term of the
  wrapper cancels);
* the joint JVP J of the wrapped student against central finite differences;
* a planted mistake in the wrapper's time derivative fails the FD pin.
"""
import math

import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs

Dual = oracle.Dual


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


TINY_RF = inputs.CONFIGS["tiny"].replace(param="rf")


def test_input_map_at_quarter_pi():
    rng = np.random.default_rng(3)
    z, zd = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
    z_rf, t_rf = oracle.rf_wrap(Dual(z, zd), Dual(np.float64(math.pi / 4), np.float64(1.0)))
    r2 = math.sqrt(2.0)
    assert np.max(np.abs(z_rf.p - z / r2)) < 1e-15
    # d/dt 1/(cos t + sin t) = (sin t - cos t)/(cos t + sin t)^2 = 0 at pi/4
    assert np.max(np.abs(z_rf.t - zd / r2)) < 1e-15
    assert abs(t_rf.p - 0.5) < 1e-15
    # d/dt sin t/(cos t + sin t) = 1/(cos t + sin t)^2 = 1/2 at pi/4
    assert abs(t_rf.t - 0.5) < 1e-15


@pytest.mark.parametrize("t", [0.03, 0.4, 1.1, 1.55])
def test_true_velocity_recovers_x0(t):
    rng = np.random.default_rng(4)
    x0 = {m: rng.standard_normal((8, 16)) for m in "va"}
    eps = {m: rng.standard_normal((8, 16)) for m in "va"}
    z = {m: math.cos(t) * x0[m] + math.sin(t) * eps[m] for m in "va"}

    def stub(zv, za, t_rf, text, mask, W, H, query_rows=None):
        # the rectified-flow noising of the same pair, and its velocity
        for zz, m in ((zv, "v"), (za, "a")):
            assert np.max(np.abs(zz.p - ((1 - t_rf.p) * x0[m] + t_rf.p * eps[m]))) < 1e-13
        return tuple(oracle.scm_oracle.const(eps[m] - x0[m]) for m in "va")

    xv, xa = oracle.block_x0(oracle.scm_oracle.const(z["v"]), oracle.scm_oracle.const(z["a"]),
                             oracle.scm_oracle.const(t), None, None, None, 1, "rf", block=stub)
    assert np.max(np.abs(xv.p - x0["v"])) < 1e-13 and np.max(np.abs(xa.p - x0["a"])) < 1e-13


@pytest.mark.parametrize("t", [0.05, 0.7, 1.5])
def test_point_mass_velocity_has_zero_jvp(t):
    rng = np.random.default_rng(5)
    x0 = {m: rng.standard_normal((8, 16)) for m in "va"}
    z = {m: rng.standard_normal((8, 16)) for m in "va"}
    zd = {m: rng.standard_normal((8, 16)) for m in "va"}

    def point_mass(zv, za, t_rf, text, mask, W, H, query_rows=None):
        # v(z_rf, t_rf) = (z_rf - x0)/t_rf, the exact velocity when all data is x0
        return tuple(oracle.scm_oracle.d_div(oracle.scm_oracle.d_sub(zz, oracle.scm_oracle.const(x0[m])), t_rf)
                     for zz, m in ((zv, "v"), (za, "a")))

    out = oracle.block_x0(Dual(z["v"], zd["v"]), Dual(z["a"], zd["a"]), Dual(np.float64(t), np.float64(1.0)),
                          None, None, None, 1, "rf", block=point_mass)
    for o, m in zip(out, "va"):
        assert np.max(np.abs(o.p - x0[m])) < 1e-12
        assert np.max(np.abs(o.t)) < 1e-11


@pytest.fixture(scope="module")
def tiny_rf():
    return inputs.make_problem(TINY_RF)


def _fd_gap(problem, t_override=None):
    cfg, data = problem["cfg"], dict(problem["data"])
    if t_override is not None:
        data["t"] = np.array([t_override])
    res = oracle.scm_sample(cfg, data, problem["teacher"], problem["student"], 0)
    t = res["t"]
    zv, za = res["z_t"]["v"], res["z_t"]["a"]
    h = 1e-6
    fp = oracle.student_field(cfg, data, problem["student"], 0, zv + h * res["F_T"]["v"],
                              za + h * res["F_T"]["a"], t + h)
    fm = oracle.student_field(cfg, data, problem["student"], 0, zv - h * res["F_T"]["v"],
                              za - h * res["F_T"]["a"], t - h)
    ct_st = math.cos(t) * math.sin(t)
    return [rel_l2(res[f"J_{m}"], ct_st * (fp[i] - fm[i]) / (2 * h)) for i, m in enumerate("va")], res


@pytest.mark.parametrize("t_override", [None, 0.06, 1.5])
def test_wrapped_jvp_matches_central_differences(tiny_rf, t_override):
    gaps, res = _fd_gap(tiny_rf, t_override)
    assert max(gaps) <= 1e-6, gaps
    # the wrapper changes the result (else the pins above would not reach the target)
    plain = oracle.scm_sample(inputs.CONFIGS["tiny"], tiny_rf["data"] if t_override is None else
                              dict(tiny_rf["data"], t=np.array([t_override])),
                              tiny_rf["teacher"], tiny_rf["student"], 0)
    assert rel_l2(res["J_v"], plain["J_v"]) > 1e-2


def test_fd_catches_a_wrong_wrapper_time_derivative(tiny_rf):
    orig = oracle.scm_oracle.rf_wrap

    def wrong(z, t):   # t_rf's derivative taken as if t_rf = t
        z_rf, t_rf = orig(z, t)
        return z_rf, Dual(t_rf.p, t.t)

    oracle.scm_oracle.rf_wrap = wrong
    try:
        res = oracle.scm_sample(TINY_RF, tiny_rf["data"], tiny_rf["teacher"], tiny_rf["student"], 0)
    finally:
        oracle.scm_oracle.rf_wrap = orig
    gaps_ok, _ = _fd_gap(tiny_rf)
    t = res["t"]
    zv, za = res["z_t"]["v"], res["z_t"]["a"]
    h = 1e-6
    fp = oracle.student_field(TINY_RF, tiny_rf["data"], tiny_rf["student"], 0, zv + h * res["F_T"]["v"],
                              za + h * res["F_T"]["a"], t + h)
    fm = oracle.student_field(TINY_RF, tiny_rf["data"], tiny_rf["student"], 0, zv - h * res["F_T"]["v"],
                              za - h * res["F_T"]["a"], t - h)
    fd = math.cos(t) * math.sin(t) * (fp[0] - fm[0]) / (2 * h)
    assert rel_l2(res["J_v"], fd) > 1e-4 and max(gaps_ok) <= 1e-6


def test_wrapped_dmd_term_runs_the_wrapper_on_every_block():
    """DMD with the wrapper: the teacher's conditional pass equals the sCM
    teacher's x0-prediction through the wrapper at the same inputs."""
    p = inputs.make_problem(TINY_RF)
    d = p["data"]
    dmd_data = dict(x0_v=d["z0_v"], x0_a=d["z0_a"], eps_v=d["eps_v"], eps_a=d["eps_a"], t=d["t"],
                    text=d["text"], text_mask=d["text_mask"])
    r = oracle.dmd_sample(TINY_RF, dmd_data, p["teacher"], p["student"], 0, cfg_v=1.0, cfg_a=1.0)
    s = oracle.scm_sample(TINY_RF, d, p["teacher"], p["student"], 0)
    for m in "va":
        assert rel_l2(r["x0_T"][m], s["x0_T"][m]) < 1e-14
