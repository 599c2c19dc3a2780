"""GPU parity over a seeded sweep of workload shapes, against the fp64 oracle.

The fixed test cases pin the named workloads and the edge cases; this sweep
draws 12 more shapes from one seeded generator so that the boundaries the
kernels tile by (16/32/64-token blocks, 192-row attention workgroups, 256-row
GEMM tiles, the 64-key stages of the attention rings) fall at many different
places: batch 1-3, one to four heads of 64 or 128, 1-400 video and 1-200 audio
tokens, 0-40 text positions with a random valid subset (prefix or scattered),
both channel widths, both block parameterisations (x0 or the rectified-flow
wrapper), beta in [0.5, 2] and gamma in [0, 1].  Two further shapes use
d = 1024 and about 2,000 tokens, which takes the projections through the
large-tile GEMM (row-major and V^T outputs, ragged row counts), and two small
ones fit their keys into a single 64-key stage.

Each shape runs the sCM target; every second one also the DMD term and every
third one the training backward.  Tolerances are those of the fixed cases:
J, gbar and Delta within 2e-2 relative L2 per (sample, modality), the sCM loss
within 1e-3, the DMD loss within 2e + e^2, weight gradients within 2e-2
relative L2 (bf16 storage, fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_FIELD = 2e-2
TOL_LOSS_SCM = 1e-3
TOL_LOSS_DMD = 2 * TOL_FIELD + TOL_FIELD ** 2
WEIGHTS = ("w_in_v", "w_in_a", "w_t", "w_qkv", "w_out_v", "w_out_a")


def _sweep():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(12):
        H = int(rng.choice([1, 2, 4]))
        dh = int(rng.choice([64, 128]))
        Nt = int(rng.integers(0, 41))
        out.append(inputs.Config(
            f"sweep{i:02d}", B=int(rng.integers(1, 4)), Nv=int(rng.integers(1, 401)),
            Na=int(rng.integers(1, 201)), Nt=Nt, Ntv=int(rng.integers(0, Nt + 1)),
            Cv=int(rng.choice([64, 128])), Ca=int(rng.choice([64, 128])), d=H * dh, H=H,
            in_dtype="bf16", beta=float(rng.uniform(0.5, 2.0)), gamma=float(rng.uniform(0.0, 1.0)),
            w_v=float(rng.uniform(0.5, 2.0)), w_a=float(rng.uniform(0.5, 2.0)),
            mask_mode=str(rng.choice(["prefix", "scatter"])), param=str(rng.choice(["x0", "rf"])),
            index=40 + i))
    for i in range(2):
        Nt = int(rng.integers(8, 65))
        out.append(inputs.Config(
            f"sweep-large{i}", B=1, Nv=int(rng.integers(1800, 2300)), Na=int(rng.integers(60, 260)),
            Nt=Nt, Ntv=int(rng.integers(1, Nt + 1)), Cv=128, Ca=64, d=1024, H=8, in_dtype="bf16",
            beta=1.0, gamma=float(rng.uniform(0.0, 1.0)), mask_mode="scatter",
            param=("x0", "rf")[i], index=60 + i))
    # and two shapes whose keys fit one 64-key stage (one of them exactly)
    out.append(inputs.Config("sweep-small0", B=2, Nv=23, Na=9, Nt=6, Ntv=4, Cv=64, Ca=64, d=256, H=2,
                             in_dtype="bf16", beta=1.5, gamma=0.3, mask_mode="scatter", param="rf", index=70))
    out.append(inputs.Config("sweep-small1", B=1, Nv=40, Na=24, Nt=0, Ntv=0, Cv=64, Ca=128, d=128, H=2,
                             in_dtype="bf16", beta=0.8, gamma=0.9, index=71))
    return out


SWEEP = _sweep()


def lib():
    from joint_video_audio_trigflow_amd import _lib
    _lib.load()
    return _lib


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def say(*a):
    print(*a, flush=True)


def dtype_of(L, cfg):
    return L.DTYPE_BF16 if cfg.in_dtype == "bf16" else L.DTYPE_FP32


def describe(cfg):
    return (f"{cfg.name}: B={cfg.B} Nv={cfg.Nv} Na={cfg.Na} Nt={cfg.Nt} (valid {cfg.Ntv}, {cfg.mask_mode}) "
            f"C={cfg.Cv}/{cfg.Ca} d={cfg.d} H={cfg.H} param={cfg.param} beta={cfg.beta:.2f} gamma={cfg.gamma:.2f}")


@pytest.mark.parametrize("k", range(len(SWEEP)), ids=lambda k: SWEEP[k].name)
def test_sweep_against_oracle(k):
    cfg = SWEEP[k]
    L = lib()
    say(describe(cfg))
    dt = dtype_of(L, cfg)

    # the sCM target
    p = inputs.make_problem(cfg)
    dev = L.to_device_problem(p)
    args = (dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"],
            dev["text"], dev["text_mask"], dev["t"])
    got = L.ScmTarget(cfg, in_dtype=dt, weight_dtype=dt)(*args)
    torch.cuda.synchronize()
    got = {key: (None if v is None else v.cpu().numpy()) for key, v in got.items()}
    ref = oracle.scm_target(p)
    worst = 0.0
    for b in range(cfg.B):
        for m in "va":
            for key in ("J", "gbar"):
                e = rel_l2(got[f"{key}_{m}"][b], ref[f"{key}_{m}"][b])
                worst = max(worst, e)
                assert e <= TOL_FIELD, (cfg.name, "scm", b, m, key, e)
        assert abs(got["loss"][b] - ref["loss"][b]) <= TOL_LOSS_SCM * abs(ref["loss"][b]), (cfg.name, b)
    say(f"  sCM target worst rel-L2 {worst:.2e}")

    # the training backward
    if k % 3 == 0:
        _, grads = L.ScmGrad(cfg, in_dtype=dt, weight_dtype=dt)(*args)
        torch.cuda.synchronize()
        gref = oracle.scm_loss_and_grads(p, ref)
        errs = {w: rel_l2(grads[w].cpu().numpy(), gref[w]) for w in WEIGHTS}
        say("  backward rel-L2:", {w: f"{e:.1e}" for w, e in errs.items()})
        for w, e in errs.items():
            assert e <= TOL_FIELD, (cfg.name, "grad", w, e)

    # the DMD term with the guided teacher
    if k % 2 == 0:
        q = inputs.make_dmd_problem(cfg)
        dq = L.to_device_dmd_problem(q)
        out = L.DmdTarget(cfg, in_dtype=dt, weight_dtype=dt)(
            dq["teacher"], dq["fake"], dq["x0_v"], dq["x0_a"], dq["eps_v"], dq["eps_a"],
            dq["text"], dq["text_mask"], dq["t"])
        torch.cuda.synchronize()
        out = {key: v.cpu().numpy() for key, v in out.items()}
        dref = oracle.dmd_target(q)
        worst = 0.0
        for b in range(cfg.B):
            for i, m in enumerate("va"):
                e = rel_l2(out[f"delta_{m}"][b], dref[f"delta_{m}"][b])
                worst = max(worst, e)
                assert e <= TOL_FIELD, (cfg.name, "dmd", b, m, e)
                assert abs(out["scales"][b, i] - dref["scales"][b, i]) <= TOL_FIELD * dref["scales"][b, i]
            assert abs(out["loss"][b] - dref["loss"][b]) <= TOL_LOSS_DMD * dref["loss"][b], (cfg.name, b)
        say(f"  DMD term worst rel-L2 {worst:.2e}")


def test_sweep_covers_the_tile_boundaries():
    """The sweep is meant to straddle the kernels' block sizes: check that it
    does (on the host, so a change of seed cannot silently shrink it)."""
    nq = [c.Nq for c in SWEEP]
    assert any(n % 16 for n in nq) and any(n < 192 for n in nq) and any(n > 192 for n in nq)
    nk = [c.Nq + c.Ntv for c in SWEEP]
    assert any(n % 64 and n > 64 for n in nk) and any(n <= 64 for n in nk)
    assert {c.param for c in SWEEP} == {"x0", "rf"} and {c.d // c.H for c in SWEEP} == {64, 128}
    assert any(c.d >= 1024 and c.N_all >= 2048 and c.N_all % 256 for c in SWEEP)
