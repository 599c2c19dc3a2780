"""GPU parity of the attention tail split, against the fp64 oracle.

The attention kernels run one workgroup per compute unit at a time, so each
XCD (32 compute units on MI355X) runs its tiles in rounds.  When the last round
would be short, the last tiles of each XCD are cut into k pieces over
consecutive ranges of 64-key stages and merged by a second kernel (only in the
entry points that carry a workspace).  The rule: with per_xcd = ceil(tiles / 8)
and rem = per_xcd mod 32, k in 2..8 (2..4 for the backward kernels) minimises
ceil(rem k / 32) / k, and a
piece never spans fewer than 512 keys of the longest possible sample (the JVP
and backward kernels stage 64 keys at a time, the forward kernel 128).  The
shapes below are chosen to take each branch of that rule:

- split-empty: 4 tiles (per_xcd 1) and 2,088 key positions of which only the
  40 latent tokens and 2-3 text tokens are valid, so k = 4 and three of the
  four pieces of every tile are empty (they must get zero weight);
- split-k3 (dh 128) and split-k3-64 (dh 64): 1,664 queries over 8 heads give
  72 JVP tiles (per_xcd 9, k = 3) and 40 forward tiles (per_xcd 5, k = 3);
- split-k8: 1,536 queries over 2 heads and 2,600 valid text keys (4,136 keys)
  give 16 JVP tiles (per_xcd 2) and 8 forward tiles (per_xcd 1), each cut into
  k = 8 pieces of at least 512 keys (the dQ kernel's 12 tiles into k = 4);
- the large sweep shapes and the full-size test take k = 2, the full-size
  teacher forward k = 4.

Each case runs the sCM target, the training backward (which reads the merged
log-sum-exp) and the DMD term, with the tolerances of the fixed cases.
"""
import math

import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs

torch = pytest.importorskip("torch")

TOL_FIELD = 2e-2
TOL_LOSS_SCM = 1e-3
TOL_LOSS_DMD = 2 * TOL_FIELD + TOL_FIELD ** 2
WEIGHTS = ("w_in_v", "w_in_a", "w_t", "w_qkv", "w_out_v", "w_out_a")

SPLIT_EMPTY = inputs.Config("split-empty", B=2, Nv=30, Na=10, Nt=2048, Ntv=3, Cv=64, Ca=64, d=256, H=2,
                            in_dtype="bf16", beta=1.2, gamma=0.6, mask_mode="scatter", index=80)
SPLIT_K3 = inputs.Config("split-k3", B=1, Nv=1600, Na=64, Nt=64, Ntv=40, Cv=128, Ca=64, d=1024, H=8,
                         in_dtype="bf16", beta=1.0, gamma=0.8, mask_mode="scatter", index=81)
SPLIT_K3_64 = inputs.Config("split-k3-64", B=1, Nv=1600, Na=64, Nt=64, Ntv=64, Cv=64, Ca=128, d=512, H=8,
                            in_dtype="bf16", beta=0.9, gamma=0.4, param="rf", index=82)
SPLIT_K8 = inputs.Config("split-k8", B=1, Nv=1400, Na=136, Nt=2600, Ntv=2600, Cv=128, Ca=64, d=256, H=2,
                         in_dtype="bf16", beta=1.1, gamma=0.7, mask_mode="scatter", index=83)
CASES = [SPLIT_EMPTY, SPLIT_K3, SPLIT_K3_64, SPLIT_K8]


def planned_pieces(tiles, n_keys, stage, slots=32, max_k=8):
    """The split rule as documented above (k = 1: no split)."""
    per_xcd = (tiles + 7) // 8
    rem = per_xcd % slots
    if rem == 0:
        return 1
    nst_max = (n_keys + stage - 1) // stage
    best_k, best = 1, 1.0
    for k in range(2, max_k + 1):
        if nst_max // k < 512 // stage:
            break
        cost = math.ceil(rem * k / slots) / k
        if cost < best - 1e-12:
            best_k, best = k, cost
    return best_k


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


def test_split_cases_take_each_branch():
    """Host-side check that the shapes exercise k = 4 with empty pieces, k = 3 and k = 8."""
    def plan(cfg, rows):
        # JVP kernel: 192 rows, 64-key stages; forward kernel: 384 rows, 128-key stages
        tiles = cfg.B * cfg.H * ((cfg.Nq + rows - 1) // rows)
        return planned_pieces(tiles, cfg.N_all, 64 if rows == 192 else 128)
    assert plan(SPLIT_EMPTY, 192) == 4 and (SPLIT_EMPTY.Nq + SPLIT_EMPTY.Ntv + 63) // 64 < 4
    assert plan(SPLIT_K3, 192) == 3 and plan(SPLIT_K3, 384) == 3
    assert plan(SPLIT_K3_64, 192) == 3
    assert plan(SPLIT_K8, 192) == 8 and plan(SPLIT_K8, 384) == 8
    dq_tiles = SPLIT_K8.B * SPLIT_K8.H * ((SPLIT_K8.Nq + 255) // 256)   # dQ kernel: 256 queries per tile
    assert planned_pieces(dq_tiles, SPLIT_K8.N_all, 64, max_k=4) == 4
    hr = inputs.CONFIGS["high-res"]
    assert plan(hr, 192) == 2 and plan(hr, 384) == 4


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_split_tail_against_oracle(cfg):
    L = lib()
    say(f"{cfg.name}: B={cfg.B} Nq={cfg.Nq} N_all={cfg.N_all} d={cfg.d} H={cfg.H} param={cfg.param}")
    dt = L.DTYPE_BF16

    p = inputs.make_problem(cfg)
    dev = L.to_device_problem(p)
    args = (dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"],
            dev["text"], dev["text_mask"], dev["t"])
    got = L.ScmTarget(cfg, in_dtype=dt, weight_dtype=dt)(*args)
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.cpu().numpy()) for k, v in got.items()}
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

    _, grads = L.ScmGrad(cfg, in_dtype=dt, weight_dtype=dt)(*args)
    torch.cuda.synchronize()
    gref = oracle.scm_loss_and_grads(p, ref)
    errs = {w: rel_l2(grads[w].cpu().numpy(), gref[w]) for w in WEIGHTS}
    say("  backward rel-L2:", {w: f"{e:.1e}" for w, e in errs.items()})
    for w, e in errs.items():
        assert e <= TOL_FIELD, (cfg.name, "grad", w, e)

    q = inputs.make_dmd_problem(cfg)
    dq = L.to_device_dmd_problem(q)
    out = L.DmdTarget(cfg, in_dtype=dt, weight_dtype=dt)(
        dq["teacher"], dq["fake"], dq["x0_v"], dq["x0_a"], dq["eps_v"], dq["eps_a"],
        dq["text"], dq["text_mask"], dq["t"])
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
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
