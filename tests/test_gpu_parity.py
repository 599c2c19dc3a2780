"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: J and gbar within a max relative L2 error of 2e-2 per (sample,
modality) and the per-sample loss within 1e-3 relative (bf16 inputs, fp32
accumulation).  Kernel-level attention parity uses 1e-2 relative L2 per
(sample, head), derived from bf16 rounding of P and P*dS (unit roundoff 2^-9)
averaged over keys.
"""
import math

import numpy as np
import pytest

import oracle
from joint_video_audio_trigflow_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_FIELD = 2e-2
TOL_LOSS = 1e-3


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


# ---------------------------------------------------------------------------
# TrigFlow elementwise maps
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [0, 8, 1000, 4096 + 24, 123457])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_trigflow_noise_and_field(n, dt):
    L = lib()
    say(f"trigflow n={n} dt={dt}")
    rng = np.random.default_rng(n)
    B = 3
    a = inputs.round_to(rng.standard_normal((B, n)), dt)
    b = inputs.round_to(rng.standard_normal((B, n)), dt)
    t = [0.02, 0.9, math.pi / 2 - 0.02]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    A = torch.from_numpy(a.astype(np.float32)).to("cuda", tdt)
    Bt = torch.from_numpy(b.astype(np.float32)).to("cuda", tdt)
    z = L.trigflow_field(L.NOISE, A, Bt, t).cpu().numpy()
    f = L.trigflow_field(L.FIELD, A, Bt, t).cpu().numpy()
    torch.cuda.synchronize()
    for i in range(B):
        ez = oracle.trigflow_noise(t[i], a[i], b[i])
        ef = oracle.trigflow_field(t[i], a[i], b[i])
        if n:
            assert np.max(np.abs(z[i] - ez)) <= 1e-6 * (1 + np.max(np.abs(ez)))
            assert np.max(np.abs(f[i] - ef)) <= 1e-6 * (1 + np.max(np.abs(ef)))


# ---------------------------------------------------------------------------
# Attention forward + JVP
# ---------------------------------------------------------------------------
def run_attention(ops, H, dh, tangent=True, out_dtype=torch.float32, ldv_pad=0):
    L = lib()
    B, Nq = ops["q"].shape[:2]
    Nk = ops["k"].shape[1]
    ldv = (Nk + 63) // 64 * 64 + ldv_pad

    def dev(x):
        return torch.from_numpy(x.astype(np.float32)).to("cuda", torch.bfloat16).contiguous()

    def devT(x):  # [B, N, H, dh] -> [B, H, dh, ldv]
        vt = np.zeros((B, H, dh, ldv), np.float32)
        vt[..., :Nk] = x.transpose(0, 2, 3, 1)
        return torch.from_numpy(vt).to("cuda", torch.bfloat16).contiguous()

    q, k, vt = dev(ops["q"]), dev(ops["k"]), devT(ops["v"])
    nk = torch.from_numpy(ops["nk"]).to("cuda")
    if tangent:
        o, od, lse = L.joint_attn_fwd_jvp(q, k, vt, nk, dev(ops["qd"]), dev(ops["kd"]), devT(ops["vd"]),
                                          out_dtype=out_dtype, want_lse=True)
    else:
        o, od, lse = L.joint_attn_fwd_jvp(q, k, vt, nk, out_dtype=out_dtype, want_lse=True)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), None if od is None else od.float().cpu().numpy(),
            lse.cpu().numpy())


ATTN_CASES = [
    # B, H, dh, Nq, Nk, nk
    (1, 1, 128, 128, 64, [64]),
    (2, 2, 128, 200, 230, [230, 150]),      # ragged queries and keys, per-sample key counts
    (1, 3, 64, 333, 517, [500]),            # dh = 64, many tiles
    (2, 1, 128, 70, 75, [75, 71]),          # single partial tiles
    (1, 2, 128, 5, 9, [1]),                 # a single valid key
]


@pytest.mark.parametrize("case", ATTN_CASES)
@pytest.mark.parametrize("tangent", [True, False])
def test_attention_matches_oracle(case, tangent):
    B, H, dh, Nq, Nk, nk = case
    say(f"attention case={case} tangent={tangent}")
    ops = inputs.make_attention_operands(B, H, dh, Nq, Nk, seed=Nq + Nk, nk_valid=nk)
    o, od, lse = run_attention(ops, H, dh, tangent)
    eo, eod, else_ = oracle.attention_fwd_jvp(ops["q"], ops["k"], ops["v"], ops["qd"], ops["kd"],
                                              ops["vd"], ops["nk"])
    for b in range(B):
        for h in range(H):
            assert rel_l2(o[b, :, h], eo[b, :, h]) < 1e-2, (b, h)
            if tangent:
                assert rel_l2(od[b, :, h], eod[b, :, h]) < 1e-2, (b, h)
    assert np.max(np.abs(lse - else_)) < 2e-2


@pytest.mark.parametrize("qk_scale,tan_scale", [(10.0, 20.0), (4.0, 1.0)])
def test_attention_peaked_softmax(qk_scale, tan_scale):
    """Large logits make softmax nearly one-hot; with large tangents the JVP
    must not lose the small result to the subtraction mu * o."""
    B, H, dh, Nq, Nk = 1, 2, 128, 150, 700
    say(f"attention peaked qk_scale={qk_scale} tan_scale={tan_scale}")
    ops = inputs.make_attention_operands(B, H, dh, Nq, Nk, seed=13, nk_valid=[650], q_scale=qk_scale,
                                         k_scale=qk_scale, tangent_scale=tan_scale)
    o, od, lse = run_attention(ops, H, dh, True)
    eo, eod, else_ = oracle.attention_fwd_jvp(ops["q"], ops["k"], ops["v"], ops["qd"], ops["kd"],
                                              ops["vd"], ops["nk"])
    for h in range(H):
        assert rel_l2(o[0, :, h], eo[0, :, h]) < 1e-2, h
        assert rel_l2(od[0, :, h], eod[0, :, h]) < 1e-2, (h, rel_l2(od[0, :, h], eod[0, :, h]))


def test_attention_bf16_output_and_padding_garbage():
    """bf16 outputs; V^T columns past nk hold huge values that must not leak."""
    L = lib()
    B, H, dh, Nq, Nk = 1, 2, 128, 130, 100
    ops = inputs.make_attention_operands(B, H, dh, Nq, Nk, seed=11, nk_valid=[77])
    ops["v"][:, 77:] = 1e30
    ops["vd"][:, 77:] = -1e30
    ops["k"][:, 77:] = 1e3
    o, od, _ = run_attention(ops, H, dh, True, out_dtype=torch.bfloat16, ldv_pad=16)
    eo, eod, _ = oracle.attention_fwd_jvp(ops["q"], ops["k"], ops["v"], ops["qd"], ops["kd"], ops["vd"],
                                          ops["nk"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(od))
    assert rel_l2(o, eo) < 1e-2 and rel_l2(od, eod) < 1e-2


def test_attention_with_sequence_major_v_through_v_transpose():
    """A caller holding V (and dV) sequence-major, in place in a fused
    [B, N, 3 H dh] projection output, converts them with t2va_v_transpose:
    the result equals the dh-major path's bit for bit."""
    L = lib()
    B, H, dh, Nq, Nk = 2, 3, 64, 90, 131
    say("attention with sequence-major V via t2va_v_transpose")
    ops = inputs.make_attention_operands(B, H, dh, Nq, Nk, seed=17, nk_valid=[131, 100])
    fused = np.zeros((B, Nk, 3, H, dh), np.float32)
    fused[:, :, 2] = ops["v"]
    fz = torch.from_numpy(fused.reshape(B, Nk, 3 * H * dh)).to("cuda", torch.bfloat16)
    v_view = fz[:, :, 2 * H * dh:].view(B, Nk, H, dh)       # strided: row stride 3 H dh
    vt = L.v_transpose(v_view)
    vdt = L.v_transpose(torch.from_numpy(ops["vd"].astype(np.float32)).to("cuda", torch.bfloat16).contiguous())
    torch.cuda.synchronize()
    assert vt.shape == (B, H, dh, 192) and torch.all(vt[..., Nk:] == 0)

    def dev(x):
        return torch.from_numpy(x.astype(np.float32)).to("cuda", torch.bfloat16).contiguous()

    nk = torch.from_numpy(ops["nk"]).to("cuda")
    o1, od1, _ = L.joint_attn_fwd_jvp(dev(ops["q"]), dev(ops["k"]), vt, nk, dev(ops["qd"]), dev(ops["kd"]), vdt)
    o2, od2, _ = run_attention(ops, H, dh, True)
    assert np.array_equal(o1.cpu().numpy(), o2) and np.array_equal(od1.cpu().numpy(), od2)


def test_attention_softmax_tangent_with_constant_values():
    """V = 1, dV = 0 gives O = 1 and dO = 0 (rows of dP sum to zero)."""
    B, H, dh, Nq, Nk = 1, 1, 128, 64, 200
    ops = inputs.make_attention_operands(B, H, dh, Nq, Nk, seed=12)
    ops["v"][:] = 1.0
    ops["vd"][:] = 0.0
    o, od, _ = run_attention(ops, H, dh, True)
    assert np.max(np.abs(o - 1)) < 1e-2
    assert np.max(np.abs(od)) < 2e-2 * np.sqrt(np.mean(np.square(ops["qd"]))) * 3


# ---------------------------------------------------------------------------
# The full sCM target
# ---------------------------------------------------------------------------
RAGGED = inputs.Config("ragged", B=2, Nv=300, Na=45, Nt=20, Ntv=13, Cv=128, Ca=64, d=256, H=2,
                       in_dtype="bf16", beta=1.5, gamma=0.7, mask_mode="scatter", index=11)
RAGGED64 = inputs.Config("ragged64", B=1, Nv=130, Na=70, Nt=0, Ntv=0, Cv=64, Ca=64, d=256, H=4,
                         in_dtype="bf16", beta=1.0, gamma=1.0, index=12)


def run_scm(problem):
    L = lib()
    cfg = problem["cfg"]
    dev = L.to_device_problem(problem)
    dt = L.DTYPE_BF16 if cfg.in_dtype == "bf16" else L.DTYPE_FP32
    op = L.ScmTarget(cfg, in_dtype=dt, weight_dtype=dt)
    out = op(dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"],
             dev["text"], dev["text_mask"], dev["t"])
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def check_against_oracle(cfg, got, ref):
    worst = {}
    for b in range(cfg.B):
        for m in "va":
            for key in ("J", "gbar"):
                e = rel_l2(got[f"{key}_{m}"][b], ref[f"{key}_{m}"][b])
                worst[f"{key}_{m}"] = max(worst.get(f"{key}_{m}", 0.0), e)
                assert e <= TOL_FIELD, (cfg.name, b, m, key, e)
            assert np.array_equal(got[f"r_{m}"][b], -got[f"gbar_{m}"][b])
        assert abs(got["loss"][b] - ref["loss"][b]) <= TOL_LOSS * abs(ref["loss"][b])
        assert np.allclose(got["norms"][b], ref["norms"][b], rtol=TOL_FIELD)
    say(cfg.name, "worst rel-L2:", {k: f"{v:.2e}" for k, v in worst.items()})


@pytest.mark.parametrize("cfg", [inputs.CONFIGS["tiny"], RAGGED, RAGGED64], ids=lambda c: c.name)
def test_scm_target_matches_oracle(cfg):
    say(f"scm_target {cfg.name}")
    p = inputs.make_problem(cfg)
    got = run_scm(p)
    ref = oracle.scm_target(p)
    check_against_oracle(cfg, got, ref)


def test_scm_target_small_config():
    cfg = inputs.CONFIGS["small"]
    say("scm_target small")
    p = inputs.make_problem(cfg)
    got = run_scm(p)
    ref = oracle.scm_target(p)
    check_against_oracle(cfg, got, ref)


def test_scm_target_deterministic_and_mask_invariant():
    say("scm_target determinism / mask invariance")
    p = inputs.make_problem(RAGGED)
    a = run_scm(p)
    b = run_scm(p)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k
    data2 = dict(p["data"])
    text2 = data2["text"].copy()
    text2[data2["text_mask"] == 0] = 7.0
    data2["text"] = text2
    c = run_scm(dict(p, data=data2))
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], c[k]), k


def test_scm_target_batch_independence():
    say("scm_target batch independence")
    p = inputs.make_problem(RAGGED)
    full = run_scm(p)
    one = {k: (v[1:2] if isinstance(v, np.ndarray) else v) for k, v in p["data"].items()}
    single = run_scm(dict(p, cfg=RAGGED.replace(B=1), data=one))
    for k in ("J_v", "J_a", "gbar_v", "gbar_a", "loss"):
        assert np.array_equal(full[k][1:2], single[k]), k


# ---------------------------------------------------------------------------
# The block as a rectified-flow velocity model behind the TrigFlow wrapper
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [inputs.CONFIGS["tiny"].replace(param="rf"), RAGGED.replace(param="rf"),
                                 inputs.CONFIGS["small"].replace(param="rf")], ids=lambda c: c.name + "-rf")
def test_scm_target_rf_wrapper_matches_oracle(cfg):
    say(f"scm_target {cfg.name} through the TrigFlow wrapper")
    p = inputs.make_problem(cfg)
    got = run_scm(p)
    ref = oracle.scm_target(p)
    check_against_oracle(cfg, got, ref)


# ---------------------------------------------------------------------------
# Edge cases of the target: every text position padded, the largest batch the
# coefficient table holds, gamma = 0, and one token per modality.
# ---------------------------------------------------------------------------
ALLPAD = inputs.Config("allpad", B=2, Nv=96, Na=40, Nt=16, Ntv=0, Cv=64, Ca=64, d=256, H=2,
                       in_dtype="bf16", index=13)
MAXB = inputs.Config("maxbatch", B=64, Nv=64, Na=32, Nt=8, Ntv=5, Cv=64, Ca=64, d=128, H=2,
                     in_dtype="bf16", mask_mode="scatter", index=14)
GAMMA0 = inputs.Config("gamma0", B=2, Nv=100, Na=30, Nt=10, Ntv=7, Cv=128, Ca=64, d=256, H=4,
                       in_dtype="bf16", beta=0.5, gamma=0.0, index=15)
ONETOK = inputs.Config("onetoken", B=2, Nv=1, Na=1, Nt=3, Ntv=2, Cv=64, Ca=64, d=128, H=1,
                       in_dtype="bf16", index=16)


@pytest.mark.parametrize("cfg", [ALLPAD, MAXB, GAMMA0, ONETOK], ids=lambda c: c.name)
def test_scm_target_edge_cases(cfg):
    say(f"scm_target edge case {cfg.name}")
    p = inputs.make_problem(cfg)
    got = run_scm(p)
    ref = oracle.scm_target(p)
    check_against_oracle(cfg, got, ref)
