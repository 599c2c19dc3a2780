"""The targets (and the training backward) under HIP graph capture.

The library allocates nothing, copies nothing between host and device and
never synchronises inside a call: a call is a fixed sequence of kernel
launches on the caller's stream, whose per-sample coefficients (from the host
t) travel as kernel arguments.  So a caller can capture a call into a HIP
graph and replay it; the replay computes the captured call (the same t,
pointers and shapes).  Each replay here follows eager work of the program's
own (the outputs are overwritten with NaN, an unrelated product runs, the
device synchronises) and must reproduce the eager result bit for bit.  The
replay time is printed beside the eager time (measured equal for these
shapes: the host issues the launches ahead of the device, so a call is bound
by its kernels and their dependencies, not by launch cost).
"""
import time

import numpy as np
import pytest

from joint_video_audio_trigflow_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


def lib():
    from joint_video_audio_trigflow_amd import _lib
    _lib.load()
    return _lib


def snapshot(out):
    return {k: v.clone() for k, v in out.items() if v is not None}


def disturb(out):
    """Eager work between replays: outputs to NaN and an unrelated product."""
    for v in out.values():
        if v is not None:
            v.fill_(float("nan"))
    a = torch.randn(256, 256, device="cuda")
    (a @ a).sum().item()
    torch.cuda.synchronize()


def check_replays(name, call, out):
    call()                                   # eager: first-call set-up happens here, outside capture
    torch.cuda.synchronize()
    ref = snapshot(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(REPLAYS):
        disturb(out)
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), (name, rep, k)
    # replay against eager time (informational)
    times = {}
    for label, fn in (("eager", call), ("graph", g.replay)):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        times[label] = (time.perf_counter() - t0) / 20 * 1e3
    print(f"{name}: eager {times['eager']:.3f} ms, graph replay {times['graph']:.3f} ms", flush=True)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_scm_target_graph_replay(name):
    L = lib()
    print(f"graph capture: scm_target {name}", flush=True)
    cfg = inputs.CONFIGS[name]
    p = inputs.make_problem(cfg)
    dev = L.to_device_problem(p)
    dt = L.DTYPE_BF16 if cfg.in_dtype == "bf16" else L.DTYPE_FP32
    op = L.ScmTarget(cfg, in_dtype=dt, weight_dtype=dt)
    args = (dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"], dev["text"],
            dev["text_mask"], dev["t"])
    check_replays(f"scm_target {name}", lambda: op(*args), op.out)
    if name != "tiny":
        return
    # and the replayed result is the oracle's (the tolerance of the parity tests)
    import oracle
    ref = oracle.scm_target(p)
    for m in "va":
        for b in range(cfg.B):
            got = op.out[f"J_{m}"][b].cpu().numpy().astype(np.float64)
            e = np.linalg.norm(got - ref[f"J_{m}"][b]) / np.linalg.norm(ref[f"J_{m}"][b])
            assert e <= 2e-2, (name, m, b, e)


def test_dmd_target_graph_replay():
    L = lib()
    print("graph capture: dmd_target small (guided teacher)", flush=True)
    cfg = inputs.CONFIGS["small"]
    p = inputs.make_dmd_problem(cfg)
    dev = L.to_device_dmd_problem(p)
    op = L.DmdTarget(cfg)
    args = (dev["teacher"], dev["fake"], dev["x0_v"], dev["x0_a"], dev["eps_v"], dev["eps_a"], dev["text"],
            dev["text_mask"], dev["t"])
    check_replays("dmd_target small", lambda: op(*args), op.out)


def test_scm_grad_graph_replay():
    """The training backward is a fixed launch sequence too (the target, the
    attention backward with its split tails, the weight-gradient GEMMs and
    their fixed-order split-K sums): a replay reproduces the gradients."""
    L = lib()
    print("graph capture: scm_grad small", flush=True)
    cfg = inputs.CONFIGS["small"]
    p = inputs.make_problem(cfg)
    dev = L.to_device_problem(p)
    op = L.ScmGrad(cfg)
    args = (dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"], dev["text"],
            dev["text_mask"], dev["t"])
    check_replays("scm_grad small", lambda: op(*args), dict(op.out, **op.grads))


def test_noalloc_entry_graph_replay():
    """The allocation-free entry point is for such callers: its scratch is the
    library's static device array, so the captured call needs no workspace."""
    L = lib()
    print("graph capture: scm_target_noalloc small", flush=True)
    cfg = inputs.CONFIGS["small"]
    p = inputs.make_problem(cfg)
    dev = L.to_device_problem(p)
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {"J_v": torch.empty((cfg.B, cfg.Nv, cfg.Cv), **f32), "J_a": torch.empty((cfg.B, cfg.Na, cfg.Ca), **f32),
           "gbar_v": torch.empty((cfg.B, cfg.Nv, cfg.Cv), **f32), "gbar_a": torch.empty((cfg.B, cfg.Na, cfg.Ca), **f32),
           "r_v": None, "r_a": None, "norms": torch.empty((cfg.B, 2), **f32), "loss": torch.empty((cfg.B,), **f32)}
    args = (dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"], dev["eps_a"], dev["text"],
            dev["text_mask"], dev["t"])
    check_replays("scm_target_noalloc small", lambda: L.scm_target_noalloc(cfg, *args, out=out), out)
