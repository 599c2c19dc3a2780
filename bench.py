#!/usr/bin/env python3
"""Throughput of the joint sCM target on one MI355X.

One step = one call of t2va_scm_target over one batch of synthetic input
already resident in HBM: TrigFlow noising, the teacher block, teacher fields,
the student block with its forward-mode JVP, the sCM direction, per-sample
per-modality L2 normalisation, residual and loss.  The default workload is the
high-resolution shape (B=1, 28,672 video + 256 audio + 256 text tokens with
102 valid, d=2048, 16 heads of 128).

Prints one JSON line.  The roofline object covers the dominant kernel, the
student attention forward+JVP, timed with HIP events recorded by the library
around each of its launches on the launch stream during the timed steps (the
only events those steps carry; the per-phase breakdown comes from a second
window of as many steps with every phase recorded).  One
launch is two dispatches at this shape: the attention kernel and the small
kernel that merges the key-range pieces of the split tail tiles; the time,
the flops and the counted traffic all cover both.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sCM-target samples/s + attn fwd+JVP TFLOP/s (% MFMA bf16 peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def workload_name(cfg) -> str:
    storage = "bf16 storage" if cfg.precision == "bf16" else "bf16 storage, split-bf16 logit path"
    return (f"{cfg.name} joint sCM target: B={cfg.B}, video {cfg.Nv}x{cfg.Cv}, audio {cfg.Na}x{cfg.Ca}, "
            f"text {cfg.Nt} ({cfg.Ntv} valid), d={cfg.d}, {cfg.H}x{cfg.dh} heads, {storage}, "
            f"teacher + student fwd+JVP")


def attention_kernel_digest() -> str:
    """SHA-256 of the source text the attention kernel is compiled from:
    attention.hip, its tile helpers (attn_tiles.h), the shared types and
    load/store helpers at the top of common.h, and the AttnParams declaration
    (the other kernels' coefficient tables and parameter blocks do not
    count)."""
    import hashlib
    csrc = os.path.join(ROOT, "joint_video_audio_trigflow_amd", "csrc")
    common = open(os.path.join(csrc, "common.h")).read()
    head = common[:common.index("// Per-sample coefficients")]
    a = common.index("struct AttnParams")
    params = common[a:common.index("};", a) + 2]
    attn = open(os.path.join(csrc, "attention.hip")).read()
    tiles = open(os.path.join(csrc, "attn_tiles.h")).read()
    return hashlib.sha256((attn + tiles + head + params).encode()).hexdigest()


def counted_traffic(cfg):
    """HBM bytes per launch of the student attention (its kernel and the
    combine kernel of the split tail), from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE runs (copy-calibrated), or None if those counters
    were taken on another workload or on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_jvp_high_res_counters.json")
    if cfg.name != "high-res" or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if attention_kernel_digest() != rec["kernel_source_digest"]:
        return None
    return rec["traffic_bytes_per_launch"]


def attention_flops(cfg, nk_per_sample) -> float:
    """Algorithmic flops of one student attention fwd+JVP launch: 12 d Nq Nk per sample."""
    return float(sum(12.0 * cfg.d * cfg.Nq * nk for nk in nk_per_sample))


def cpu_baseline(cfg, budget_s: float) -> dict:
    """Time the fp64 oracle on a bounded sample of the workload and extrapolate.

    The oracle runs every block through dual numbers (teacher with zero
    tangents), so its cost is two blocks of: the QKV projection of every token
    and, per head, the chunked dual attention of every query row over all
    valid keys.  We time whole 512-row chunks of both on operands of the real
    shapes and scale linearly in rows and heads.
    """
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    dh, d = cfg.dh, cfg.d
    nk = cfg.Nq + cfg.Ntv
    chunk = 512
    mk = lambda *s: oracle.Dual(rng.standard_normal(s), rng.standard_normal(s))
    K, V = mk(nk, dh), mk(nk, dh)
    Q = mk(chunk, dh)
    X = mk(chunk, d)
    W = rng.standard_normal((3 * d, d)) / math.sqrt(d)
    n_att = n_proj = 0
    t_att = t_proj = 0.0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.attention(Q, K, V, chunk=chunk)
        t_att += time.perf_counter() - t0
        n_att += 1
        t0 = time.perf_counter()
        oracle.scm_oracle.d_linear(X, W)
        t_proj += time.perf_counter() - t0
        n_proj += 1
        if time.perf_counter() - t_start > budget_s:
            break
    per_att = t_att / n_att
    per_proj = t_proj / n_proj
    q_chunks = math.ceil(cfg.Nq / chunk)
    proj_chunks = math.ceil(cfg.N_all / chunk)
    per_sample = 2 * (cfg.H * q_chunks * per_att + proj_chunks * per_proj)
    return {
        "value": 1.0 / per_sample, "unit": "samples/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"{n_att} x oracle.attention (fp64 dual) of {chunk} query rows x {nk} keys x dh {dh}, "
                   f"{n_proj} x dual QKV projection of {chunk} rows ({d}->{3 * d}); extrapolated to "
                   f"2 blocks x {cfg.H} heads x {q_chunks} query chunks + {proj_chunks} projection "
                   f"chunks per sample ({per_sample:.0f} s/sample)"),
    }


def profiled_window(call, steps):
    """Per-phase times of `steps` more calls with every phase's events, after
    the timed calls (which carry only the events they read): the breakdown
    reported beside the timed figures."""
    import torch
    from joint_video_audio_trigflow_amd import _lib
    _lib.profile_set_phases(None)
    _lib.profile_enable(steps)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    phases, n = _lib.profile_read()
    _lib.profile_enable(0)
    return phases, n


def time_dmd(cfg, problem, steps, scm_ms) -> dict:
    """The joint DMD term (guided teacher: conditional + null-condition passes,
    fake-score block, residual-scale normaliser) on the same workload, timed
    after the sCM steps; the stage-3 step is one sCM target plus one DMD term."""
    import torch
    from joint_video_audio_trigflow_amd import _lib, inputs
    dp = inputs.make_dmd_problem(cfg, data=problem["data"])
    dev = _lib.to_device_dmd_problem(dp)
    dt = _lib.DTYPE_BF16 if cfg.in_dtype == "bf16" else _lib.DTYPE_FP32
    op = _lib.DmdTarget(cfg, in_dtype=dt, weight_dtype=dt)
    call = lambda: op(dev["teacher"], dev["fake"], dev["x0_v"], dev["x0_a"], dev["eps_v"],
                      dev["eps_a"], dev["text"], dev["text_mask"], dev["t"])
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    phases, n = profiled_window(call, steps)
    ms = 1000.0 * elapsed / steps
    return {"steps": steps, "ms_per_call": ms, "samples_per_s": cfg.B / (ms * 1e-3),
            "guidance": [cfg.cfg_v, cfg.cfg_a],
            "phases_ms_per_call": {"total": phases["total"] / n, "fwd_attention": phases["teacher_attn"] / n,
                                   "gemm": phases["gemm"] / n, "other": phases["other"] / n},
            "stage3_ms_per_step": scm_ms + ms}


def time_grad(cfg, problem, dev, steps, nk) -> dict:
    """The sCM target plus the training backward of its loss (gradients of all
    student weights), timed after the sCM steps on the same resident inputs."""
    import torch
    from joint_video_audio_trigflow_amd import _lib
    dt = _lib.DTYPE_BF16 if cfg.in_dtype == "bf16" else _lib.DTYPE_FP32
    # the backward is built for bf16 precision (it recomputes the softmax from bf16 Q and K)
    op = _lib.ScmGrad(cfg.replace(precision="bf16"), in_dtype=dt, weight_dtype=dt)
    call = lambda: op(dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"],
                      dev["eps_a"], dev["text"], dev["text_mask"], dev["t"])
    call()
    torch.cuda.synchronize()
    # the timed calls record only the attention backward's events
    _lib.profile_set_phases(["bwd_attn"])
    _lib.profile_enable(steps)
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed, n_timed = _lib.profile_read()
    _lib.profile_enable(0)
    _lib.profile_set_phases(None)
    phases, n = profiled_window(call, steps)
    ms = 1000.0 * elapsed / steps
    bwd_ms = timed["bwd_attn"] / n_timed
    # algorithmic attention-backward work: 2.5x the forward's 4 d Nq nk (dP, dV, dQ, dK and
    # recomputing S); the two kernels also recompute dP, 14 d Nq nk in all
    flops = sum(10.0 * cfg.d * cfg.Nq * k for k in nk)
    return {"steps": steps, "ms_per_call": ms, "samples_per_s": cfg.B / (ms * 1e-3), "precision": "bf16",
            "phases_ms_per_call": {k: v / n for k, v in phases.items()},
            "attn_bwd_tflops": flops / (bwd_ms * 1e-3) / 1e12,
            "attn_bwd_flops_per_launch": flops}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="high-res")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dmd-steps", type=int, default=5,
                    help="also time the joint DMD term on the same workload (0: skip)")
    ap.add_argument("--grad-steps", type=int, default=5,
                    help="also time the target plus its training backward (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from joint_video_audio_trigflow_amd import _lib, inputs

    if args.copy_calibration:
        n = args.copy_calibration * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": args.steps}), flush=True)
        return 0

    _lib.load()
    cfg = inputs.CONFIGS[args.config]
    problem = inputs.make_problem(cfg)
    dev = _lib.to_device_problem(problem)
    dt = _lib.DTYPE_BF16 if cfg.in_dtype == "bf16" else _lib.DTYPE_FP32
    op = _lib.ScmTarget(cfg, in_dtype=dt, weight_dtype=dt)
    call = lambda: op(dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"],
                      dev["eps_a"], dev["text"], dev["text_mask"], dev["t"])
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: warmup done", file=sys.stderr, flush=True)

    # The timed steps record only the student attention's events (the
    # roofline's kernel time: HIP events on the stream the library launches
    # on); every other phase's events would add device time to the steps.
    _lib.profile_set_phases(["student_attn"])
    _lib.profile_enable(args.steps)
    # one event between steps on the launch stream (torch's current stream,
    # which the binding passes to the library): per-step times for the median
    # and min
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        call()
        marks[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    timed, ncalls = _lib.profile_read()
    _lib.profile_enable(0)
    assert ncalls == args.steps, (ncalls, args.steps)
    phases, nphase = profiled_window(call, args.steps)
    loss = op.out["loss"].cpu().numpy()
    if not np.all(np.isfinite(loss)):
        raise RuntimeError(f"non-finite loss {loss}")

    ms_step = 1000.0 * elapsed / args.steps
    nk = [cfg.Nq + int(m.sum()) for m in problem["data"]["text_mask"]]
    flops = attention_flops(cfg, nk)
    attn_ms = timed["student_attn"] / ncalls
    achieved = flops / (attn_ms * 1e-3) / 1e12
    teacher_ms = phases["teacher_attn"] / nphase
    teacher_tf = flops / 3.0 / (teacher_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": cfg.B * args.steps / elapsed,
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": step_ms[len(step_ms) // 2] if len(step_ms) % 2 else
        0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2]),
        "ms_per_step_min": step_ms[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents/noise/text, N(0,1/fan_in) weights)",
        "config": {"workload": workload_name(cfg), "global_batch": cfg.B,
                   "tokens": cfg.N_all, "valid_keys": nk, "precision": cfg.precision,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": counted_traffic(cfg),
                     "kernel": f"attn_fwd_jvp_kernel<{cfg.dh},true> + attn_combine_kernel<{cfg.dh},true>",
                     "flops_per_launch": flops,
                     "avg_launch_ms": attn_ms},
        "phases_ms_per_step": {k: v / nphase for k, v in phases.items()},
        "teacher_attn_tflops": teacher_tf,
    }
    if args.dmd_steps > 0:
        rec["dmd_target"] = time_dmd(cfg, problem, args.dmd_steps, ms_step)
    if args.grad_steps > 0:
        rec["scm_grad"] = time_grad(cfg, problem, dev, args.grad_steps, nk)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
