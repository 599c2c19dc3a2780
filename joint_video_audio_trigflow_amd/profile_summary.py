"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

Reads a --kernel-trace --stats directory and two --pmc runs (FETCH_SIZE,
WRITE_SIZE) of bench.py, plus the same counters for bench.py
--copy-calibration (a plain device-to-device copy of known size), and prints
a markdown summary with per-kernel average durations, counter values per
dispatch, the calibration factors, the resulting HBM traffic per launch and
the achieved HBM bandwidth (traffic over the traced average duration).
Usage: python -m joint_video_audio_trigflow_amd.profile_summary <rocprof output dir>

With --per-config <file>..., it reads bench.py's JSON lines (one per
workload) and prints one row per workload: samples/s, the step's mean,
median and min, the student attention's time and rate against the dense bf16
peak, the teacher attention's rate, and the DMD term's and the backward's
times when present.

With --counters-record <dir> <out.json>, after the summary above it writes the
record bench.py reads for the roofline's "traffic" field: the student
attention's counted bytes per launch (its kernel and its split-tail merge),
the calibration factors, the commands, and the digest of the attention
sources the counters were taken on.

With --clock <dir>, it reads one --pmc --kernel-trace run per subdirectory of
<dir> instead and prints, per attention and GEMM kernel, the average of each
counter per dispatch and these derived figures (MI355X: 8 XCDs, 256 CUs,
1024 SIMDs; GRBM_GUI_ACTIVE reads as the sum over the XCDs):
  clock      = GRBM_GUI_ACTIVE / 8 / kernel duration
  MFMA busy  = SQ_VALU_MFMA_BUSY_CYCLES / 1024 / (GRBM_GUI_ACTIVE / 8)
  LDS active = SQ_LDS_IDX_ACTIVE / 256 / (GRBM_GUI_ACTIVE / 8)
"""
from __future__ import annotations

import collections
import csv
import glob
import json
import os
import sys


def short(name: str) -> str:
    for key, label in (("attn_fwd_jvp_kernel<128, true, false>", "attn_fwd_jvp<128,true> (student fwd+JVP)"),
                       ("attn_fwd_jvp_kernel<128, false, false>", "attn_fwd_jvp<128,false> (forward: teacher, fake)"),
                       ("attn_fwd_jvp_kernel<128, true, true>", "attn_fwd_jvp<128,true,split> (student, split)"),
                       ("attn_fwd_jvp_kernel<128, false, true>", "attn_fwd_jvp<128,false,split> (forward, split)"),
                       ("attn_combine_kernel<128, true, false>", "attn_combine<128,true> (JVP split-tail merge)"),
                       ("attn_combine_kernel<128, false, false>", "attn_combine<128,false> (forward split-tail merge)"),
                       ("attn_combine_kernel<128, true, true>", "attn_combine<128,true,split> (JVP merge, split)"),
                       ("attn_combine_kernel<128, false, true>", "attn_combine<128,false,split> (forward merge, split)"),
                       ("attn_bwd_dkv_kernel<128>", "attn_bwd_dkv<128> (backward dK, dV)"),
                       ("attn_bwd_dq_kernel<128>", "attn_bwd_dq<128> (backward dQ)"),
                       ("attn_bwd_dkv_merge_kernel<128>", "attn_bwd_dkv_merge<128> (split-tail sum)"),
                       ("attn_bwd_dq_merge_kernel<128>", "attn_bwd_dq_merge<128> (split-tail sum)"),
                       ("gemm_bf16_large_kernel", "gemm_bf16_large (256x256 tiles)"),
                       ("gemm_bf16_kernel", "gemm_bf16 (128x128 tiles)"),
                       ("gemm_bf16_ring_kernel", "gemm_bf16_ring (128x128 tiles, long K)"),
                       ("copyBuffer", "copyBuffer"),
                       ("elementwise_kernel", "torch copy")):
        if key in name:
            return label
    for key in ("trigflow_kernel", "text_rows_kernel", "scm_direction_kernel", "normalise_kernel",
                "time_linear_kernel", "time_embedding_kernel", "cast_set_kernel", "dmd_direction_kernel",
                "transpose16_set_kernel", "transpose16_kernel", "transpose_kernel", "rowterm_kernel", "seed_kernel",
                "colsum_kernel", "time_grad_kernel", "reduce_splits_kernel", "zero_rows_kernel", "fill_nk_kernel",
                "mix_kernel", "guide_kernel", "dup_cols_kernel", "fold_finish_kernel"):
        if key in name:
            return key
    return name[:60]


def counters(path):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def main(d):
    stats = list(csv.DictReader(open(glob.glob(os.path.join(d, "trace", "*kernel_stats.csv"))[0])))
    print("| kernel | calls | avg ms | total % |\n|---|---|---|---|")
    for r in stats:
        print(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | {float(r['Percentage']):.2f} |")
    fetch = counters(glob.glob(os.path.join(d, "FETCH_SIZE", "*counter_collection.csv"))[0])
    write = counters(glob.glob(os.path.join(d, "WRITE_SIZE", "*counter_collection.csv"))[0])
    cf = counters(glob.glob(os.path.join(d, "copy_FETCH_SIZE", "*counter_collection.csv"))[0])
    cw = counters(glob.glob(os.path.join(d, "copy_WRITE_SIZE", "*counter_collection.csv"))[0])
    copy_kib = 1024 * 1024  # --copy-calibration 1024: 1 GiB read and 1 GiB written per launch
    copy_name = next(k for k in cf if "copy" in k.lower() and cf[k] > 1000)
    f_fac, w_fac = copy_kib / cf[copy_name], copy_kib / cw[copy_name]
    print(f"\nCopy calibration ({copy_name}, 1 GiB): FETCH_SIZE {cf[copy_name]:.0f} KiB, "
          f"WRITE_SIZE {cw[copy_name]:.0f} KiB per launch -> factors {f_fac:.3f} (fetch), {w_fac:.3f} (write)\n")
    print("| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/dispatch (scaled) |\n|---|---|---|---|")
    out = {}
    for k in fetch:
        if k in write:
            b = (fetch[k] * f_fac + write[k] * w_fac) * 1024
            out[k] = b
            print(f"| {k} | {fetch[k]:.0f} | {write[k]:.0f} | {b / 1e9:.3f} GB |")
    # achieved HBM bandwidth: counted bytes per dispatch over the traced
    # average duration (same kernel names; the two runs share the workload)
    avg_ms = {short(r["Name"]): float(r["AverageNs"]) / 1e6 for r in stats}
    print("\nAchieved HBM bandwidth (counted bytes per dispatch / traced average duration; "
          "MI355X HBM3E peak 8 TB/s):\n")
    print("| kernel | avg ms | HBM bytes/dispatch | TB/s | % of 8 TB/s |\n|---|---|---|---|---|")
    bw = {}
    for k, b in sorted(out.items(), key=lambda kv: -kv[1]):
        if k in avg_ms and avg_ms[k] > 0 and k != "copyBuffer":
            tbs = b / (avg_ms[k] * 1e-3) / 1e12
            bw[k] = tbs
            print(f"| {k} | {avg_ms[k]:.4f} | {b / 1e9:.3f} GB | {tbs:.2f} | {100 * tbs / 8:.0f} % |")
    return dict(fetch_factor=f_fac, write_factor=w_fac, bytes=out, fetch=fetch, write=write, tb_per_s=bw)


def clock_table(d):
    """Counters of the kernels that matter, from every <d>/*/ pmc run."""
    keep = ("attn_", "gemm_")
    vals = collections.defaultdict(dict)
    durs = collections.defaultdict(list)
    for sub in sorted(glob.glob(os.path.join(d, "*", ""))):
        cc = glob.glob(os.path.join(sub, "*counter_collection.csv"))
        tr = glob.glob(os.path.join(sub, "*kernel_trace.csv"))
        if not cc:
            continue
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(cc[0])):
            k = short(r["Kernel_Name"])
            if k.startswith(keep):
                agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k, cs in agg.items():
            for c, v in cs.items():
                vals[k][c] = sum(v) / len(v)
        for r in csv.DictReader(open(tr[0])) if tr else []:
            k = short(r["Kernel_Name"])
            if k.startswith(keep):
                durs[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    print("| kernel | ms | clock GHz | MFMA busy | LDS active | counters per dispatch |\n|---|---|---|---|---|---|")
    out = {}
    for k, cs in sorted(vals.items()):
        t = sum(durs[k]) / len(durs[k]) if durs[k] else float("nan")
        cyc = cs.get("GRBM_GUI_ACTIVE", float("nan")) / 8
        row = dict(ms=t * 1e3, clock_ghz=cyc / t / 1e9,
                   mfma_busy=cs.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / 1024 / cyc,
                   lds_active=cs.get("SQ_LDS_IDX_ACTIVE", float("nan")) / 256 / cyc, counters=cs)
        out[k] = row
        cstr = ", ".join(f"{c} {v:.4g}" for c, v in sorted(cs.items()))
        print(f"| {k} | {row['ms']:.3f} | {row['clock_ghz']:.2f} | {100 * row['mfma_busy']:.1f} % | "
              f"{100 * row['lds_active']:.1f} % | {cstr} |")
    return out


def per_config(paths):
    """One row per bench.py JSON line (the last line of each file)."""
    rows = []
    for path in paths:
        lines = [ln for ln in open(path).read().splitlines() if ln.startswith("{")]
        rows.append(json.loads(lines[-1]))
    print("| workload | B | precision | samples/s | ms/step mean / median / min | student attn ms | "
          "student attn TFLOP/s (% of 2.5 PF) | teacher attn TFLOP/s | DMD ms/call | target + backward ms | "
          "attn backward TFLOP/s |\n|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        c, rf = r["config"], r["roofline"]
        name = c["workload"].split(" ")[0]
        dmd = r.get("dmd_target", {}).get("ms_per_call")
        grad = r.get("scm_grad", {})
        fmt = lambda x, f: "-" if x is None else f.format(x)
        print(f"| {name} | {c['global_batch']} | {c.get('precision', 'bf16')} | {r['value']:.1f} | "
              f"{r['ms_per_step']:.3f} / {r.get('ms_per_step_median', float('nan')):.3f} / "
              f"{r.get('ms_per_step_min', float('nan')):.3f} | {rf['avg_launch_ms']:.3f} | "
              f"{rf['achieved']:.0f} ({100 * rf['frac']:.1f} %) | {r.get('teacher_attn_tflops', float('nan')):.0f} | "
              f"{fmt(dmd, '{:.3f}')} | {fmt(grad.get('ms_per_call'), '{:.3f}')} | "
              f"{fmt(grad.get('attn_bwd_tflops'), '{:.0f}')} |")
    return rows


COUNTER_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <dir>/FETCH_SIZE -o run -- python3 bench.py "
    "--steps 2 --warmup 1 --no-cpu-baseline --dmd-steps 1 --grad-steps 1",
    "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <dir>/WRITE_SIZE -o run -- python3 bench.py "
    "--steps 2 --warmup 1 --no-cpu-baseline --dmd-steps 1 --grad-steps 1",
    "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <dir>/copy_FETCH_SIZE -o run -- python3 "
    "bench.py --copy-calibration 1024 --steps 3",
    "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <dir>/copy_WRITE_SIZE -o run -- python3 "
    "bench.py --copy-calibration 1024 --steps 3",
    "python -m joint_video_audio_trigflow_amd.profile_summary --counters-record <dir> "
    "profiles/attn_fwd_jvp_high_res_counters.json",
]


def counters_record(d, out_path):
    """The student attention's counted traffic per launch, for bench.py."""
    res = main(d)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    k, c = "attn_fwd_jvp<128,true> (student fwd+JVP)", "attn_combine<128,true> (JVP split-tail merge)"
    rec = {
        "kernel": "attn_fwd_jvp_kernel<128,true>",
        "workload": "high-res joint sCM target (bench.py defaults)",
        "kernel_source_digest": bench.attention_kernel_digest(),
        "kernel_source_digest_of": "bench.attention_kernel_digest(): attention.hip + attn_tiles.h + common.h up "
                                   "to the per-sample coefficient table + struct AttnParams",
        "fetch_kib_per_dispatch": res["fetch"][k],
        "write_kib_per_dispatch": res["write"][k],
        "fetch_factor": res["fetch_factor"],
        "write_factor": res["write_factor"],
        "traffic_bytes_per_launch": res["bytes"][k] + res["bytes"].get(c, 0.0),
        "commands": COUNTER_COMMANDS,
        "combine_fetch_kib_per_dispatch": res["fetch"].get(c, 0.0),
        "combine_write_kib_per_dispatch": res["write"].get(c, 0.0),
    }
    json.dump(rec, open(out_path, "w"), indent=1)
    return rec


if __name__ == "__main__":
    if sys.argv[1] == "--counters-record":
        counters_record(sys.argv[2], sys.argv[3])
        sys.exit(0)
    if sys.argv[1] == "--per-config":
        per_config(sys.argv[2:])
        sys.exit(0)
    if sys.argv[1] == "--clock":
        res = clock_table(sys.argv[2])
        if len(sys.argv) > 3:
            json.dump(res, open(sys.argv[3], "w"), indent=1)
        sys.exit(0)
    res = main(sys.argv[1])
    if len(sys.argv) > 2:
        json.dump(res, open(sys.argv[2], "w"), indent=1)
