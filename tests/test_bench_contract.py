"""bench.py's contract where it needs no GPU: more than one GPU is refused
with a message, and counted HBM traffic is reported only for the kernel
sources the counters were taken on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_sources_it_was_counted_on():
    sys.path.insert(0, ROOT)
    import bench
    from joint_video_audio_trigflow_amd import inputs
    rec = json.load(open(os.path.join(ROOT, "profiles", "attn_fwd_jvp_high_res_counters.json")))
    t = bench.counted_traffic(inputs.CONFIGS["high-res"])
    if rec["kernel_source_digest"] == bench.attention_kernel_digest():
        assert t is not None and t > 0.9e9      # at least the algorithmic bytes
    else:
        assert t is None                        # counters of another kernel version
    assert bench.counted_traffic(inputs.CONFIGS["standard"]) is None
