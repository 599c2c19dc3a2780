"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message, and the traffic record matches the kernel sources."""
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


def test_counter_record_describes_the_current_attention_sources():
    sys.path.insert(0, ROOT)
    import bench
    from joint_video_audio_trigflow_amd import inputs
    rec = json.load(open(os.path.join(ROOT, "profiles", "attn_fwd_jvp_high_res_counters.json")))
    assert rec["kernel_source_digest"] == bench.attention_kernel_digest()
    t = bench.counted_traffic(inputs.CONFIGS["high-res"])
    assert t is not None and t > 0.9e9          # at least the algorithmic bytes
    assert bench.counted_traffic(inputs.CONFIGS["standard"]) is None
