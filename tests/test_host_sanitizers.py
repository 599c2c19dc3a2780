"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The host API (csrc/t2va_api.cpp) is compiled with both sanitizers on its host
code (-Xarch_host: the device code is not instrumented) and linked with the
library's other objects and tests/host/abi_checks.cpp, a driver that calls
every entry point with arguments that must be rejected before anything
reaches the GPU, plus the workspace-size queries over the descriptors' ranges.
The run must exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "joint_video_audio_trigflow_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_validation_paths_are_clean_under_asan_and_ubsan(tmp_path):
    from joint_video_audio_trigflow_amd import build
    cc = hipcc()
    no_packed = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    base = ["-std=c++17", "-fPIC", f"--offload-arch={build.ARCH}", "-I", os.path.join(ROOT, "include")]
    objs, procs = [], []
    for src in sorted(os.listdir(CSRC)):
        if not src.endswith((".hip", ".cpp")):
            continue
        obj = str(tmp_path / (src + ".o"))
        # the host API with both sanitizers; the kernels' sources as the library builds them
        flags = base + (["-O1", "-g", *SAN] if src == "t2va_api.cpp" else ["-O3"]) + no_packed
        procs.append(subprocess.Popen([cc, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        objs.append(obj)
    for pr in procs:
        out, _ = pr.communicate()
        assert pr.returncode == 0, out.decode(errors="replace")[-3000:]
    drv = str(tmp_path / "abi_checks.o")
    subprocess.run([cc, "-O1", "-g", *base, *SAN, "-x", "hip", "--cuda-host-only", "-c",
                    os.path.join(ROOT, "tests", "host", "abi_checks.cpp"), "-o", drv], check=True, capture_output=True)
    exe = str(tmp_path / "abi_checks")
    subprocess.run([cc, f"--offload-arch={build.ARCH}", *SAN, drv, *objs, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "abi checks ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
