"""The library's host-side code (argument checks, workspace and launch plans, status
strings) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/host_sanitize_main.cpp calls every sizing and plan entry point over a grid of
shapes, dtypes (including unsupported values), temperatures and top-k values, and the
entry points with arguments they must refuse before any HIP call.  It is built with the
sanitizers on the host pass only (-Xarch_host before each -fsanitize=; the device code is
compiled as usual and never runs) and must run clean, leak check included."""
import os
import subprocess
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def test_host_code_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "host_sanitize"
    srcs = sorted(str(p) for p in (ROOT / "rejection_sampling_verify_02_amd" / "csrc").glob("*.hip"))
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", str(ROOT / "include"), "-I", str(ROOT / "rejection_sampling_verify_02_amd" / "csrc"),
           str(ROOT / "tests" / "host_sanitize_main.cpp"), *srcs, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    got = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    # the statuses of include/spec_verify.h and include/sv_probe.h for the refused calls
    assert got["null"] == "1" and got["shape"] == "2" and got["dtype"] == "3" and got["temp"] == "4"
    assert got["workspace"] == "5" and got["align"] == "6" and got["sample"] == "1"
    assert got["typical"] == "8" and got["probe"] == "2" and got["epoch"] == "0"
