"""Build the gfx950 library in-tree: ``libspec_verify.so`` next to this file, from every
HIP source under ``csrc/``.

    python -m rejection_sampling_verify_02_amd.build

hipcc cross-compiles for gfx950 without a GPU present.  Packed-FP32 instructions
are disabled for the device code (the host pass warns that it does not know the
feature; that warning is harmless).
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
SRCS = sorted(CSRC.glob("*.hip"))  # every kernel source, one library
LIB = PKG / "libspec_verify.so"
# The same sources with the timeline stamps compiled in (a measurement build: bench.py
# --timeline); the product library above has none.
LIB_TIMELINE = PKG / "libspec_verify_timeline.so"
ARCH = os.environ.get("SV_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: Path, timeline: bool = False) -> list[str]:
    return [
        "/opt/rocm/bin/hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", *(["-DSV_TIMELINE"] if timeline else []),
        "-I", str(ROOT / "include"), "-I", str(CSRC),
        "-o", str(out), *[str(p) for p in SRCS],
    ]


def build(verbose: bool = False) -> Path:
    """Both libraries, compiled side by side; returns the product library's path."""
    jobs = []
    for lib, tl in ((LIB, False), (LIB_TIMELINE, True)):
        tmp = lib.with_name(lib.name + ".tmp")
        cmd = hipcc_command(tmp, tl)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((lib, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = []
    for lib, tmp, proc in jobs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out + err)
            failed.append(lib.name)
        else:
            os.replace(tmp, lib)
    if failed:
        raise RuntimeError("hipcc failed to build " + ", ".join(failed))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
