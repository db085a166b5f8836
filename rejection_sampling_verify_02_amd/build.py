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
ARCH = os.environ.get("SV_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: Path) -> list[str]:
    return [
        "/opt/rocm/bin/hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", str(ROOT / "include"), "-I", str(CSRC),
        "-o", str(out), *[str(p) for p in SRCS],
    ]


def build(verbose: bool = False) -> Path:
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libspec_verify.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
