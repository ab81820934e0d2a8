"""Build libstagegemm.so (the HIP kernels and the C-ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libstagegemm.so")
PROBE_LIB = os.path.join(PKG, "libsgprobe.so")
RESOURCES = os.path.join(PKG, "kernel_resources.txt")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions are kept out of all code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    return [os.path.join(CSRC, "stagegemm.hip"), os.path.join(CSRC, "attention.hip")]


def probe_sources() -> list[str]:
    """Measurement probe (MFMA ceiling on given operands), a separate library."""
    return [os.path.join(CSRC, "mfma_ceiling.hip")]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libstagegemm.so next to this file and
    record per-kernel register / LDS / occupancy remarks in
    kernel_resources.txt.  Always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC,
           "-Rpass-analysis=kernel-resource-usage", *sources(), "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        sys.stderr.write(p.stdout + p.stderr)
        raise RuntimeError("hipcc failed building libstagegemm.so")
    os.replace(tmp, LIB)
    remarks = [ln for ln in p.stderr.splitlines() if "remark:" in ln]
    with open(RESOURCES, "w") as f:
        f.write("\n".join(_clean(r) for r in remarks) + "\n")
    tmp = PROBE_LIB + ".tmp"
    p2 = subprocess.run([HIPCC, *FLAGS, *probe_sources(), "-o", tmp], capture_output=True, text=True)
    if p2.returncode != 0:
        sys.stderr.write(p2.stdout + p2.stderr)
        raise RuntimeError("hipcc failed building libsgprobe.so")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        sys.stdout.write(p.stderr)
    return LIB


def _clean(line: str) -> str:
    # strip absolute paths so the record does not depend on the checkout
    return re.sub(r"^.*?/csrc/", "csrc/", line)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
