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
# compiler remarks (registers, LDS, occupancy per kernel): a build log, kept
# out of the source tree's history under the ignored build/ directory
RESOURCES = os.path.join(ROOT, "build", "kernel_resources.txt")

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


def _device_asm(source: str) -> str:
    """Compile one source to gfx950 assembly under build/ and return its path."""
    out_dir = os.path.join(ROOT, "build")
    os.makedirs(out_dir, exist_ok=True)
    asm = os.path.join(out_dir, os.path.splitext(os.path.basename(source))[0] + ".s")
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only",
           "-S", "-I", INCLUDE, "-I", CSRC, source, "-o", asm]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        sys.stderr.write(p.stdout + p.stderr)
        raise RuntimeError(f"hipcc failed compiling {os.path.basename(source)} to assembly")
    return asm


def m0_uses(asm: str, function=None) -> tuple[int, list[str]]:
    """m0 operands in a compiled assembly file, within the functions whose
    symbol `function(name)` accepts (every function when None): the count
    inside inline-assembly regions and the lines outside them."""
    inside, take, found, stray = False, function is None, 0, []
    with open(asm) as f:
        for n, line in enumerate(f, 1):
            head = None if inside else re.match(r"^([A-Za-z_.$][\w.$]*):", line)
            if head and not head.group(1).startswith("."):      # a function's symbol
                take = function is None or function(head.group(1))
            if ";;#ASMSTART" in line:
                inside = True
                continue
            if ";;#ASMEND" in line:
                inside = False
                continue
            code = line.split(";", 1)[0]
            if take and re.search(r"\bm0\b", code):
                if inside:
                    found += 1
                else:
                    stray.append(f"{n}: {line.strip()}")
    return found, stray


def check_m0_confined() -> int:
    """The attention kernels and the schedule-10 GEMM mainloop issue their
    LDS-DMA through inline assembly that writes m0 (the LDS address register
    of the instruction) and lists it as clobbered.  The compiler does not
    preserve a reserved register across such a statement, so the DMA is safe
    only while no compiler-generated code in those functions uses m0: all of
    attention.hip, and in stagegemm.hip the kernels instantiated for schedules
    10-12 and 14 (the other GEMM kernels load through the compiler's own LDS-DMA
    builtin, which sets m0 itself).  Compile both to assembly and check that
    every m0 operand there lies inside an inline-assembly region; raise
    otherwise (for instance after a compiler update).  Returns the number of
    m0 operands found, all inside the DMA statements."""
    total = 0
    checks = [("attention.hip", None),
              # Cfg<..., 10 | 11 | 12 | 14>: the template's last argument mangles as Li10EE ...
              ("stagegemm.hip", lambda name: any(f"Li{k}EE" in name for k in (10, 11, 12, 14)))]
    for src, function in checks:
        found, stray = m0_uses(_device_asm(os.path.join(CSRC, src)), function)
        if stray:
            raise RuntimeError(f"compiler-generated code uses m0 in {src}, which the inline "
                               "LDS-DMA clobbers:\n" + "\n".join(stray[:20]))
        if found == 0:
            raise RuntimeError(f"no m0 operand found in the DMA statements of {src}: the check "
                               "no longer sees them")
        total += found
    return total


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libstagegemm.so next to this file and
    record per-kernel register / LDS / occupancy remarks in
    build/kernel_resources.txt.  Always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC,
           "-Rpass-analysis=kernel-resource-usage", *sources(), "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        sys.stderr.write(p.stdout + p.stderr)
        raise RuntimeError("hipcc failed building libstagegemm.so")
    os.replace(tmp, LIB)
    remarks = [ln for ln in p.stderr.splitlines() if "remark:" in ln]
    os.makedirs(os.path.dirname(RESOURCES), exist_ok=True)
    with open(RESOURCES, "w") as f:
        f.write("\n".join(_clean(r) for r in remarks) + "\n")
    tmp = PROBE_LIB + ".tmp"
    p2 = subprocess.run([HIPCC, *FLAGS, *probe_sources(), "-o", tmp], capture_output=True, text=True)
    if p2.returncode != 0:
        sys.stderr.write(p2.stdout + p2.stderr)
        raise RuntimeError("hipcc failed building libsgprobe.so")
    os.replace(tmp, PROBE_LIB)
    check_m0_confined()
    if verbose:
        sys.stdout.write(p.stderr)
    return LIB


def _clean(line: str) -> str:
    # strip absolute paths so the record does not depend on the checkout
    return re.sub(r"^.*?/csrc/", "csrc/", line)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
