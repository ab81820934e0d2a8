"""The oracle's pins, re-run against a build of oracle.c with the address and
undefined-behaviour sanitizers.

oracle.c does 128-bit integer arithmetic, shifts by computed amounts and
indexes flat arrays with products of dimensions; a silent overflow, an
out-of-range shift or an out-of-bounds read there could still pass the value
pins by chance.  This test builds the same source with
-fsanitize=address,undefined (every report fatal), preloads the sanitizer
runtimes into a child Python and runs the oracle's pin files against that
build.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from oracle import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_gemm.py", "tests/test_oracle_beta.py", "tests/test_oracle_codec.py",
        "tests/test_oracle_attention.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build(force=True, out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = dict(os.environ)
    env.update({
        _native.LIBRARY_ENV: lib,
        "LD_PRELOAD": f"{asan}:{ubsan}",
        # Python itself is not instrumented: its arenas are not leaks
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
        "OMP_NUM_THREADS": "4",
    })
    # -s: a sanitizer report goes to the child's stderr, not into pytest's capture
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *PINS]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (p.stdout + p.stderr)[-4000:]
    assert p.returncode == 0, tail
    assert "passed" in p.stdout and "AddressSanitizer" not in p.stderr, tail
    assert "runtime error" not in p.stderr, tail
