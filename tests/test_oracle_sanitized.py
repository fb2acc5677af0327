"""The oracle's pins, re-run against an AddressSanitizer + UndefinedBehaviorSanitizer
build of the same C source (CPU only).

The oracle is compiled a second time with gcc's -fsanitize=address,undefined
into a temporary directory and loaded in a child interpreter in place of the
normal build (LH_ORACLE_LIB), with the sanitizer runtimes preloaded.  Any
out-of-bounds access, use after free or undefined operation in the oracle
aborts the child, and the sanitizer's report is shown.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lh_oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_causality.py", "tests/test_oracle_parent_kept.py",
        "tests/test_oracle_score_modes.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "liblh_oracle_sanitized.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", lib, SRC, "-lm"], check=True)
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ, LH_ORACLE_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS=f"detect_leaks=0:log_path={log}", UBSAN_OPTIONS=f"print_stacktrace=1:log_path={log}",
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(f).read() for f in sorted(glob.glob(log + "*")))
    assert r.returncode == 0 and not reports, (reports or "") + r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
