"""The oracle's own checks (its pins, the twin comparisons, the option and
convolution pins) run once more against a build of ssm_oracle.c with
AddressSanitizer and UndefinedBehaviorSanitizer, in a child process with the
ASan runtime preloaded: an out-of-bounds access, a use after free or
undefined behaviour in the oracle fails this test."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

from tests.conftest import ROOT

ORACLE_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_bwd_twins.py",
                "tests/test_oracle_options.py", "tests/test_oracle_conv.py"]


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_checks_pass_under_asan_and_ubsan(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's ASan runtime is not available")
    from oracle import oracle_c
    lib = oracle_c.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    env = dict(os.environ)
    env["ORACLE_LIB_OVERRIDE"] = lib
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # Python's own allocations are not instrumented: leaks are not reported
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *ORACLE_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in r.stdout


def test_sanitizer_catches_a_planted_out_of_bounds_read(tmp_path):
    """The same harness on a copy of the oracle whose forward reads u one
    whole (B,L,D) array past the end: ASan must stop the run (so a green run
    above means something)."""
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's ASan runtime is not available")
    from oracle import oracle_c
    src = open(oracle_c._SRC).read()
    planted = src.replace("const double x = j->u[idx];", "const double x = j->u[idx + 3 * 64 * 16];", 1)
    assert planted != src
    bad = tmp_path / "ssm_oracle_planted.c"
    bad.write_text(planted)
    lib = str(tmp_path / "liboracle_planted.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-o", lib, str(bad), "-lm", "-lpthread"])
    env = dict(os.environ)
    env["ORACLE_LIB_OVERRIDE"] = lib
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0"
    code = ("import numpy as np; from oracle import oracle_c; r = np.random.default_rng(0); "
            "u = r.standard_normal((1, 64, 16)); oracle_c.scan_fwd(u, u, -np.ones((16, 4)), "
            "r.standard_normal((1, 64, 4)), r.standard_normal((1, 64, 4)))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr, r.stderr[-2000:]
