"""Sanitizer builds of the oracle (host code; no GPU).

tests/oracle_sanitize_main.c calls every oracle entry point on a tiny problem, threaded
paths included.  It is built with gcc together with oracle/prism_oracle.c under
AddressSanitizer + UndefinedBehaviorSanitizer, and under ThreadSanitizer (the oracle splits
zones, rows and query blocks over pthreads), and must run clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "prism_oracle.c")
MAIN = os.path.join(ROOT, "tests", "oracle_sanitize_main.c")

BUILDS = {
    "address+undefined": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    "thread": ["-fsanitize=thread", "-fPIE", "-pie"],
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", list(BUILDS))
def test_oracle_under_sanitizer(tmp_path, name):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", *BUILDS[name], "-I", os.path.join(ROOT, "oracle"), MAIN, SRC, "-o", exe,
           "-lm", "-lpthread"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and "cannot find" in b.stderr and "san" in b.stderr:
        pytest.skip(f"{name} runtime not installed: {b.stderr.strip().splitlines()[-1]}")
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-4000:]
    assert "oracle driver ok" in out
