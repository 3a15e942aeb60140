"""The C-ABI front end (argument validation, split planning, the launch arguments it computes)
built for the host with the address and undefined-behaviour sanitizers and driven through a
table of valid, invalid and extreme arguments (tests/abi_sanitize.cpp). The kernel launchers are
stubs in this build, so no call reaches a device; any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_softmax_attention_fa_amd", "csrc")
# host-side sanitizers only (the build has no device code)
SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.fail("hipcc not found")


def test_front_end_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    cmd = [hipcc(), "--offload-host-only", "-std=c++17", "-O1", "-g", *SANITIZE.split(),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "fa_api.hip"),
           os.path.join(ROOT, "tests", "abi_sanitize.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "cases failed: 0" in r.stdout
