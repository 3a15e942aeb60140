"""The address arithmetic of the direct global -> LDS tile loads (fa_dma.h, used by the tuned
forward kernels, d = 128 and 64, and both backward kernels), walked on the host for every load of every wave:
N = 1..600 and the workloads' lengths, both masks, head widths 64 and 128. Each load must read
inside its head, read the row and chunk it should, write inside its LDS slot, and cover every
place of its tile once. The forward kernels' ring schedule is walked as well (which phase
interval requests, reads and reuses each slot, for rings of 4 to 6 slots). Three planted mistakes
must be caught: the dQ kernel's earlier base row (not clamped to N-1, which made the unsigned
lane offsets wrap for N < 64), loads that do not pull rows past N-1 back, and a ring lead one
tile deeper than the slots allow."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_softmax_attention_fa_amd", "csrc")
NS = [str(n) for n in range(1, 601)] + ["1000", "1024", "4096", "8192", "32768"]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.fail("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("dma") / "dma_bounds")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "dma_bounds.cpp"), "-o", exe], check=True)
    return exe


def run(exe, *args):
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=600)


def test_every_load_in_bounds(checker):
    r = run(checker, *NS)
    assert r.returncode == 0, r.stderr[-2000:]
    loads = int(r.stdout.split("loads checked:")[1].split(",")[0])
    assert loads > 10 ** 9


def test_unclamped_dq_base_is_caught(checker):
    r = run(checker, "--old-dq-base", *NS[:100])
    assert r.returncode == 1 and "dq" in r.stderr and "wraps below 0" in r.stderr


def test_missing_pull_back_is_caught(checker):
    r = run(checker, "--no-back", "1", "31", "65", "100", "300")
    assert r.returncode == 1 and "read outside the head" in r.stderr


def test_too_deep_ring_lead_is_caught(checker):
    r = run(checker, "--deep-lead", "64", "300", "1000")
    assert r.returncode == 1 and "slot rewritten before its last read" in r.stderr
