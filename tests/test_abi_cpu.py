"""The C-ABI library on a machine without a GPU: it loads, exports every symbol the header
declares, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import exact_softmax_attention_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        pytest.fail("libfa.so is not built (run python -m exact_softmax_attention_fa_amd.build)")
    return fa.load_library()


def test_header_declares_entry_points():
    assert header_functions() == ["fa_bwd", "fa_fwd", "fa_fwd_f32", "fa_status_string"]


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r"\bT\s+(fa_\w+)", out.stdout))
        assert set(header_functions()) <= exported


def test_status_strings(lib):
    assert fa.fa_status_string(fa.FA_OK) == "ok"
    assert fa.fa_status_string(fa.FA_ERR_INVALID_ARG) == "invalid argument"
    assert "256" in fa.fa_status_string(fa.FA_ERR_UNSUPPORTED)
    assert fa.fa_status_string(fa.FA_ERR_HIP) == "HIP launch error"
    assert fa.fa_status_string(12345) == "unknown status"


# Fake, well-separated "device" addresses: validation only compares them, never touches them.
BIG = 1 << 40
Q, K, V, O, L = BIG, 2 * BIG, 3 * BIG, 4 * BIG, 5 * BIG


def call(fn, q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=16, d=64, scale=0.125, causal=0):
    return fn(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_f32], ids=["bf16", "f32"])
@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(d=257), fa.FA_ERR_UNSUPPORTED),
    (dict(d=4096), fa.FA_ERR_UNSUPPORTED),
    (dict(B=2 ** 31 - 1, H=2 ** 31 - 1, N=2 ** 31 - 1, d=128), fa.FA_ERR_INVALID_ARG),   # > 2^62 elements
    (dict(N=2 ** 25, d=128), fa.FA_ERR_UNSUPPORTED),                                 # N*d above 2^31
    (dict(o=Q + 64), fa.FA_ERR_INVALID_ARG),                                          # o overlaps q
    (dict(lse=V + 8), fa.FA_ERR_INVALID_ARG),                                         # lse overlaps v
    (dict(lse=O + 16), fa.FA_ERR_INVALID_ARG),                                        # lse overlaps o
])
def test_invalid_arguments_rejected_on_host(lib, fn, kwargs, status):
    assert call(fn, **kwargs) == status


DO, DQ, DK, DV, DL = 6 * BIG, 7 * BIG, 8 * BIG, 9 * BIG, 10 * BIG


def call_bwd(q=Q, k=K, v=V, o=O, dout=DO, lse=L, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=1, N=16, d=64,
             scale=0.125, causal=0):
    return fa.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dout=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(dq=None), fa.FA_ERR_INVALID_ARG),
    (dict(delta=None), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dq=Q + 64), fa.FA_ERR_INVALID_ARG),       # dq overlaps q
    (dict(dk=DQ + 2), fa.FA_ERR_INVALID_ARG),       # dk overlaps dq
    (dict(delta=DO + 8), fa.FA_ERR_INVALID_ARG),    # workspace overlaps dout
    (dict(dv=L + 4), fa.FA_ERR_INVALID_ARG),        # dv overlaps lse
])
def test_backward_invalid_arguments_rejected_on_host(lib, kwargs, status):
    assert call_bwd(**kwargs) == status


def test_missing_library_fails_loudly(tmp_path):
    code = ("import exact_softmax_attention_fa_amd as fa\n"
            "try:\n    fa.fa_status_string(0)\nexcept RuntimeError as e:\n    print('RAISED', e)\n")
    env = dict(os.environ, FA_LIBRARY=str(tmp_path / "nope.so"), PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert "RAISED" in out.stdout and "not built" in out.stdout


def test_product_never_imports_oracle():
    """The HIP path's package and its sources mention no module of the oracle."""
    pkg = os.path.join(ROOT, "exact_softmax_attention_fa_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
                assert "oracle/" not in text, f


def test_oracle_imports_nothing_from_the_product():
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "exact_softmax_attention_fa_amd" not in text, f
            assert "torch" not in text, f
