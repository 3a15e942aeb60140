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
    assert header_functions() == ["fa_bwd", "fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc",
                                  "fa_fwd_splitkv_plan", "fa_status_string"]


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
    assert "workspace" in fa.fa_status_string(fa.FA_ERR_WORKSPACE)
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
    (dict(q=Q + 8), fa.FA_ERR_INVALID_ARG),                                           # q not 16-byte aligned
    (dict(v=V + 2), fa.FA_ERR_INVALID_ARG),                                           # v not 16-byte aligned
    (dict(o=O + 4), fa.FA_ERR_INVALID_ARG),                                           # o not 16-byte aligned
    (dict(lse=L + 2), fa.FA_ERR_INVALID_ARG),                                         # lse not 4-byte aligned
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
    (dict(dk=DQ + 16), fa.FA_ERR_INVALID_ARG),      # dk overlaps dq
    (dict(delta=DO + 8), fa.FA_ERR_INVALID_ARG),    # workspace overlaps dout
    (dict(dv=L + 16), fa.FA_ERR_INVALID_ARG),       # dv overlaps lse
    (dict(dout=DO + 8), fa.FA_ERR_INVALID_ARG),     # dout not 16-byte aligned
    (dict(dq=DQ + 4), fa.FA_ERR_INVALID_ARG),       # dq not 16-byte aligned
    (dict(delta=DL + 2), fa.FA_ERR_INVALID_ARG),    # delta not 4-byte aligned
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


# ---- split-KV planning and host checks (no HIP call is made by any of these) ---------------

def plan(B=1, H=1, N=256, d=64, dtype=fa.FA_F32, causal=0, num_splits=0):
    return fa.fa_fwd_splitkv_plan(B, H, N, d, dtype, causal, num_splits)


def expected_plan(B, H, N, d, dtype, num_splits, tile, rows, causal=0):
    """The plan rule restated: at most one column per key tile, columns of whole tiles, no
    empty column; below 256 workgroups the default aims at 256 of them (2048 under the causal
    mask, where the columns past the diagonal exit at once), in columns of at least 1024 keys."""
    import math
    dp = 64 if d <= 64 else (128 if d <= 128 else 256)
    tiles = math.ceil(N / tile)
    base = B * H * math.ceil(N / rows)
    want = num_splits or (1 if base >= 256 else min(math.ceil((2048 if causal else 256) / base), math.ceil(N / 1024)))
    want = max(1, min(want, 64, tiles))
    chunk = math.ceil(tiles / want) * tile
    ns = math.ceil(N / chunk)
    if ns == 1:
        return 1, 0
    rows_all = ns * B * H * N
    u = rows_all * dp * 4
    return ns, (u + 255) // 256 * 256 + rows_all * 8


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("B,H,N,d,dtype,ns", [
    (1, 1, 256, 64, fa.FA_F32, 0),      # the fp32 single-head workload: too few keys to split
    (1, 1, 256, 64, fa.FA_F32, 3),
    (1, 1, 256, 64, fa.FA_F32, 64),     # clamped to the 8 key tiles
    (1, 1, 8192, 128, fa.FA_BF16, 0),
    (1, 1, 8192, 128, fa.FA_BF16, 7),
    (2, 8, 1024, 64, fa.FA_BF16, 0),    # 256 workgroups already: one column
    (1, 2, 1000, 96, fa.FA_BF16, 5),
    (1, 1, 33, 200, fa.FA_F32, 4),      # 2 key tiles of 32
    (1, 1, 1, 64, fa.FA_BF16, 8),       # one key: one column
    (1, 1, 32768, 128, fa.FA_BF16, 0),  # 128 workgroups: 2 columns, 16 under the causal mask
    (1, 1, 3000, 64, fa.FA_BF16, 0),    # 3 columns at most (1024 keys or more each)
    (1, 3, 4000, 64, fa.FA_BF16, 0),
])
def test_splitkv_plan(lib, B, H, N, d, dtype, ns, causal):
    st, nsplit, wbytes = plan(B, H, N, d, dtype, causal, ns)
    assert st == fa.FA_OK
    if dtype == fa.FA_F32:
        tile, rows = 32, {64: 32, 128: 64, 256: 128}[64 if d <= 64 else (128 if d <= 128 else 256)]
    else:
        tile = 32 if d > 128 else 64
        rows = {64: 64, 128: 256, 256: 128}[64 if d <= 64 else (128 if d <= 128 else 256)]
    assert (nsplit, wbytes) == expected_plan(B, H, N, d, dtype, ns, tile, rows, causal)


@pytest.mark.parametrize("kwargs,status", [
    (dict(num_splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=65), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=257), fa.FA_ERR_UNSUPPORTED),
])
def test_splitkv_plan_rejects(lib, kwargs, status):
    assert plan(**kwargs)[0] == status


WS = 11 * BIG


def call_split(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=256, d=64, scale=0.125, causal=0, dtype=fa.FA_F32,
               num_splits=8, ws=WS, ws_bytes=1 << 30):
    return fa.fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=100), fa.FA_ERR_INVALID_ARG),
    (dict(d=300), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=1000), fa.FA_ERR_WORKSPACE),
    (dict(ws=WS + 16), fa.FA_ERR_INVALID_ARG),          # not 256-byte aligned
    (dict(ws=O + 256), fa.FA_ERR_INVALID_ARG),          # overlaps o
    (dict(ws=L - 256), fa.FA_ERR_INVALID_ARG),          # overlaps lse
    (dict(o=Q + 64), fa.FA_ERR_INVALID_ARG),            # o overlaps q
])
def test_splitkv_invalid_arguments_rejected_on_host(lib, kwargs, status):
    assert call_split(**kwargs) == status


def test_splitkv_workspace_exactly_the_plan_passes_host_checks(lib):
    """A workspace of exactly the planned size passes the size check (one byte less does not);
    checked with an invalid q so that nothing is launched."""
    st, ns, need = plan(num_splits=8)
    assert ns == 8 and need > 0
    assert call_split(q=None, ws_bytes=need) == fa.FA_ERR_INVALID_ARG
    assert call_split(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=5), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=65), fa.FA_ERR_INVALID_ARG),
    (dict(d=300), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1, H=4, N=65536, d=128, dtype=fa.FA_BF16, num_splits=64), fa.FA_ERR_SCRATCH),   # > 64 MiB of states
])
def test_noalloc_rejects_on_host(lib, kwargs, status):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=256, d=64, scale=0.125, causal=0, dtype=fa.FA_F32, num_splits=8)
    a.update(kwargs)
    assert fa.fa_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                     a["scale"], a["causal"], a["dtype"], a["num_splits"], None) == status
