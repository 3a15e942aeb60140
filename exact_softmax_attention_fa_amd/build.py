"""Build the HIP library libfa.so in-tree for gfx950 with hipcc.

Usage: ``python -m exact_softmax_attention_fa_amd.build`` (or ``build()`` from Python).
Every call recompiles. The library lands next to this file, where the binding loads it.

Timing variants: ``python -m exact_softmax_attention_fa_amd.build -D NAME=VALUE ... -o PATH`` builds
the same sources with build-time tile macros (e.g. ``-D FA_BF16_D64W_NW=8``) into PATH instead of the
product library; bench.py loads such a library through ``FA_LIBRARY=PATH`` and marks its line
non-product.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_fwd_bf16_tuned.hip", "fa_fwd_f32.hip", "fa_splitkv.hip",
           "fa_noalloc.hip", "fa_bwd_bf16.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # scores and statistics are never NaN for finite inputs: lets max() skip NaN quieting
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def build(verbose: bool = False, extra_flags=(), output: str | None = None) -> str:
    lib = os.path.abspath(output) if output else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, lib)
    return lib


def main(argv) -> None:
    import argparse
    ap = argparse.ArgumentParser(description="build libfa.so (or a timing variant) for gfx950")
    ap.add_argument("-v", action="store_true", help="print the hipcc command and its messages")
    ap.add_argument("-D", action="append", default=[], metavar="NAME=VALUE",
                    help="build-time macro (tile configuration) for a timing variant")
    ap.add_argument("-o", default=None, metavar="PATH", help="output library (default: the product library)")
    args = ap.parse_args(argv)
    if args.D and not args.o:
        ap.error("a variant built with -D needs its own output path (-o)")
    print(build(verbose=args.v, extra_flags=[f"-D{d}" for d in args.D], output=args.o))


if __name__ == "__main__":
    main(sys.argv[1:])
