"""Fused forward pass of exact softmax attention on AMD MI355X (gfx950).

Thin ctypes binding over the C-ABI library ``libfa.so`` (declared in include/fa.h).
The binding only marshals arguments: every step of the computation runs in the HIP
kernels. PyTorch supplies device memory and the stream.

Entry points with the C names:
  fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> status   (bf16, raw pointers)
  fa_fwd_f32(...)                                              -> status   (fp32, raw pointers)
  fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, workspace,
                 workspace_bytes, stream)                      -> status   (key range split)
  fa_fwd_splitkv_plan(B, H, N, d, dtype, causal, num_splits)   -> (status, nsplit, workspace bytes)
  fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, stream)
                                                               -> status   (library-owned buffer)
  fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, stream) -> status
  fa_status_string(status)                                     -> str
and tensor-level conveniences:
  fwd(q, k, v, scale=None, causal=False) -> (o, lse)
  fwd_splitkv(q, k, v, scale=None, causal=False, num_splits=0) -> (o, lse)
  bwd(q, k, v, o, lse, dout, scale=None, causal=False) -> (dq, dk, dv)
If the library has not been built, every call raises RuntimeError; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv", "fa_fwd_splitkv_plan", "fa_fwd_splitkv_noalloc", "fa_bwd",
           "fa_status_string", "FA_ERR_SCRATCH", "FA_NOALLOC_SCRATCH_BYTES",
           "fwd", "fwd_splitkv", "bwd", "library_path", "load_library", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_WORKSPACE", "FA_BF16", "FA_F32", "FaError"]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_WORKSPACE, FA_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
FA_NOALLOC_SCRATCH_BYTES = 64 << 20
FA_BF16, FA_F32 = 0, 1

_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


def library_path() -> str:
    return os.environ.get("FA_LIBRARY", os.path.join(_PKG, "libfa.so"))


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def load_library():
    """Load libfa.so once; raise RuntimeError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(build it with `python -m exact_softmax_attention_fa_amd.build`)")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7). Loading torch
    # first makes the library bind to that runtime, the one that owns torch's memory and
    # streams; loaded the other way round, the process would hold two HIP runtimes and every
    # launch on a torch stream would fail.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                ctypes.c_void_p]
    for name in ("fa_fwd", "fa_fwd_f32"):
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int,
                                                                          ctypes.c_void_p]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = argtypes[:11] + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                                   ctypes.c_void_p]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = argtypes[:11] + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_fwd_splitkv_plan.argtypes = [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_int),
                                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_fwd_splitkv_plan.restype = ctypes.c_int
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int:
    """bf16 forward on raw device pointers (ints); returns the C status code."""
    return load_library().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int:
    """fp32 forward on raw device pointers (ints); returns the C status code."""
    return load_library().fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, workspace, workspace_bytes,
                   stream) -> int:
    """Split-KV forward on raw device pointers (ints); returns the C status code."""
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, workspace,
                                         workspace_bytes, stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, stream) -> int:
    """Split-KV forward with the library's own partial-state buffer (allocates nothing)."""
    return load_library().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits,
                                                 stream)


def fa_fwd_splitkv_plan(B, H, N, d, dtype, causal, num_splits):
    """Host-only plan of a split-KV call: (status, split columns, workspace bytes)."""
    ns, wb = ctypes.c_int(0), ctypes.c_size_t(0)
    st = load_library().fa_fwd_splitkv_plan(B, H, N, d, dtype, causal, num_splits, ctypes.byref(ns),
                                            ctypes.byref(wb))
    return st, ns.value, wb.value


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, stream) -> int:
    """bf16 backward on raw device pointers (ints); returns the C status code."""
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, stream)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
        return_lse: bool = True, stream=None):
    """Attention forward on torch tensors of shape [B, H, N, d] (bf16 or float32, on the GPU).

    Returns (o, lse) with o like q and lse float32 [B, H, N] (None if return_lse is False
    and no lse buffer is given). ``scale`` defaults to 1/sqrt(d). The work is enqueued on
    ``stream`` (default: torch's current stream) and is not waited for.
    """
    import torch

    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B,H,N,d] shape, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, H, N) or lse.dtype != torch.float32
                              or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B,H,N] tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            B, H, N, d, float(scale), 1 if causal else 0, handle)
    if st != FA_OK:
        raise FaError(st, fn.__name__)
    return out, lse


def fwd_splitkv(q, k, v, scale: float | None = None, causal: bool = False, num_splits: int = 0, workspace=None,
                stream=None):
    """Attention forward through the split-KV entry point (key range split over workgroups, then
    a merge). Same tensors and result as ``fwd``; returns (o, lse). The workspace (uint8 device
    tensor) is allocated with torch when not given; it must hold the bytes the plan reports."""
    import torch

    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B,H,N,d] shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dtype = FA_BF16 if q.dtype == torch.bfloat16 else FA_F32
    st, _, need = fa_fwd_splitkv_plan(B, H, N, d, dtype, 1 if causal else 0, num_splits)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv_plan")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                        float(scale), 1 if causal else 0, dtype, num_splits, ws_ptr, ws_bytes, handle)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv")
    return out, lse


def bwd(q, k, v, o, lse, dout, scale: float | None = None, causal: bool = False, stream=None):
    """Gradients (dq, dk, dv) of attention on bf16 torch tensors [B, H, N, d] (d = 64 or 128).

    ``o`` and ``lse`` are the forward's outputs for the same inputs, ``dout`` the gradient of
    the loss with respect to ``o``. Allocates the outputs and the fp32 [B, H, N] workspace with
    torch and enqueues the work on ``stream`` (default: the current stream) without waiting.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor shaped like q on q's device")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B,H,N] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, float(scale),
                1 if causal else 0, handle)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv
