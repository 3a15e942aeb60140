"""Backward pass on the GPU (fa_bwd through the C-ABI) against the fp64 oracle's gradients.

Inputs q, k, v, dout are seeded bf16 draws. The forward outputs o and lse that fa_bwd takes
come either from the oracle (rounded to the storage formats: o to bf16, lse to fp32) or
from fa_fwd itself (the end-to-end use); the oracle's gradients are always computed from
q, k, v, dout alone."""
import math

import numpy as np
import pytest

from exact_softmax_attention_fa_amd import inputs
from gpu_util import note, to_device
from oracle import attention as oracle
from oracle import backward as oracle_bwd

pytestmark = pytest.mark.gpu

# Tolerance per gradient tensor g (derived in the design notes from the bf16 roundings of o,
# P and dS): max |g_gpu - g_ref| <= 2^-6 * max(1, max |g_ref|) and
# mean |g_gpu - g_ref| <= 2^-9 * max(1, max |g_ref|).
def check(g_gpu, g_ref, label):
    scale = max(1.0, float(np.abs(g_ref).max()))
    err = np.abs(g_gpu - g_ref)
    assert np.all(np.isfinite(g_gpu)), f"{label}: non-finite gradient"
    mx, mn = float(err.max()) / scale, float(err.mean()) / scale
    assert mx <= 2.0 ** -6, f"{label}: max abs error {mx:.3e} x {scale:.3g} above 2^-6"
    assert mn <= 2.0 ** -9, f"{label}: mean abs error {mn:.3e} x {scale:.3g} above 2^-9"
    return mx, mn


def run_case(B, H, N, d, causal, seed, scale=None, forward="oracle"):
    import torch
    import exact_softmax_attention_fa_amd as fa
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    t = inputs.make_backward(B, H, N, d, seed)
    q64, k64, v64, do64 = (oracle.as_fp64(t[x], "bf16") for x in ("q", "k", "v", "dout"))
    dq_r, dk_r, dv_r = oracle_bwd.gradients(q64, k64, v64, do64, scale, causal)
    q, k, v, dout = (to_device(t[x], "bf16") for x in ("q", "k", "v", "dout"))
    note(f"backward B{B} H{H} N{N} d{d} causal={causal} scale={scale:.4g} forward={forward}")
    if forward == "oracle":
        o_ref, lse_ref = oracle.attention(q64, k64, v64, scale, causal)
        o = to_device(inputs.f32_to_bf16_bits(o_ref.astype(np.float32)), "bf16")
        lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    else:
        o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dout, scale=scale, causal=causal)
    torch.cuda.synchronize()
    out = {}
    for name, g, r in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        out[name] = check(g.double().cpu().numpy(), r, f"{name} B{B} H{H} N{N} d{d} causal={causal}")
    return out


SHAPES = [(1, 1, 1), (1, 2, 31), (2, 1, 64), (1, 1, 100), (1, 2, 129), (1, 1, 257)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_shapes(B, H, N, d, causal):
    run_case(B, H, N, d, causal, seed=2000 + B * 100 + H * 10 + N + d)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_end_to_end(causal):
    """fa_fwd's own o and lse feed fa_bwd."""
    run_case(2, 2, 300, 128, causal, seed=2500, forward="gpu")
    run_case(1, 3, 200, 64, causal, seed=2501, forward="gpu")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.35])
def test_backward_scales(scale):
    run_case(1, 2, 96, 64, False, seed=2600, scale=scale)
    run_case(1, 1, 96, 128, True, seed=2601, scale=scale)


def test_backward_medium():
    """Several key blocks and query blocks, both masks, end to end."""
    run_case(1, 4, 1024, 128, True, seed=2700, forward="gpu")
    run_case(1, 2, 1024, 64, False, seed=2701, forward="gpu")


@pytest.mark.parametrize("d,N,causal", [(64, 77, False), (128, 300, True)])
def test_backward_delta_workspace(d, N, causal):
    """The delta workspace fa_bwd writes holds sum_c dO_ic O_ic per row (fp32 sum of exact
    bf16 products: error at most a few units of 2^-24 times sum_c |dO_ic O_ic| per term)."""
    import torch
    import exact_softmax_attention_fa_amd as fa
    B, H, seed = 2, 3, 2800 + d + N
    scale = 1.0 / math.sqrt(d)
    t = inputs.make_backward(B, H, N, d, seed)
    q, k, v, dout = (to_device(t[x], "bf16") for x in ("q", "k", "v", "dout"))
    note(f"backward delta B{B} H{H} N{N} d{d} causal={causal}")
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, scale,
                   1 if causal else 0, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    o64 = o.double().cpu().numpy()
    do64 = oracle.as_fp64(t["dout"], "bf16")
    ref = oracle_bwd.delta(o64, do64)
    bound = 2.0 ** -16 * np.abs(o64 * do64).sum(axis=-1) + 1e-30
    got = delta.double().cpu().numpy()
    assert np.all(np.isfinite(got)), "delta rows left unwritten"
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


@pytest.mark.parametrize("B,H,N,causal", [(1, 16, 8192, False), (4, 16, 4096, True)])
def test_backward_full_size_sampled(B, H, N, causal):
    """The backward pass at the headline shape and at the N = 4096 causal shape (d = 128), on
    fa_fwd's own o and lse, against the oracle on sampled query rows of dQ and sampled keys of
    dK and dV (tile edges, the middle, the last row and seeded rows), which the oracle computes
    row by row and column by column."""
    import torch
    import exact_softmax_attention_fa_amd as fa
    d = 128
    scale = 1.0 / math.sqrt(d)
    t = inputs.make_backward(B, H, N, d, seed=9100 + N)
    q, k, v, dout = (to_device(t[x], "bf16") for x in ("q", "k", "v", "dout"))
    note(f"backward full size B{B} H{H} N{N} d{d} causal={causal}")
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dout, scale=scale, causal=causal)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(N, 24, seed=9200 + N)
    q64, k64, v64, do64 = (oracle.as_fp64(t[x], "bf16") for x in ("q", "k", "v", "dout"))
    sq, sk, sv = oracle_bwd.gradients_sampled(q64, k64, v64, do64, scale, causal, rows, rows)
    for name, g, r in (("dq", dq, sq), ("dk", dk, sk), ("dv", dv, sv)):
        check(g[:, :, rows].double().cpu().numpy(), r, f"{name} full size B{B} H{H} N{N} causal={causal}")
