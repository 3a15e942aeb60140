"""The C-ABI entry points captured in a HIP graph (torch.cuda.graph): the library launches only
kernels on the caller's stream (no allocation, copy or fill), so a captured forward and backward
pass replays to the same results as the eager calls. Every replay runs after eager work and a
synchronisation of its own, and is compared with the eager results bit for bit."""
import math

import numpy as np
import pytest

import exact_softmax_attention_fa_amd as fa
from exact_softmax_attention_fa_amd import inputs
from gpu_util import note, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_backward_replayed_from_a_graph(causal):
    import torch

    B, H, N, d = 1, 2, 300, 128
    scale = 1.0 / math.sqrt(d)
    t = inputs.make_backward(B, H, N, d, seed=4242)
    q, k, v, dout = (to_device(t[x], "bf16") for x in ("q", "k", "v", "dout"))
    note(f"graph capture fa_fwd + fa_bwd B{B} H{H} N{N} d{d} causal={causal}")

    o_ref, lse_ref = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq_ref, dk_ref, dv_ref = fa.bwd(q, k, v, o_ref, lse_ref, dout, scale=scale, causal=causal)
    torch.cuda.synchronize()

    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    delta = torch.empty_like(lse)
    flag = 1 if causal else 0
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        handle = torch.cuda.current_stream().cuda_stream
        st_f = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, N, d, scale, flag, handle)
        st_b = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                         lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                         B, H, N, d, scale, flag, handle)
    assert st_f == fa.FA_OK and st_b == fa.FA_OK

    for rep in range(4):
        # eager work between replays: other calls of the library and torch fills of the outputs
        other, _ = fa.fwd(k, q, v, scale=scale, causal=not causal)
        for x in (o, lse, dq, dk, dv, delta):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in (("o", o, o_ref), ("lse", lse, lse_ref), ("dq", dq, dq_ref),
                               ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"
        assert np.isfinite(other.float().cpu().numpy()).all()
