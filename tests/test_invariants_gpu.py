"""Properties of the HIP path that hold exactly or by construction at any size, plus the
boundary's behaviour on a real device (streams, optional lse, untouched inputs, errors)."""
import math

import numpy as np
import pytest

import exact_softmax_attention_fa_amd as fa
from exact_softmax_attention_fa_amd import inputs
from gpu_util import note, run_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_first_row_is_v0(dtype):
    """Row 0 of a causal pass sees only key 0: weight exactly 1, so o_0 = v_0 bit for bit."""
    t = inputs.make_random(2, 3, 300, 128 if dtype == "bf16" else 64, dtype, seed=5)
    note(f"causal row 0 {dtype}")
    o, l = run_gpu(t, dtype, 0.1, True)
    v0 = to_device(t["v"], dtype).double().cpu().numpy()[:, :, 0]
    assert np.array_equal(o[:, :, 0], v0)
    q = to_device(t["q"], dtype).double().cpu().numpy()[:, :, 0]
    k = to_device(t["k"], dtype).double().cpu().numpy()[:, :, 0]
    assert np.allclose(l[:, :, 0], 0.1 * np.sum(q * k, axis=-1), atol=1e-4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_means(dtype, causal):
    """Q = 0: uniform weights over the visible keys; lse = ln(count)."""
    N, d = 517, 64
    t = inputs.make_random(1, 2, N, d, dtype, seed=6)
    t["q"] = np.zeros_like(t["q"])
    note(f"zero queries {dtype} causal={causal}")
    o, l = run_gpu(t, dtype, 0.125, causal)
    v = to_device(t["v"], dtype).double().cpu().numpy()
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    ref = (np.cumsum(v, axis=2) / counts[None, None, :, None]) if causal else \
        np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert np.abs(o - ref).max() <= (1e-5 if dtype == "f32" else 2e-2)
    assert np.abs(l - np.log(counts)[None, None, :]).max() <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_constant_values(dtype):
    """V = 1 everywhere: every output is 1 (the weights sum to 1)."""
    t = inputs.make_random(1, 2, 333, 128, dtype, seed=7, k_std=3.0)
    t["v"] = np.full_like(t["v"], 0x3F80 if dtype == "bf16" else 1.0)
    note(f"constant values {dtype}")
    o, _ = run_gpu(t, dtype, 1 / math.sqrt(128), False)
    assert np.abs(o - 1.0).max() <= (1e-5 if dtype == "f32" else 8e-3)


def test_repeated_runs_identical():
    import torch
    t = inputs.make_random(1, 4, 1000, 128, "bf16", seed=8)
    q, k, v = (to_device(t[x], "bf16") for x in "qkv")
    note("repeat determinism")
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_inputs_untouched_and_lse_optional():
    import torch
    t = inputs.make_random(2, 2, 190, 64, "bf16", seed=9)
    q, k, v = (to_device(t[x], "bf16") for x in "qkv")
    copies = [x.clone() for x in (q, k, v)]
    note("inputs untouched, lse optional")
    o_a, l_a = fa.fwd(q, k, v)
    o_b, l_b = fa.fwd(q, k, v, return_lse=False)
    torch.cuda.synchronize()
    assert l_b is None and torch.equal(o_a, o_b)
    assert all(torch.equal(a, b) for a, b in zip((q, k, v), copies))


def test_non_default_stream():
    import torch
    t = inputs.make_random(1, 2, 400, 128, "bf16", seed=10)
    q, k, v = (to_device(t[x], "bf16") for x in "qkv")
    note("side stream")
    ref, _ = fa.fwd(q, k, v)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, _ = fa.fwd(q, k, v, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(ref, out)


def test_errors_on_device():
    import torch
    q = torch.zeros((1, 1, 8, 320), dtype=torch.bfloat16, device="cuda")
    note("unsupported head width (above 256)")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q.clone(), q.clone())
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q.clone(), q.clone(), scale=float("nan"))
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    # output aliasing an input is rejected before launch
    st = fa.fa_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), None, 1, 1, 8, 64, 0.1, 0,
                   torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_INVALID_ARG
