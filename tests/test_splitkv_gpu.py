"""Split-KV forward (the key range split over workgroups, partial states merged by a second
kernel) against the fp64 oracle, element by element, through the C-ABI.

Split counts 1/2/4/8, ragged key and query tails, both masks, both dtypes and several head
widths; the fp32 single-head workload and a long single head with the library's own split
choice; keys far above the running maximum that land in one column only (the merge then weighs
columns whose references differ by up to 2^144); and a workspace reused by a second, smaller
call."""
import math

import numpy as np
import pytest

from exact_softmax_attention_fa_amd import inputs
from gpu_util import compare, note, to_device
from oracle import attention as oracle

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def run_split(t, dtype, scale, causal, num_splits, workspace=None):
    import torch
    import exact_softmax_attention_fa_amd as fa
    q, k, v = (to_device(t[x], dtype) for x in "qkv")
    o, l = fa.fwd_splitkv(q, k, v, scale=scale, causal=causal, num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), l.double().cpu().numpy()


def split_parity(t, dtype, scale, causal, num_splits, label, workspace=None):
    note(f"split-KV parity {label}")
    o, l = run_split(t, dtype, scale, causal, num_splits, workspace)
    o_ref, l_ref = oracle.attention_stored(t["q"], t["k"], t["v"], dtype, scale, causal)
    return compare(o, l, o_ref, l_ref, dtype, label)


def plan(t, dtype, causal, num_splits):
    import exact_softmax_attention_fa_amd as fa
    B, H, N, d = t["q"].shape
    st, ns, wb = fa.fa_fwd_splitkv_plan(B, H, N, d, fa.FA_BF16 if dtype == "bf16" else fa.FA_F32,
                                        1 if causal else 0, num_splits)
    assert st == fa.FA_OK
    return ns, wb


@pytest.mark.parametrize("N,d", [(256, 64), (300, 128), (517, 96), (200, 256), (301, 41), (150, 200)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ns", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_counts(dtype, ns, causal, N, d):
    t = inputs.make_random(1, 2, N, d, dtype, seed=900 + N + d + ns)
    got = plan(t, dtype, causal, ns)[0]
    assert 1 <= got <= ns
    split_parity(t, dtype, 1.0 / math.sqrt(d), causal, ns, f"{dtype} N{N} d{d} causal={causal} splits={ns}->{got}")


def test_fp32_single_head_workload_split():
    """The fp32 single-head workload (8 query tiles) in 8 columns of one key tile each (its 256
    keys are too few for the library's own choice to split them)."""
    w = W["fwd_f32_b1_h1_n256_d64"]
    t = inputs.make(w)
    assert plan(t, w.dtype, w.causal, 0)[0] == 1
    assert plan(t, w.dtype, w.causal, 8)[0] == 8
    split_parity(t, w.dtype, w.resolved_scale(), w.causal, 8, f"{w.name} 8 columns")


@pytest.mark.parametrize("causal", [False, True])
def test_long_single_head_default_split(causal):
    """One head of the headline shape (N = 8192, d = 128, wide-spread keys with boosted logits):
    32 query tiles, the default split gives 8 columns of 16 key tiles."""
    w = inputs.Workload("one_head_widek", 1, 1, 8192, 128, "bf16", causal, 3004,
                        k_std=3.0, boost_frac=0.01, boost_logit=8.0)
    t = inputs.make(w)
    assert plan(t, "bf16", causal, 0)[0] == 8
    split_parity(t, "bf16", w.resolved_scale(), causal, 0, f"N8192 d128 one head causal={causal} default split")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_spikes_in_one_column(dtype, causal):
    """Two keys far above every other score, in the third and fifth of 8 columns: the columns'
    references differ by up to 144 natural units, the merge must give the rest weight ~0."""
    N, d = 512, 64
    scale = 1.0 / math.sqrt(d)
    t = inputs.make_random(1, 2, N, d, dtype, seed=4242)
    q, k = t["q"].copy(), t["k"].copy()
    one = inputs.f32_to_bf16_bits(np.float32(1.0)) if dtype == "bf16" else np.float32(1.0)
    q[..., d - 1] = one
    k[..., d - 1] = 0
    for key, logit in ((140, 50.0), (300, 100.0)):
        val = np.float32(logit / scale)
        k[:, :, key, d - 1] = inputs.f32_to_bf16_bits(val) if dtype == "bf16" else val
    t = {"q": q, "k": k, "v": t["v"]}
    split_parity(t, dtype, scale, causal, 8, f"spikes {dtype} causal={causal}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_other_scales(scale):
    t = inputs.make_random(2, 1, 333, 64, "bf16", seed=515)
    split_parity(t, "bf16", scale, True, 4, f"scale {scale}")


def test_workspace_reused_by_a_smaller_call():
    """Two calls in a row on one workspace, the second smaller: each matches the oracle."""
    import torch
    t1 = inputs.make_random(1, 3, 640, 128, "bf16", seed=61)
    t2 = inputs.make_random(1, 1, 200, 64, "bf16", seed=62)
    need = plan(t1, "bf16", False, 8)[1]
    assert need >= plan(t2, "bf16", True, 4)[1] > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    split_parity(t1, "bf16", 1 / math.sqrt(128), False, 8, "first call", workspace=ws)
    split_parity(t2, "bf16", 1 / math.sqrt(64), True, 4, "second, smaller call", workspace=ws)
