"""The unfused comparison that bench.py times (scores and probabilities written to device
memory as N x N matrices, library GEMMs and a softmax) meets the oracle's tolerances, so its
timings compare two correct implementations. Outputs only (it computes no log-normaliser)."""
import math

import numpy as np
import pytest

import bench
from exact_softmax_attention_fa_amd import inputs
from gpu_util import compare, note, to_device
from oracle import attention as oracle

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def run_naive(t, dtype, scale, causal):
    import torch
    q, k, v = (to_device(t[x], dtype) for x in "qkv")
    N = q.shape[2]
    kt = k.transpose(-1, -2).contiguous()
    mask = torch.ones(N, N, dtype=torch.bool, device=q.device).triu_(1) if causal else None
    o = bench.naive_attention(q, kt, v, scale, causal, mask)
    torch.cuda.synchronize()
    return o.double().cpu().numpy()


@pytest.mark.parametrize("name", ["fwd_f32_b1_h1_n256_d64", "fwd_bf16_b2_h8_n1024_d64"])
def test_naive_small_workloads_full(name):
    w = W[name]
    note(f"naive comparison {name}")
    t = inputs.make(w)
    o = run_naive(t, w.dtype, w.resolved_scale(), w.causal)
    o_ref, _ = oracle.attention_stored(t["q"], t["k"], t["v"], w.dtype, w.resolved_scale(), w.causal)
    compare(o, None, o_ref, None, w.dtype, f"naive {name}")


@pytest.mark.parametrize("causal", [False, True])
def test_naive_wide_keys_full(causal):
    """The boosted wide-spread keys of the headline workload at a size the oracle covers in full:
    the scores must stay fp32 (rounding them to bf16 moves the output by ~0.1)."""
    w = inputs.Workload("widek_small", 1, 4, 1100, 128, "bf16", causal, 2004,
                        k_std=3.0, boost_frac=0.01, boost_logit=8.0)
    note(f"naive comparison wide keys causal={causal}")
    t = inputs.make(w)
    o = run_naive(t, "bf16", w.resolved_scale(), causal)
    o_ref, _ = oracle.attention_stored(t["q"], t["k"], t["v"], "bf16", w.resolved_scale(), causal)
    compare(o, None, o_ref, None, "bf16", f"naive wide keys causal={causal}")


def test_naive_headline_sampled_rows():
    w = W[inputs.HEADLINE]
    note("naive comparison headline, sampled rows")
    t = inputs.make(w)
    o = run_naive(t, w.dtype, w.resolved_scale(), w.causal)
    rows = np.stack([np.stack([inputs.sample_rows(w.N, 32, seed=w.seed * 100 + b * w.H + h)[:32]
                               for h in range(w.H)]) for b in range(w.B)])
    o_ref, _ = oracle.attention_stored(t["q"], t["k"], t["v"], w.dtype, w.resolved_scale(), w.causal, rows=rows)
    idx_b = np.arange(w.B)[:, None, None]
    idx_h = np.arange(w.H)[None, :, None]
    compare(o[idx_b, idx_h, rows], None, o_ref, None, w.dtype, "naive headline sampled rows")
