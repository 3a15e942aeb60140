"""Seeded input generators: storage rounding, determinism, workload structure."""
import math

import numpy as np
import torch

from exact_softmax_attention_fa_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 7,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 3.0e38], dtype=np.float32)])
    mine = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert inputs.f32_to_bf16_bits(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert inputs.f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def test_workloads_shapes_and_seeds():
    w = inputs.WORKLOADS["fwd_f32_b1_h1_n256_d64"]
    a, b = inputs.make(w), inputs.make(w)
    assert a["q"].dtype == np.float32 and a["q"].shape == (1, 1, 256, 64)
    assert all(np.array_equal(a[x], b[x]) for x in "qkv")
    w2 = inputs.WORKLOADS["fwd_bf16_b2_h8_n1024_d64"]
    c = inputs.make(w2)
    assert c["k"].dtype == np.uint16 and c["k"].shape == (2, 8, 1024, 64)
    assert not np.array_equal(c["q"], c["k"])


def test_boosted_keys_structure():
    w = inputs.Workload("boost", 1, 3, 500, 32, "bf16", False, 77, k_std=3.0, boost_frac=0.01, boost_logit=8.0)
    t = inputs.make(w)
    qlast = t["q"][..., -1]
    klast = t["k"][..., -1]
    assert np.all(qlast == 0x3F80)  # 1.0
    coord = inputs.f32_to_bf16_bits(np.array([8.0 * math.sqrt(32)], np.float32))[0]
    for h in range(3):
        boosted = np.flatnonzero(klast[0, h] != 0)
        assert len(boosted) == math.ceil(0.01 * 500)
        assert np.all(klast[0, h, boosted] == coord)


def test_flop_and_byte_counts():
    w = inputs.WORKLOADS[inputs.HEADLINE]
    assert w.flops == 4 * 16 * 8192 ** 2 * 128
    assert w.algorithmic_bytes == 4 * 16 * 8192 * 128 * 2 + 4 * 16 * 8192
    wc = inputs.WORKLOADS["fwd_bf16_b1_h8_n32768_d128_causal"]
    assert wc.flops == 2 * 8 * 32768 ** 2 * 128


def test_scalar_case_and_sampled_rows():
    s = inputs.scalar_case([0, 1, 2], [10, 20, 30])
    assert s["k"].shape == (1, 1, 3, 1) and np.all(s["q"] == 1)
    r = inputs.sample_rows(8192, 64, seed=3)
    assert r[0] == 0 and r[-1] == 8191 and len(np.unique(r)) == len(r)
    assert {63, 64, 127, 128, 4096}.issubset(set(r.tolist()))
