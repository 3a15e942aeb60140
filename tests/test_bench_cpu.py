"""Host-side checks of bench.py: the one-GPU contract, the work counts of each workload, the
kernel-source keys of the stored HBM traffic, and the CPU oracle leg on a tiny sample."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_softmax_attention_fa_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


# 4*B*H*N^2*d (halved when causal) and q, k, v read + o written once + 4-byte lse per row,
# computed by hand for each workload's sizes
EXPECTED = {
    "fwd_f32_b1_h1_n256_d64": (4 * 1 * 1 * 256 ** 2 * 64, 4 * 1 * 1 * 256 * 64 * 4 + 4 * 256),
    "fwd_bf16_b2_h8_n1024_d64": (4 * 2 * 8 * 1024 ** 2 * 64, 4 * 2 * 8 * 1024 * 64 * 2 + 4 * 2 * 8 * 1024),
    "fwd_bf16_b4_h16_n4096_d128_causal": (2 * 4 * 16 * 4096 ** 2 * 128,
                                          4 * 4 * 16 * 4096 * 128 * 2 + 4 * 4 * 16 * 4096),
    "fwd_bf16_b1_h16_n8192_d128_widek": (4 * 1 * 16 * 8192 ** 2 * 128,
                                         4 * 1 * 16 * 8192 * 128 * 2 + 4 * 16 * 8192),
    "fwd_bf16_b1_h8_n32768_d128_causal": (2 * 1 * 8 * 32768 ** 2 * 128,
                                          4 * 1 * 8 * 32768 * 128 * 2 + 4 * 8 * 32768),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_work_counts(name):
    w = inputs.WORKLOADS[name]
    flops, nbytes = EXPECTED[name]
    assert w.flops == flops
    assert w.algorithmic_bytes == nbytes


def test_headline_is_the_metric_workload():
    w = inputs.WORKLOADS[inputs.HEADLINE]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal) == (1, 16, 8192, 128, "bf16", False)


@pytest.mark.parametrize("name", sorted(inputs.WORKLOADS))
def test_kernel_sources_exist_and_hash(name):
    w = inputs.WORKLOADS[name]
    for rel in bench.kernel_sources(w):
        assert os.path.isfile(os.path.join(ROOT, rel)), rel
    h = bench.kernel_hash(w)
    assert len(h) == 16 and int(h, 16) >= 0


def test_stored_traffic_is_keyed_by_workload_and_kernel():
    for name, entry in bench.TRAFFIC.items():
        assert name in inputs.WORKLOADS
        assert entry["bytes"] > inputs.WORKLOADS[name].algorithmic_bytes // 2
        assert len(entry["kernel_hash"]) == 16


def test_cpu_baseline_leg_runs_the_oracle_on_a_sample():
    w = inputs.WORKLOADS["fwd_bf16_b2_h8_n1024_d64"]
    t = inputs.make(w)
    res = bench.cpu_baseline(w, t, rows_per_head=4)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s"
    assert res["value"] > 0 and res["cores"] >= 1
    assert "4 of 1024 query rows" in res["sample"]
