"""HIP path against the fp64 oracle, element by element, on seeded inputs.

Small and medium sizes are compared in full (they span several query and key tiles and
ragged tails); the full-size workloads are compared on sampled query rows of every
(b, h) that the oracle computes one by one."""
import math

import numpy as np
import pytest

from exact_softmax_attention_fa_amd import inputs
from gpu_util import bf16_peaky_tolerance, compare, fp32_row_tolerance, full_parity, note, run_gpu, sampled_parity
from oracle import attention as oracle

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


# ---- the five workloads -------------------------------------------------------------------

def test_fp32_single_head_full():
    w = W["fwd_f32_b1_h1_n256_d64"]
    full_parity(inputs.make(w), w.dtype, w.resolved_scale(), w.causal, w.name)


def test_bf16_b2_h8_n1024_full():
    w = W["fwd_bf16_b2_h8_n1024_d64"]
    full_parity(inputs.make(w), w.dtype, w.resolved_scale(), w.causal, w.name)


@pytest.mark.parametrize("name,rows", [
    ("fwd_bf16_b4_h16_n4096_d128_causal", 24),
    ("fwd_bf16_b1_h16_n8192_d128_widek", 64),
    ("fwd_bf16_b1_h8_n32768_d128_causal", 256),
])
def test_full_size_sampled_rows(name, rows):
    sampled_parity(W[name], rows, name)


@pytest.mark.parametrize("name", ["fwd_bf16_b4_h16_n4096_d128_causal", "fwd_bf16_b1_h16_n8192_d128_widek"])
def test_full_size_every_row(name):
    """The N = 4096 causal and the headline workloads compared with the oracle on every query
    row of every head (the oracle takes seconds to tens of seconds on the host)."""
    w = W[name]
    full_parity(inputs.make(w), w.dtype, w.resolved_scale(), w.causal, f"every row {name}")


def test_widek_small_full():
    """The boosted-key construction at a size the oracle covers in full (several tiles)."""
    w = inputs.Workload("widek_small", 1, 4, 1100, 128, "bf16", False, 2004,
                        k_std=3.0, boost_frac=0.01, boost_logit=8.0)
    full_parity(inputs.make(w), "bf16", w.resolved_scale(), False, w.name)


@pytest.mark.parametrize("causal", [False, True])
def test_causal_medium_full(causal):
    t = inputs.make_random(1, 3, 777, 128, "bf16", seed=31)
    full_parity(t, "bf16", 1 / math.sqrt(128), causal, f"n777 causal={causal}")


@pytest.mark.parametrize("d,H", [(64, 2), (64, 86), (128, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_late_keys_far_above_the_running_max(d, H, causal):
    """Keys whose logits lie far above every earlier score arrive in later tiles (a raise of
    the exponent reference after the first tile, twice, the second by 100 in natural units):
    every query that sees them puts its weight there. Logit offsets come from a constant last
    query coordinate, as in the boosted-key workload. d = 64 runs the generic kernel on 2 heads
    and the tuned one on 86 (258 tiles of 256 queries); d = 128 always runs the tuned one."""
    N, scale = 700, 1.0 / math.sqrt(d)
    t = inputs.make_random(1, H, N, d, "bf16", seed=77)
    q, k = t["q"].copy(), t["k"].copy()
    q[..., d - 1] = inputs.f32_to_bf16_bits(np.float32(1.0))
    k[..., d - 1] = 0
    for key, logit in ((210, 50.0), (610, 100.0)):
        k[:, :, key, d - 1] = inputs.f32_to_bf16_bits(np.float32(logit / scale))
    t = {"q": q, "k": k, "v": t["v"]}
    full_parity(t, "bf16", scale, causal, f"late spikes d{d} H{H} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("gap", [30.0, 40.0])
@pytest.mark.parametrize("d,H", [(128, 2), (64, 86)])
def test_large_gap_without_a_raise(d, H, gap, causal):
    """The tuned kernel (d = 128; d = 64 on 86 heads, 258 tiles of 256 queries): a key 30 or 40
    natural units above every score of the first tiles arrives in a later tile. The tuned kernel
    raises its exponent reference only when a tile's per-lane sum passes 2^64, so probabilities
    of about e^30 = 2^43 and e^40 = 2^58 flow through the bf16 probabilities and the fp32
    denominator and numerator without a raise."""
    N, scale = 700, 1.0 / math.sqrt(d)
    t = inputs.make_random(1, H, N, d, "bf16", seed=78)
    q, k = t["q"].copy(), t["k"].copy()
    q[..., d - 1] = inputs.f32_to_bf16_bits(np.float32(1.0))
    k[..., d - 1] = 0
    k[:, :, 333, d - 1] = inputs.f32_to_bf16_bits(np.float32(gap / scale))
    t = {"q": q, "k": k, "v": t["v"]}
    full_parity(t, "bf16", scale, causal, f"gap {gap} without a raise, d{d} H{H} causal={causal}")


def _sweep_case(i: int):
    """Seeded random case i: batch, heads, sequence length, head width, dtype, mask and scale."""
    rng = np.random.default_rng(7000 + i)
    dtype = "bf16" if i % 3 else "f32"
    d = int(rng.choice([64, 128, 64, 128, int(rng.integers(1, 257))]))
    N = int(rng.integers(1, 701))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    causal = bool(rng.integers(0, 2))
    scale = float(rng.choice([1.0 / math.sqrt(d), rng.uniform(-0.3, 0.3)]))
    return B, H, N, d, dtype, causal, scale


@pytest.mark.parametrize("i", range(24))
def test_random_shape_sweep(i):
    """24 seeded random shapes over every kernel (d up to 256, ragged N, both masks and dtypes,
    scales of either sign), each compared in full with the oracle."""
    B, H, N, d, dtype, causal, scale = _sweep_case(i)
    t = inputs.make_random(B, H, N, d, dtype, seed=8000 + i)
    label = f"sweep {i}: B{B} H{H} N{N} d{d} {dtype} causal={causal} scale={scale:.4f}"
    # fp32: a bound per query row from that row's own logits
    tol = fp32_row_tolerance(t, scale, causal) if dtype == "f32" else None
    full_parity(t, dtype, scale, causal, label, tol)


# ---- scalar examples through fp32 (d = 1, scale = 1) ----------------------------------------

def test_scalar_three_scores():
    t = inputs.scalar_case([0, 1, 2], [10, 20, 30])
    note("scalar three scores")
    o, l = run_gpu(t, "f32", 1.0, False)
    assert np.all(np.abs(o[0, 0, :, 0] - 25.752104) <= 1e-5), o.ravel()
    assert np.all(np.abs(l[0, 0] - math.log(1 + math.e + math.e ** 2)) <= 1e-5)


def test_scalar_shift_by_1000():
    t = inputs.scalar_case([1000, 1001, 1002], [10, 20, 30])
    note("scalar shift")
    o, l = run_gpu(t, "f32", 1.0, False)
    assert np.all(np.abs(o[0, 0, :, 0] - 25.752104) <= 1e-5), o.ravel()
    assert np.all(np.abs(l[0, 0] - (1000 + math.log(1 + math.e + math.e ** 2))) <= 1e-3)


def test_scalar_block_example():
    t = inputs.scalar_case([1, 2, 1001, 1002], [2, -1, 4, 8])
    note("scalar block example")
    o, l = run_gpu(t, "f32", 1.0, False)
    closed = (4 * math.exp(-1) + 8) / (math.exp(-1) + 1)
    assert np.all(np.abs(o[0, 0, :, 0] - closed) <= 1e-5), o.ravel()
    assert np.all(np.abs(l[0, 0] - (1002 + math.log(1 + math.exp(-1)))) <= 1e-3)


def test_scalar_causal_prefixes():
    """Causal on the block example: row i is the softmax-weighted sum of the first i+1 items."""
    s, v = [1, 2, 1001, 1002], [2, -1, 4, 8]
    t = inputs.scalar_case(s, v)
    note("scalar causal prefixes")
    o, _ = run_gpu(t, "f32", 1.0, True)
    from oracle import online
    for i in range(4):
        assert abs(o[0, 0, i, 0] - online.online_scalar(s[:i + 1], v[:i + 1])) <= 1e-5


# ---- shapes, tails and head widths ------------------------------------------------------------

SHAPES = [(1, 1, 1), (1, 2, 3), (2, 1, 63), (1, 2, 64), (1, 1, 65), (1, 2, 127), (1, 1, 129),
          (1, 1, 255), (2, 2, 257), (1, 1, 1000)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_shapes(B, H, N, d, causal):
    t = inputs.make_random(B, H, N, d, "bf16", seed=B * 1000 + H * 100 + N + d)
    full_parity(t, "bf16", 1 / math.sqrt(d), causal, f"bf16 B{B} H{H} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("d", [1, 8, 17, 40, 72, 96, 120])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_other_head_widths(d, causal):
    t = inputs.make_random(1, 2, 200, d, "bf16", seed=500 + d)
    full_parity(t, "bf16", 1 / math.sqrt(d), causal, f"bf16 d{d} causal={causal}")


@pytest.mark.parametrize("d", [1, 3, 33, 64, 100, 128])
@pytest.mark.parametrize("N", [1, 5, 64, 97, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_shapes(N, d, causal):
    t = inputs.make_random(1, 2, N, d, "f32", seed=700 + N + d)
    full_parity(t, "f32", 1 / math.sqrt(d), causal, f"f32 N{N} d{d} causal={causal}",
                fp32_row_tolerance(t, 1 / math.sqrt(d), causal))


@pytest.mark.parametrize("d", [129, 160, 200, 256])
@pytest.mark.parametrize("N", [33, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_wide_heads(d, N, causal):
    """Head widths above 128 run on the 256-wide kernel (masked loads below 256)."""
    t = inputs.make_random(1, 2, N, d, "bf16", seed=1100 + N + d)
    full_parity(t, "bf16", 1 / math.sqrt(d), causal, f"bf16 N{N} d{d} causal={causal}")


@pytest.mark.parametrize("d", [160, 256])
@pytest.mark.parametrize("N", [33, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_wide_heads(d, N, causal):
    t = inputs.make_random(1, 2, N, d, "f32", seed=1200 + N + d)
    full_parity(t, "f32", 1 / math.sqrt(d), causal, f"f32 N{N} d{d} causal={causal}",
                fp32_row_tolerance(t, 1 / math.sqrt(d), causal))


@pytest.mark.parametrize("dtype,d,N,BH", [("bf16", 64, 1000, 1), ("bf16", 40, 600, 2), ("bf16", 64, 300, 3),
                                          ("f32", 64, 256, 1), ("f32", 64, 100, 1), ("f32", 100, 200, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_key_split_groups(dtype, d, N, BH, causal):
    """Small grids split the key range over up to 4 groups of waves in a workgroup and merge
    their statistics (these shapes give splits of 2 and 4, with groups that see no key on the
    first causal query tiles and a ragged last tile)."""
    t = inputs.make_random(1, BH, N, d, dtype, seed=1300 + N + d + BH)
    tol = fp32_row_tolerance(t, 1 / math.sqrt(d), causal) if dtype == "f32" else None
    full_parity(t, dtype, 1 / math.sqrt(d), causal, f"{dtype} split N{N} d{d} BH{BH} causal={causal}", tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_other_scales(dtype, scale):
    """Negative, zero and large scales. At |scale| = 2.5 with d = 64 the logits are 20x
    larger than the workloads', so the fp32 bound 1e-5 (stated for scale = 1/sqrt(d)) is scaled by
    that factor of 20."""
    t = inputs.make_random(1, 2, 150, 64, dtype, seed=901)
    for causal in (False, True):
        tol = fp32_row_tolerance(t, scale, causal) if dtype == "f32" else None
        full_parity(t, dtype, scale, causal, f"{dtype} scale={scale} causal={causal}", tol)


@pytest.mark.parametrize("B,H,N,d", [(2, 64, 200, 64), (2, 64, 300, 48), (1, 128, 250, 64), (2, 64, 257, 17)])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_d64_wide_blocks(B, H, N, d, causal):
    """Grids of at least 256 workgroups of 128 queries run the 4-wave blocks at head widths up
    to 64 (many heads; ragged query and key tails, partial head widths, two or three query
    tiles per head). At width exactly 64 these grids stay below 256 tiles of 256 queries, where
    the tuned kernel would take over."""
    t = inputs.make_random(B, H, N, d, "bf16", seed=1400 + N + d + H)
    full_parity(t, "bf16", 1 / math.sqrt(d), causal, f"bf16 wide B{B} H{H} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("name", ["sweep_bf16_b1_h16_n8192_d32", "sweep_bf16_b1_h16_n8192_d64",
                                  "sweep_bf16_b1_h16_n8192_d96", "sweep_bf16_b1_h16_n8192_d256"])
def test_head_width_sweep_sampled_rows(name):
    """The other head widths at the headline's B, H and N (the 4-wave blocks at width 32, the
    tuned two-group kernel at exactly 64, the generic 128- and 256-wide blocks above), on
    sampled rows of every head."""
    sampled_parity(inputs.ALL_WORKLOADS[name], 32, name)


@pytest.mark.parametrize("B,H,N", [(4, 64, 256), (1, 128, 513)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [1 / 8, -0.3, 0.0, 2.5])
def test_bf16_d64_tuned(B, H, N, causal, scale):
    """Width exactly 64 with at least 256 tiles of 256 queries runs the tuned two-group kernel
    (its own key-row swizzle and DMA map): every output compared, a whole tile per head and a
    ragged one, at the workload scale and at negative, zero and large scales (2.5: logits 20x
    the workload's, so the reference is raised often). Above the workload scale the output
    bound is the one for peaky weights, 3 * 2^-8 * max|v| (bf16_peaky_tolerance)."""
    t = inputs.make_random(B, H, N, 64, "bf16", seed=1500 + N + H)
    tol = bf16_peaky_tolerance(t["v"]) if abs(scale) * 8 > 1 else None
    full_parity(t, "bf16", scale, causal, f"bf16 tuned d64 B{B} H{H} N{N} scale={scale} causal={causal}", tol)


@pytest.mark.parametrize("B,H,N", [(1, 256, 1), (1, 256, 33), (2, 128, 65), (1, 256, 130), (2, 128, 255),
                                   (1, 300, 65)])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_d64_tuned_short(B, H, N, causal):
    """The tuned d = 64 kernel on short sequences over at least 256 heads: items of one or two key
    tiles (N = 1, 33, 65, 130, 255), a ragged first tile, the final-phase slot for those tile
    counts, and (300 heads) resident workgroups running a second short item."""
    t = inputs.make_random(B, H, N, 64, "bf16", seed=1700 + N + H)
    full_parity(t, "bf16", 1 / 8, causal, f"bf16 tuned d64 short B{B} H{H} N{N} causal={causal}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("B,H,N", [(3, 40, 600), (2, 100, 300), (1, 130, 1000)])
@pytest.mark.parametrize("causal", [False, True])
def test_tuned_more_items_than_cus(d, B, H, N, causal):
    """Tuned-kernel grids (d = 128, and d = 64 at these sizes) with more (query tile, head)
    items than CUs, where each workgroup stays resident and runs a sequence of items; ragged N,
    so items of different lengths and ragged last tiles follow each other in one workgroup.
    Oracle on sampled rows of every head."""
    label = f"bf16 B{B} H{H} N{N} d{d} causal={causal} ({B * H * -(-N // 256)} items)"
    note(f"resident workgroups {label}")
    t = inputs.make_random(B, H, N, d, "bf16", seed=7000 + B * 100 + H + N + d)
    scale = 1 / math.sqrt(d)
    o, l = run_gpu(t, "bf16", scale, causal)
    rows = np.stack([np.stack([inputs.sample_rows(N, 16, seed=B * H * 10 + b * H + h)[:16] for h in range(H)])
                     for b in range(B)])
    o_ref, l_ref = oracle.attention_stored(t["q"], t["k"], t["v"], "bf16", scale, causal, rows=rows)
    ib = np.arange(B)[:, None, None]
    ih = np.arange(H)[None, :, None]
    compare(o[ib, ih, rows], l[ib, ih, rows], o_ref, l_ref, "bf16", label)
