"""fa_fwd_splitkv_noalloc (partial states in the library's own per-GPU buffer) against
fa_fwd_splitkv with a caller workspace, through the C-ABI: two calls in a row, the second on a
smaller input, each equal to the workspace entry point's output bit for bit (same kernels, same
inputs) and within the oracle's tolerances; and the size limit rejected on the host."""
import math

import numpy as np
import pytest

from exact_softmax_attention_fa_amd import inputs
from gpu_util import compare, note, to_device
from oracle import attention as oracle

pytestmark = pytest.mark.gpu


def _call_both(t, dtype, scale, causal, num_splits):
    import torch
    import exact_softmax_attention_fa_amd as fa
    q, k, v = (to_device(t[x], dtype) for x in "qkv")
    B, H, N, d = q.shape
    code = fa.FA_BF16 if dtype == "bf16" else fa.FA_F32
    st, ns, need = fa.fa_fwd_splitkv_plan(B, H, N, d, code, int(causal), num_splits)
    assert st == fa.FA_OK and ns > 1 and 0 < need <= fa.FA_NOALLOC_SCRATCH_BYTES
    stream = torch.cuda.current_stream()
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws, l_ws = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    o_na, l_na = torch.full_like(q, 7.0), torch.full((B, H, N), 7.0, dtype=torch.float32, device="cuda")
    args = (B, H, N, d, float(scale), int(causal), code, num_splits)
    assert fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ws.data_ptr(), l_ws.data_ptr(), *args,
                             ws.data_ptr(), need, stream.cuda_stream) == fa.FA_OK
    assert fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_na.data_ptr(), l_na.data_ptr(),
                                     *args, stream.cuda_stream) == fa.FA_OK
    torch.cuda.synchronize()
    return ns, (o_ws.double().cpu().numpy(), l_ws.double().cpu().numpy()), \
        (o_na.double().cpu().numpy(), l_na.double().cpu().numpy())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    cases = [(2, 3, 1000, 128, True, 8), (1, 1, 300, 64, False, 4)]   # second call smaller
    for i, (B, H, N, d, causal, ns_req) in enumerate(cases):
        label = f"noalloc call {i + 1} {dtype} B{B} H{H} N{N} d{d} causal={causal} splits={ns_req}"
        note(label)
        t = inputs.make_random(B, H, N, d, dtype, seed=700 + i)
        scale = 1.0 / math.sqrt(d)
        ns, (o_ws, l_ws), (o_na, l_na) = _call_both(t, dtype, scale, causal, ns_req)
        assert np.array_equal(o_na, o_ws), f"{label}: output differs from fa_fwd_splitkv"
        assert np.array_equal(l_na, l_ws), f"{label}: lse differs from fa_fwd_splitkv"
        o_ref, l_ref = oracle.attention_stored(t["q"], t["k"], t["v"], dtype, scale, causal)
        compare(o_na, l_na, o_ref, l_ref, dtype, label)


def test_noalloc_rejects_plans_beyond_its_buffer():
    """A plan needing more than the fixed buffer returns FA_ERR_SCRATCH before any launch (the
    pointers are never touched)."""
    import exact_softmax_attention_fa_amd as fa
    B, H, N, d = 1, 4, 65536, 128
    st, ns, need = fa.fa_fwd_splitkv_plan(B, H, N, d, fa.FA_BF16, 0, 64)
    assert st == fa.FA_OK and need > fa.FA_NOALLOC_SCRATCH_BYTES
    big = 1 << 40
    st = fa.fa_fwd_splitkv_noalloc(big, 2 * big, 3 * big, 4 * big, 5 * big, B, H, N, d, 0.088, 0, fa.FA_BF16, 64,
                                   None)
    assert st == fa.FA_ERR_SCRATCH
    assert "64 MiB" in fa.fa_status_string(st)
