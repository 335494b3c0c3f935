"""The allocation-free entry point w4a16_kv_attention_static, through the C
ABI, against w4a16_kv_attention (the same kernels with a caller workspace) on
the same inputs: two calls in a row, the second on a smaller input, so the
second reuses the library's partials array after a larger call. Both must
agree bit for bit, and each meets the oracle's tolerance."""
import numpy as np
import pytest

import bit_weight_quantized_w4a16_amd as w4
import oracle
import workload

torch = pytest.importorskip("torch")

DEV = "cuda:0"
A = oracle.kv_attention_ref


def test_static_workspace_limits(w4a16_lib):
    """Host-side refusals: nothing is enqueued, no device is touched."""
    L = w4.lib()
    B = 0x7F0000000000
    assert L.w4a16_kv_attention_static(8, None, B, B + 2**20, 64, 32, 8, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_kv_attention_static(6, B, B + 2**24, B + 2**30, 64, 32, 8, None) == w4.W4A16_ERR_SHAPE
    assert w4.w4a16_kv_workspace_bytes(129024, 32) <= w4.W4A16_KV_STATIC_WORKSPACE_BYTES
    assert w4.w4a16_kv_workspace_bytes(129025, 32) > w4.W4A16_KV_STATIC_WORKSPACE_BYTES
    assert L.w4a16_kv_attention_static(8, B, B + 2**24, B + 2**30, 129025, 32, 8, None) == w4.W4A16_ERR_SIZE


def _both(bits, T, Hq, Hkv, seed):
    cache = workload.kv_cache(bits, seed, 0, T, Hkv)
    q = workload.kv_query(seed, 0, Hq)
    kv = w4.upload_packed(w4.w4a16_kv_pack(bits, *cache), DEV)
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    o_static = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    o_ws = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(w4.w4a16_kv_workspace_bytes(T, Hq) // 4, dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    print(f"[no-alloc] bits={bits} T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    st = w4.w4a16_kv_attention_static_raw(bits, qd.data_ptr(), kv.data_ptr(), o_static.data_ptr(), T, Hq, Hkv, s)
    assert st == w4.W4A16_OK, w4.w4a16_status_string(st)
    st = w4.w4a16_kv_attention_raw(bits, qd.data_ptr(), kv.data_ptr(), o_ws.data_ptr(), T, Hq, Hkv, ws.data_ptr(),
                                   ws.numel() * 4, s)
    assert st == w4.W4A16_OK, w4.w4a16_status_string(st)
    torch.cuda.synchronize()
    a = o_static.cpu().numpy().astype(np.float64)
    b = o_ws.cpu().numpy().astype(np.float64)
    o_ref, B = A.attention(bits, q, *cache)
    for o, label in ((a, "static"), (b, "workspace")):
        ok = A.within_tolerance(o, o_ref, B)
        assert ok.all(), f"{label}: {int((~ok).sum())} of {ok.size} outside tolerance"
    assert np.array_equal(a, b), f"max |static - workspace| = {np.abs(a - b).max()}"


@pytest.mark.gpu
def test_static_matches_workspace_entry_point_two_calls(w4a16_lib):
    # the 8B INT4 context of the KV budget (the larger call), then a smaller INT8 one
    _both(4, workload.KV_CONTEXT[4], 32, 8, 91)
    _both(8, 1000, 16, 8, 92)
