"""Closed form of decode attention over the sentinel KV cache
(workload.kv_sentinel_cache), shared by the oracle pins and the GPU tests."""
import numpy as np

import workload

D = 128


def sentinel_closed_form(bits, T, Hq, Hkv):
    """o and B of the sentinel cache: zero keys give every token weight 1/T,
    so o[h, d] = (1/T) * sum over tokens of the (nonnegative) value in
    channel (h // (Hq/Hkv), d): 0.25 * KV_SENTINEL_CODE per token of each
    block marking that channel."""
    total = np.zeros((Hkv, D))
    for b in range(-(-T // workload.KV_BLOCK)):
        g, d = workload.kv_sentinel_channel(b, Hkv)
        n = min(T, (b + 1) * workload.KV_BLOCK) - b * workload.KV_BLOCK
        total[g, d] += n * 0.25 * workload.KV_SENTINEL_CODE
    o = total[np.arange(Hq) // (Hq // Hkv)] / T
    return o, o.copy()
