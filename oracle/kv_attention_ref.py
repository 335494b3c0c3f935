"""Plain fp64 reference for decode attention over a quantised KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by the bench's CPU-baseline
leg; never by the product path.

What is computed, and where it comes from
-----------------------------------------
The core-modules page (section 5.4, memory manager: KV budget and loading
strategies) sizes the KV cache of an 8B model with grouped-query attention
(8 KV heads, head size 128, 32 layers) at 131,072 bytes per token in fp16 and
halves / quarters it with INT8 / INT4 values. Decode attention reads that
whole cache once per generated token, per layer: the other bandwidth-bound
operation of the decode step besides the weight GEMVs. The page does not
define the INT8/INT4 formats; the readings used here follow the weight codes
of this package (groups of 32 consecutive values with binary16 parameters):

* the cache of one layer holds keys and values k[t, g, d], v[t, g, d] for
  tokens t < T, KV heads g < Hkv and d < D = 128, quantised per
  (t, g, group of 32 consecutive d);
* INT8 (symmetric): value = s * q, q a signed 8-bit code, one binary16 scale s
  per group;
* INT4 (affine): value = s * q + m, q an unsigned 4-bit code (codes uint8
  [..., 64], low nibble = even d), a binary16 scale s and min m per group;
* query heads h < Hq share KV head g = h // (Hq / Hkv) (grouped-query
  attention);
* for each query head: score_t = (q_h . k_hat[t, g]) / sqrt(D),
  p = softmax(score) over t, o_h = sum_t p_t * v_hat[t, g].

The output is o [Hq, D] in fp64, with the tolerance scale
B[h, d] = sum_t p_t * |v_hat[t, g, d]|: a result o' passes when
|o' - o| <= 1e-3 * B + 1e-5 element by element (the weight GEMV's rule, with
the attention weights in the place of the activations).

fp64 is far more precise than the device's fp32 arithmetic: the dequantised
values and the products q*k are exact in fp64, the softmax and the sums are
correctly rounded to about 1e-15 relative.

Parity status: the pages print no attention values. The pins are
hand-derived cases (uniform attention, a single token), a pure-Python
re-implementation on tiny shapes, special cases that reduce to the pinned
codec oracle's dequantisation, and invariances (token permutation, grouped
heads, a constant added to every score).
"""
from __future__ import annotations

import numpy as np

D = 128
GROUP = 32
BITS = (8, 4)


def dequantise_cache(bits: int, codes, scale, mn=None) -> np.ndarray:
    """Codes of one cache tensor -> fp64 values [T, Hkv, D].

    bits = 8: codes int8 [T, Hkv, D], scale binary16 [T, Hkv, D/32].
    bits = 4: codes uint8 [T, Hkv, D/2] (low nibble = even d), scale and min
    binary16 [T, Hkv, D/32].
    """
    codes = np.asarray(codes)
    s = np.repeat(np.asarray(scale).astype(np.float64), GROUP, axis=-1)
    if bits == 8:
        if codes.dtype != np.int8 or codes.shape[-1] != D:
            raise TypeError("INT8 codes must be int8 [T, Hkv, 128]")
        return s * codes.astype(np.float64)
    if bits == 4:
        if codes.dtype != np.uint8 or codes.shape[-1] != D // 2:
            raise TypeError("INT4 codes must be uint8 [T, Hkv, 64]")
        q = np.empty(codes.shape[:-1] + (D,), dtype=np.float64)
        q[..., 0::2] = codes & 0x0F
        q[..., 1::2] = codes >> 4
        return s * q + np.repeat(np.asarray(mn).astype(np.float64), GROUP, axis=-1)
    raise ValueError("bits must be 8 or 4")


def attention(bits: int, q, k_codes, k_scale, k_min, v_codes, v_scale, v_min, heads=None):
    """(o, B) in fp64, both [len(heads), D], for the query heads `heads`
    (default: all Hq) of one layer.

    q: binary16 [Hq, D]. The cache tensors are in the layout of
    dequantise_cache; k_min / v_min are ignored for INT8.
    """
    q = np.asarray(q)
    Hq = q.shape[0]
    k = dequantise_cache(bits, k_codes, k_scale, k_min)
    v = dequantise_cache(bits, v_codes, v_scale, v_min)
    T, Hkv, _ = k.shape
    if T < 1 or Hq % Hkv or q.shape[1] != D:
        raise ValueError("need T >= 1, Hq a multiple of Hkv and q [Hq, 128]")
    G = Hq // Hkv
    heads = range(Hq) if heads is None else heads
    o = np.empty((len(heads), D))
    B = np.empty((len(heads), D))
    for i, h in enumerate(heads):
        g = h // G
        score = (k[:, g, :] @ q[h].astype(np.float64)) / np.sqrt(D)
        e = np.exp(score - score.max())
        p = e / e.sum()
        o[i] = p @ v[:, g, :]
        B[i] = p @ np.abs(v[:, g, :])
    return o, B


def tolerance(B):
    return 1e-3 * np.asarray(B) + 1e-5


def within_tolerance(o_test, o_ref, B):
    return np.abs(np.asarray(o_test, dtype=np.float64) - o_ref) <= tolerance(B)
