"""Pins for the fp64 oracle of decode attention over a quantised KV cache.

Independent of the oracle's own formula, and chosen so that a plausible slip
fails one of them (a wrong query-head -> KV-head mapping, a missing 1/sqrt(D),
swapped nibbles, unnormalised weights, a wrong tolerance scale):

* a pure-Python re-implementation (integer code decoding, math.exp, fsum) on
  tiny shapes;
* closed forms: one token gives o = v_hat exactly; all-zero INT8 keys give
  scores of exactly 0, hence uniform weights and o = the mean of v_hat;
* the dequantisation reduces to the pinned codec oracle (INT8 = symmetric
  8-bit code, INT4 = the 4-bit group-affine code, on the same bytes);
* invariances: permuting the tokens, and a grouped head equals a single-head
  problem on its own KV head;
* a dominant token: a key aligned with the query at a large scale takes the
  whole weight.
"""
import math

import numpy as np
import pytest

import oracle
import workload

A = oracle.kv_attention_ref
D = 128


def _problem(bits, T, Hq, Hkv, seed=0):
    cache = workload.kv_cache(bits, 500 + seed, 0, T, Hkv)
    q = workload.kv_query(500 + seed, 0, Hq)
    return q, cache


def _value(bits, codes, scale, mn, t, g, d):
    """One cache value, decoded with integer arithmetic."""
    if bits == 8:
        b = int(np.asarray(codes[t, g, d]).view(np.uint8))
        c = b - 256 if b >= 128 else b
        return float(scale[t, g, d // 32]) * c
    hi, lo = divmod(int(codes[t, g, d // 2]), 16)
    c = hi if d % 2 else lo
    return float(scale[t, g, d // 32]) * c + float(mn[t, g, d // 32])


def _python_attention(bits, q, cache):
    kc, ks, km, vc, vs, vm = cache
    T, Hkv = ks.shape[0], ks.shape[1]
    Hq = q.shape[0]
    G = Hq // Hkv
    o = [[0.0] * D for _ in range(Hq)]
    for h in range(Hq):
        g = h // G
        scores = [math.fsum(float(q[h, d]) * _value(bits, kc, ks, km, t, g, d) for d in range(D)) / math.sqrt(D)
                  for t in range(T)]
        mx = max(scores)
        e = [math.exp(s - mx) for s in scores]
        tot = math.fsum(e)
        for d in range(D):
            o[h][d] = math.fsum(e[t] / tot * _value(bits, vc, vs, vm, t, g, d) for t in range(T))
    return np.array(o)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T,Hq,Hkv", [(1, 1, 1), (3, 4, 2), (5, 8, 2)])
def test_pure_python_reimplementation(bits, T, Hq, Hkv):
    q, cache = _problem(bits, T, Hq, Hkv, seed=T)
    o, B = A.attention(bits, q, *cache)
    ref = _python_attention(bits, q, cache)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [8, 4])
def test_single_token_returns_its_value(bits):
    q, cache = _problem(bits, 1, 8, 2, seed=3)
    o, B = A.attention(bits, q, *cache)
    v = A.dequantise_cache(bits, cache[3], cache[4], cache[5])
    for h in range(8):
        np.testing.assert_array_equal(o[h], v[0, h // 4])
        np.testing.assert_array_equal(B[h], np.abs(v[0, h // 4]))


def test_zero_int8_keys_give_uniform_weights():
    q, (kc, ks, km, vc, vs, vm) = _problem(8, 37, 4, 1, seed=4)
    kc = np.zeros_like(kc)
    o, B = A.attention(8, q, kc, ks, km, vc, vs, vm)
    v = vs.astype(np.float64).repeat(32, axis=-1) * vc.astype(np.float64)
    for h in range(4):
        np.testing.assert_allclose(o[h], v[:, 0, :].mean(axis=0), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(B[h], np.abs(v[:, 0, :]).mean(axis=0), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("bits,codec", [(8, "q8_sym"), (4, "q4")])
def test_dequantisation_is_the_codec_oracle(bits, codec):
    _, (kc, ks, km, _, _, _) = _problem(bits, 19, 8, 4, seed=5)
    got = A.dequantise_cache(bits, kc, ks, km).reshape(19 * 4, D)
    rows = kc.reshape(19 * 4, -1)
    ref = oracle.codecs_ref.dequantise(codec, rows, ks.reshape(19 * 4, 4), None if km is None else km.reshape(-1, 4))
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("bits", [8, 4])
def test_token_permutation_invariance(bits):
    q, cache = _problem(bits, 64, 8, 2, seed=6)
    perm = np.random.default_rng(1).permutation(64)
    o, B = A.attention(bits, q, *cache)
    o2, B2 = A.attention(bits, q, *[None if c is None else c[perm] for c in cache])
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(B2, B, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bits", [8, 4])
def test_grouped_head_is_a_single_head_problem(bits):
    q, cache = _problem(bits, 50, 8, 2, seed=7)
    o, B = A.attention(bits, q, *cache)
    for h in (0, 3, 4, 7):
        g = h // 4
        sub = [None if c is None else c[:, g:g + 1] for c in cache]
        o1, B1 = A.attention(bits, q[h:h + 1], *sub)
        np.testing.assert_array_equal(o1[0], o[h])
        np.testing.assert_array_equal(B1[0], B[h])


def test_dominant_token_takes_the_weight():
    T = 40
    q = np.zeros((1, D), np.float16)
    q[0, :] = 4.0
    kc = np.zeros((T, 1, D), np.int8)
    kc[17] = 127                    # score of token 17: 128 * 4 * 127 * s / sqrt(128) >> every other
    ks = np.full((T, 1, 4), 0.01, np.float16)
    _, (_, _, _, vc, vs, vm) = _problem(8, T, 1, 1, seed=8)
    o, B = A.attention(8, q, kc, ks, None, vc, vs, vm)
    v = A.dequantise_cache(8, vc, vs)
    np.testing.assert_allclose(o[0], v[17, 0], rtol=1e-12, atol=1e-12)


def test_rejects_bad_inputs():
    q, cache = _problem(8, 4, 4, 2)
    with pytest.raises(ValueError):
        A.attention(8, q[:3], *cache)
    with pytest.raises(TypeError):
        A.dequantise_cache(8, cache[0].view(np.uint8), cache[1])
    with pytest.raises(ValueError):
        A.dequantise_cache(5, cache[0], cache[1])


def test_kv_recipe_shapes():
    for bits, T in workload.KV_CONTEXT.items():
        assert T == {8: 38863, 4: 77726}[bits]
        cache = workload.kv_cache(bits, 1, 0, 5, 8)
        assert cache[0].shape == ((5, 8, 128) if bits == 8 else (5, 8, 64))
        assert cache[1].shape == (5, 8, 4) and (cache[2] is None) == (bits == 8)
    assert workload.kv_query(1, 0).shape == (32, 128)
