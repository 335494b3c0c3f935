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


# --------------------------------------------------------------------------
# Temperature: a hand-derived two-token case (tests/golden/kv_two_token.json)
# --------------------------------------------------------------------------
import json  # noqa: E402
import os  # noqa: E402

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_two_token.json")))


def _two_token_inputs(case):
    """The fixture's cache: one query head, one KV head, two tokens."""
    bits = case["bits"]
    q = np.zeros((1, D), np.float16)
    q[0, 0] = 1.0
    if bits == 8:
        kc = np.zeros((2, 1, D), np.int8)
        kc[0, 0, 0] = case["k_code0"]
        vc = np.zeros((2, 1, D), np.int8)
        vc[0] = case["v_code0"]
        vc[1] = case["v_code1"]
        km = vm = None
    else:
        kc = np.zeros((2, 1, D // 2), np.uint8)
        kc[0, 0, 0] = case["k_code0"]                       # low nibble: dim 0
        vc = np.zeros((2, 1, D // 2), np.uint8)
        vc[0] = case["v_code0"] | (case["v_code0"] << 4)
        vc[1] = case["v_code1"] | (case["v_code1"] << 4)
        km = np.full((2, 1, 4), case["k_min"], np.float16)
        vm = np.full((2, 1, 4), case["v_min"], np.float16)
    ks = np.full((2, 1, 4), case["k_scale"], np.float16)
    vs = np.full((2, 1, 4), case["v_scale"], np.float16)
    return bits, q, (kc, ks, km, vc, vs, vm)


def _golden_matches(case, attention):
    bits, q, cache = _two_token_inputs(case)
    o, B = attention(bits, q, *cache)
    return np.allclose(o, case["o"], rtol=1e-13, atol=0) and np.allclose(B, case["B"], rtol=1e-13, atol=0)


def test_two_token_golden_values_are_their_closed_forms():
    d = GOLDEN["delta"]
    assert d == pytest.approx(8 / math.sqrt(128), rel=1e-15)
    p0 = 1 / (1 + math.exp(-d))
    c8, c4 = GOLDEN["cases"]
    assert c8["o"] == pytest.approx(math.tanh(d / 2), rel=1e-15) and c8["B"] == 1.0
    assert c4["o"] == pytest.approx(1.875 * p0 - 1, rel=1e-15)
    assert c4["B"] == pytest.approx(1 - 0.125 * p0, rel=1e-15)


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: f"int{c['bits']}")
def test_two_token_golden(case):
    assert _golden_matches(case, A.attention)


class _NumpyWithSqrt:
    """numpy, except for sqrt: a planted mistake in the oracle's temperature."""

    def __init__(self, sqrt):
        self._sqrt = sqrt

    def __getattr__(self, name):
        return self._sqrt if name == "sqrt" else getattr(np, name)


@pytest.mark.parametrize("mutant", [lambda x: 1.0, lambda x: x, lambda x: x ** 0.25],
                         ids=["no temperature", "1/D", "D^-1/4"])
def test_two_token_golden_catches_a_wrong_temperature(monkeypatch, mutant):
    monkeypatch.setattr(A, "np", _NumpyWithSqrt(mutant))
    assert not any(_golden_matches(case, A.attention) for case in GOLDEN["cases"])


@pytest.mark.parametrize("bits", [8, 4])
def test_constant_score_shift_invariance(bits):
    """Adding the same amount to every token's score leaves the weights alone:
    give every token the same key value in dim 127, then change the query in
    that dim."""
    q, (kc, ks, km, vc, vs, vm) = _problem(bits, 90, 4, 1, seed=9)
    ks = ks.copy()
    ks[:, :, 3] = 0.25
    kc = kc.copy()
    if bits == 8:
        kc[:, :, 127] = 6
    else:
        kc[:, :, 63] = (kc[:, :, 63] & 0x0F) | (6 << 4)     # high nibble: dim 127
        km = km.copy()
        km[:, :, 3] = -0.5
    o, B = A.attention(bits, q, kc, ks, km, vc, vs, vm)
    q2 = q.copy()
    q2[:, 127] = (q2[:, 127].astype(np.float32) + 2.0).astype(np.float16)
    o2, B2 = A.attention(bits, q2, kc, ks, km, vc, vs, vm)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(B2, B, rtol=1e-12, atol=1e-14)
    q3 = q.copy()
    q3[:, 5] = (q3[:, 5].astype(np.float32) + 2.0).astype(np.float16)   # a dim the keys differ in
    o3, _ = A.attention(bits, q3, kc, ks, km, vc, vs, vm)
    assert np.abs(o3 - o).max() > 1e-6


# --------------------------------------------------------------------------
# Sentinel cache: every block of 64 tokens visible on its own
# --------------------------------------------------------------------------
from kv_sentinel import sentinel_closed_form  # noqa: E402

@pytest.mark.parametrize("bits,T,Hq,Hkv", [(8, 3001, 32, 8), (4, 2222, 16, 2), (4, 300, 8, 1)])
def test_sentinel_cache_oracle_is_its_closed_form(bits, T, Hq, Hkv):
    cache = workload.kv_sentinel_cache(bits, T, Hkv)
    q = workload.kv_query(77, 0, Hq)
    o, B = A.attention(bits, q, *cache)
    o_cf, B_cf = sentinel_closed_form(bits, T, Hq, Hkv)
    np.testing.assert_allclose(o, o_cf, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(B, B_cf, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("bits,T,Hkv", [(8, 38863, 8), (4, 77726, 8), (8, 40000, 1), (4, 80000, 1)])
def test_sentinel_cache_shows_every_block(bits, T, Hkv):
    """At the full 8B contexts and the one-KV-head merge shapes, removing any
    single block (or counting it twice) moves its channel by far more than the
    tolerance: each block carries at least 8 % of its channel (a tenth of
    it with one KV head over 80,000 tokens), against a 0.1 % tolerance."""
    nb = -(-T // workload.KV_BLOCK)
    share = np.zeros((Hkv, D))
    counts = np.zeros((Hkv, D))
    for b in range(nb):
        g, d = workload.kv_sentinel_channel(b, Hkv)
        counts[g, d] += min(T, (b + 1) * workload.KV_BLOCK) - b * workload.KV_BLOCK
    worst = 1.0
    for b in range(nb):
        g, d = workload.kv_sentinel_channel(b, Hkv)
        n = min(T, (b + 1) * workload.KV_BLOCK) - b * workload.KV_BLOCK
        worst = min(worst, n / counts[g, d])
        share[g, d] = max(share[g, d], n / counts[g, d])
    o, B = sentinel_closed_form(bits, T, Hkv, Hkv)
    tol = A.tolerance(B)
    # the smallest block moves its channel by worst * o, against a tolerance of 1e-3 * o + 1e-5
    marked = counts > 0
    assert worst >= 0.08, worst
    assert (worst * o[marked] > 10 * tol[marked]).all()
