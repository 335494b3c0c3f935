"""Pins for the fp64 oracle of the weight-code variants (q4_sym, q5, q8_sym).

Each pin is independent of the oracle's own formula, and together they catch
the plausible slips: a wrong code offset or sign convention (q - 8, int8 read
as unsigned), a dropped fifth bit, a wrong group index, swapped nibbles, a
transposed operand, a lossy accumulation:

* hand-derived worked examples (tests/golden/tiny_codecs.json);
* exact rational brute force on tiny shapes, decoding the code bytes with
  plain integer arithmetic written here;
* special cases that reduce to the pinned 4-bit group-affine oracle: q4_sym
  is q4 with min = -8 * scale, q5 with codes below 16 is q4 on the same
  nibbles, q8_sym with codes 0..15 is q4 with min = 0;
* closed forms (codes at the symmetric centre give 0; a constant code c gives
  c * sum_g scale_g * sum_{k in g} x_k), odd symmetry of q8_sym, and the
  fifth-bit split of q5.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload

HERE = os.path.dirname(__file__)
C = oracle.codecs_ref


def _golden():
    with open(os.path.join(HERE, "golden", "tiny_codecs.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("codec", ["q4_sym", "q5", "q8_sym", "pal4"])
def test_golden_tiny_examples(codec):
    fx = _golden()
    case = fx["cases"][codec]
    x = np.array(fx["x"], dtype=np.float16)
    if "codes_hex" in case:
        codes = np.array([list(bytes.fromhex(h)) for h in case["codes_hex"]], dtype=np.uint8)
    else:
        codes = np.array(case["codes"], dtype=np.int8 if codec == "q8_sym" else np.uint8)
    mn = np.array(case["min"], dtype=np.float16) if "min" in case else None
    y, B = C.gemv(codec, x, codes, np.array(case["scale"], dtype=np.float16), mn)
    np.testing.assert_array_equal(y, np.array(case["y"]))
    np.testing.assert_array_equal(B, np.array(case["B"]))


def _code_value(codec, codes, n, k):
    """The code of weight (n, k), decoded from the raw bytes with integer arithmetic."""
    if codec in ("q4_sym", "pal4"):
        hi, lo = divmod(int(codes[n, k // 2]), 16)
        return (hi if k % 2 else lo) - (8 if codec == "q4_sym" else 0)
    if codec == "q5":
        return int(codes[n, k])
    b = int(np.asarray(codes[n, k]).view(np.uint8))
    return b - 256 if b >= 128 else b


def _exact(codec, x, codes, scale, mn):
    M, K = x.shape
    N = scale.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    B = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            if codec == "pal4":  # palette entry of the code
                w = Fraction(float(scale[n, _code_value(codec, codes, n, k)]))
            else:
                w = Fraction(float(scale[n, k // 32])) * _code_value(codec, codes, n, k)
            if mn is not None:
                w += Fraction(float(mn[n, k // 32]))
            for m in range(M):
                p = w * Fraction(float(x[m, k]))
                y[m][n] += p
                B[m][n] += abs(p)
    return y, B


@pytest.mark.parametrize("codec", ["q4_sym", "q5", "q8_sym", "pal4"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (8, 5, 96)])
def test_exact_rational_bruteforce(codec, M, N, K):
    x, codes, scale, mn = workload.random_codec_problem(codec, 7, M, N, K)
    flat = x.reshape(-1)
    flat[:4] = np.array([65504.0, 2.0 ** -14, 2.0 ** -24, -0.0], dtype=np.float16)
    scale.reshape(-1)[:1] = np.float16(2.0 ** -24)
    if mn is not None:
        mn.reshape(-1)[:1] = np.float16(-0.0)
    y, B = C.gemv(codec, x, codes, scale, mn)
    ye, Be = _exact(codec, x, codes, scale, mn)
    for m in range(M):
        for n in range(N):
            bound = 4 * K * 2.0 ** -53 * float(Be[m][n])
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Fraction(bound)
            assert abs(Fraction(B[m, n]) - Be[m][n]) <= Fraction(bound)


@pytest.mark.parametrize("M,N,K", [(1, 7, 64), (3, 33, 512)])
def test_q4_sym_is_q4_with_min_minus_eight_scales(M, N, K):
    x, codes, scale, _ = workload.random_codec_problem("q4_sym", 2, M, N, K)
    mn = (-8.0 * scale.astype(np.float64)).astype(np.float16)
    assert np.array_equal(mn.astype(np.float64), -8.0 * scale.astype(np.float64))  # exact in binary16
    y, B = C.gemv("q4_sym", x, codes, scale)
    y4, B4 = oracle.gemv(x, codes, scale, mn)
    np.testing.assert_array_equal(y, y4)
    np.testing.assert_array_equal(B, B4)


@pytest.mark.parametrize("M,N,K", [(2, 9, 96), (1, 40, 1024)])
def test_q5_below_sixteen_is_q4_on_the_same_nibbles(M, N, K):
    x, codes, scale, mn = workload.random_codec_problem("q5", 3, M, N, K)
    lo = codes & 0x0F
    packed = (lo[:, 0::2] | (lo[:, 1::2] << 4)).astype(np.uint8)
    y, B = C.gemv("q5", x, lo, scale, mn)
    y4, B4 = oracle.gemv(x, packed, scale, mn)
    np.testing.assert_array_equal(y, y4)
    np.testing.assert_array_equal(B, B4)


@pytest.mark.parametrize("M,N,K", [(2, 9, 96), (4, 17, 256)])
def test_q8_sym_small_codes_is_q4_with_zero_min(M, N, K):
    x, codes, scale, _ = workload.random_codec_problem("q8_sym", 4, M, N, K)
    small = (codes.view(np.uint8) & 0x0F).astype(np.int8)
    u = small.view(np.uint8)
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    y, B = C.gemv("q8_sym", x, small, scale)
    y4, B4 = oracle.gemv(x, packed, scale, np.zeros_like(scale))
    np.testing.assert_array_equal(y, y4)
    np.testing.assert_array_equal(B, B4)


@pytest.mark.parametrize("M,N,K", [(1, 7, 64), (3, 33, 512)])
def test_pal4_affine_palette_is_q4(M, N, K):
    """A palette lut[n][c] = s_n * c + m_n (exact in binary16) is the 4-bit
    group-affine code with that scale and min in every group of row n."""
    x, codes, _, _ = workload.random_codec_problem("pal4", 12, M, N, K)
    rng = np.random.default_rng(3)
    s = rng.integers(1, 8, size=N).astype(np.float64) / 64.0     # a few mantissa bits: s*c + m exact
    m = -rng.integers(0, 32, size=N).astype(np.float64) / 16.0
    lut = (s[:, None] * np.arange(16)[None, :] + m[:, None]).astype(np.float16)
    assert np.array_equal(lut.astype(np.float64), s[:, None] * np.arange(16)[None, :] + m[:, None])
    G = K // 32
    y, B = C.gemv("pal4", x, codes, lut)
    y4, B4 = oracle.gemv(x, codes, np.repeat(s[:, None], G, 1).astype(np.float16), np.repeat(m[:, None], G, 1).astype(np.float16))
    np.testing.assert_array_equal(y, y4)
    np.testing.assert_array_equal(B, B4)


def _group_sums(x):
    M, K = x.shape
    return x.astype(np.float64).reshape(M, K // 32, 32).sum(axis=2)


@pytest.mark.parametrize("M,N,K", [(1, 5, 64), (3, 11, 320)])
def test_closed_forms_constant_codes(M, N, K):
    x, _, scale, mn = workload.random_codec_problem("q5", 5, M, N, K)
    xs = _group_sums(x)
    s64, m64 = scale.astype(np.float64), mn.astype(np.float64)
    # q4_sym at its centre code 8: every weight is exactly 0
    y, B = C.gemv("q4_sym", x, np.full((N, K // 2), 0x88, np.uint8), scale)
    assert not y.any() and not B.any()
    # q4_sym all codes 0: -8 s per group
    y, B = C.gemv("q4_sym", x, np.zeros((N, K // 2), np.uint8), scale)
    np.testing.assert_allclose(y, xs @ (-8.0 * s64).T, rtol=0, atol=1e-12 * (1 + B.max()))
    # q5 all codes 31: (31 s + m) per group
    y, B = C.gemv("q5", x, np.full((N, K), 31, np.uint8), scale, mn)
    np.testing.assert_allclose(y, xs @ (31.0 * s64 + m64).T, rtol=0, atol=1e-12 * (1 + B.max()))
    # q8_sym constant codes -128 and 127
    for c in (-128, 127):
        y, B = C.gemv("q8_sym", x, np.full((N, K), c, np.int8), scale)
        np.testing.assert_allclose(y, xs @ (c * s64).T, rtol=0, atol=1e-12 * (1 + B.max()))


def test_q8_sym_odd_symmetry():
    x, codes, scale, _ = workload.random_codec_problem("q8_sym", 6, 2, 13, 128)
    codes = np.where(codes == -128, np.int8(-127), codes).astype(np.int8)
    y, B = C.gemv("q8_sym", x, codes, scale)
    yn, Bn = C.gemv("q8_sym", x, (-codes.astype(np.int16)).astype(np.int8), scale)
    np.testing.assert_array_equal(yn, -y)
    np.testing.assert_array_equal(Bn, B)


def test_q5_fifth_bit_split():
    # y(lo + 16 h; s, m) = y(lo; s, m) + 16 * y(h; s, 0), within fp64 rounding
    x, codes, scale, mn = workload.random_codec_problem("q5", 8, 3, 21, 256)
    lo, h = codes & 0x0F, codes >> 4
    y, B = C.gemv("q5", x, codes, scale, mn)
    y1, _ = C.gemv("q5", x, lo, scale, mn)
    y2, _ = C.gemv("q5", x, h.astype(np.uint8), scale, np.zeros_like(mn))
    np.testing.assert_allclose(y, y1 + 16.0 * y2, rtol=0, atol=1e-12 * (1 + B.max()))
    assert (h <= 1).all() and h.any()


@pytest.mark.parametrize("codec", ["q4_sym", "q5", "q8_sym", "pal4"])
def test_one_hot_x_selects_single_weight(codec):
    N, K = 6, 96
    _, codes, scale, mn = workload.random_codec_problem(codec, 9, 1, N, K)
    for k in (0, 1, 31, 32, 63, 95):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, k] = 1.0
        y, B = C.gemv(codec, x, codes, scale, mn)
        for n in range(N):
            if codec == "pal4":
                w = float(scale[n, _code_value(codec, codes, n, k)])
            else:
                w = float(scale[n, k // 32]) * _code_value(codec, codes, n, k)
            if mn is not None:
                w += float(mn[n, k // 32])
            assert y[0, n] == w and B[0, n] == abs(w)


def test_rejects_bad_inputs():
    x = np.zeros((1, 64), np.float16)
    s = np.ones((2, 2), np.float16)
    with pytest.raises(ValueError):
        C.gemv("q3", x, np.zeros((2, 32), np.uint8), s, s)
    with pytest.raises(ValueError):
        C.gemv("q5", x, np.full((2, 64), 32, np.uint8), s, s)
    with pytest.raises(TypeError):
        C.gemv("q8_sym", x, np.zeros((2, 64), np.uint8), s)
    with pytest.raises(ValueError):
        C.gemv("q5", x, np.zeros((2, 64), np.uint8), s, None)
    with pytest.raises(ValueError):   # a palette must have 16 entries per row
        C.gemv("pal4", x, np.zeros((2, 32), np.uint8), s)


def test_codec_workload_recipe():
    for codec in workload.CODECS:
        codes, scale, mn = workload.codec_weights(codec, 2, 0, 0, 8, 64)
        assert codes.shape == C.code_shape(codec, 8, 64)
        assert scale.shape == ((8, 16) if codec == "pal4" else (8, 2)) and scale.dtype == np.float16
        assert (mn is None) == C.SYMMETRIC[codec]
    q4 = workload.codec_weights("q4", 2, 0, 0, 8, 64)
    base = workload.weights(2, 0, 0, 8, 64)
    for a, b in zip(q4, base):
        np.testing.assert_array_equal(a, b)
