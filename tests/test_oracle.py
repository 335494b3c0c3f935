"""Pins for the fp64 oracle, independent of the oracle's own formula.

Each test is chosen so that a plausible slip in the oracle (nibble order,
group index, a dropped min term, a transposed operand, a wrong sign, a lossy
accumulation) fails at least one of them:

* a hand-derived worked example (tests/golden/tiny_gemv.json);
* closed forms that the group-affine format fixes: all-zero codes give
  y = sum_g min_g * sum_{k in g} x_k, all-15 codes give (15 s + min) per group;
* the quantise/dequantise round trip |w - w_hat| <= scale/2 and, through it,
  agreement with a library matmul of the unquantised weights;
* an independent bit-level nibble decode (numpy.unpackbits) for scale=1, min=0,
  where the product is an exact integer matmul;
* exact rational brute force on tiny shapes (bounds the fp64 rounding);
* linearity and invariance under permuting whole 32-groups of K;
* the tolerance scale B against its definition's invariants.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workload

HERE = os.path.dirname(__file__)


def _rand(seed, M, N, K):
    return workload.random_problem(seed, M, N, K)


def test_golden_tiny_example():
    with open(os.path.join(HERE, "golden", "tiny_gemv.json")) as f:
        fx = json.load(f)
    codes = np.array([list(bytes.fromhex(h)) for h in fx["codes_hex"]], dtype=np.uint8)
    scale = np.array(fx["scale"], dtype=np.float16)
    mn = np.array(fx["min"], dtype=np.float16)
    x = np.array(fx["x"], dtype=np.float16)
    assert codes.shape == (fx["N"], fx["K"] // 2)
    y, B = oracle.gemv(x, codes, scale, mn)
    np.testing.assert_array_equal(y, np.array(fx["y"]))
    np.testing.assert_array_equal(B, np.array(fx["B"]))


@pytest.mark.parametrize("N,K,M", [(5, 64, 1), (7, 96, 3), (33, 4096, 2)])
def test_closed_form_zero_codes(N, K, M):
    x, _, scale, mn = _rand(1, M, N, K)
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    y, B = oracle.gemv(x, codes, scale, mn)
    xs = x.astype(np.float64).reshape(M, K // 32, 32).sum(axis=2)      # [M, G]
    expect = xs @ mn.astype(np.float64).T                                # [M, N]
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-12 * (1 + B.max()))
    # |w_hat| = |min| here, so B is |x|-sums times |min|
    axs = np.abs(x.astype(np.float64)).reshape(M, K // 32, 32).sum(axis=2)
    np.testing.assert_allclose(B, axs @ np.abs(mn.astype(np.float64)).T, rtol=1e-13)


@pytest.mark.parametrize("N,K,M", [(5, 64, 1), (9, 160, 4)])
def test_closed_form_all_fifteen(N, K, M):
    x, _, scale, mn = _rand(2, M, N, K)
    codes = np.full((N, K // 2), 0xFF, dtype=np.uint8)
    y, _ = oracle.gemv(x, codes, scale, mn)
    xs = x.astype(np.float64).reshape(M, K // 32, 32).sum(axis=2)
    per_group = 15.0 * scale.astype(np.float64) + mn.astype(np.float64)   # [N, G]
    np.testing.assert_allclose(y, xs @ per_group.T, rtol=0, atol=1e-12 * (1 + np.abs(y).max()))


def test_one_hot_x_selects_single_weight():
    """x = e_k returns w_hat[:, k] exactly; checked against a scalar per-element decode."""
    N, K = 6, 96
    _, codes, scale, mn = _rand(3, 1, N, K)
    eye = np.eye(K, dtype=np.float16)
    y, B = oracle.gemv(eye, codes, scale, mn)          # y[k, n] = w_hat[n, k]
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            q = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
            w = float(scale[n, k // 32]) * q + float(mn[n, k // 32])
            assert y[k, n] == w
            assert B[k, n] == abs(w)


def test_bitlevel_decode_integer_matmul():
    """scale = 1, min = 0: y = x @ q.T with q decoded from bits by numpy.unpackbits."""
    rng = np.random.default_rng(7)
    N, K, M = 11, 128, 3
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bits = np.unpackbits(codes, axis=1, bitorder="little").reshape(N, K // 2, 2, 4)
    q = (bits * np.array([1, 2, 4, 8])).sum(axis=3).reshape(N, K)        # [lo, hi] per byte
    xi = rng.integers(-8, 9, size=(M, K))
    scale = np.ones((N, K // 32), dtype=np.float16)
    mn = np.zeros((N, K // 32), dtype=np.float16)
    y, _ = oracle.gemv(xi.astype(np.float16), codes, scale, mn)
    np.testing.assert_array_equal(y, (xi @ q.T).astype(np.float64))


def _exact(x, codes, scale, mn):
    M, K = x.shape
    N = codes.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    B = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            q = (byte >> (4 * (k % 2))) & 0xF
            w = Fraction(float(scale[n, k // 32])) * q + Fraction(float(mn[n, k // 32]))
            for m in range(M):
                p = w * Fraction(float(x[m, k]))
                y[m][n] += p
                B[m][n] += abs(p)
    return y, B


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (8, 5, 96)])
def test_exact_rational_bruteforce(M, N, K):
    x, codes, scale, mn = _rand(4, M, N, K)
    # include extreme binary16 values: max normal, min normal, a subnormal, -0
    flat = x.reshape(-1)
    flat[:4] = np.array([65504.0, 2.0 ** -14, 2.0 ** -24, -0.0], dtype=np.float16)
    scale.reshape(-1)[:1] = np.float16(2.0 ** -24)
    mn.reshape(-1)[:1] = np.float16(-0.0)
    y, B = oracle.gemv(x, codes, scale, mn)
    ye, Be = _exact(x, codes, scale, mn)
    for m in range(M):
        for n in range(N):
            bound = 4 * K * 2.0 ** -53 * float(Be[m][n])
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Fraction(bound)
            assert abs(Fraction(B[m, n]) - Be[m][n]) <= Fraction(bound)


@settings(max_examples=60, deadline=None)
@given(
    seed=st.integers(0, 2**31 - 1),
    spread=st.floats(1e-3, 50.0),
    center=st.floats(-20.0, 20.0),
    const_group=st.booleans(),
)
def test_quantise_roundtrip_bound(seed, spread, center, const_group):
    rng = np.random.default_rng(seed)
    N, K = 3, 64
    w = center + spread * rng.standard_normal((N, K))
    if const_group:
        w[0, :32] = np.float16(center).astype(np.float64)   # degenerate: one exact value
        w[1, 32:] = center + 1e-7                             # degenerate: inexact value
    codes, s16, m16 = oracle.quantise(w)
    w_hat = oracle.dequantise(codes, s16, m16)
    s = np.repeat(s16.astype(np.float64), 32, axis=1)
    slack = 8 * np.finfo(np.float64).eps * (np.abs(w) + np.abs(w_hat) + 15 * s)
    assert np.all(np.abs(w - w_hat) <= s / 2 + slack)
    assert np.all(m16.astype(np.float64) <= w.reshape(N, K // 32, 32).min(axis=2))


@pytest.mark.parametrize("N,K,M", [(48, 256, 1), (37, 512, 8)])
def test_roundtrip_against_library_matmul(N, K, M):
    """gemv(x, quantise(W)) agrees with x @ W.T up to sum_k |x_k| * scale/2 (W non-square)."""
    rng = np.random.default_rng(N * K)
    # a per-(row, group) level plus small in-group noise, so the quantisation
    # step is small next to |w| and the bound is tight enough to catch a wrong
    # group index, a dropped min or a transposed operand
    level = rng.uniform(-0.08, 0.07, size=(N, K // 32))
    w = np.repeat(level, 32, axis=1) + 0.01 * rng.uniform(0.0, 1.0, size=(N, K))
    codes, s16, m16 = oracle.quantise(w)
    x = (1.0 + 0.5 * rng.standard_normal((M, K))).astype(np.float16)
    y, B = oracle.gemv(x, codes, s16, m16)
    ref = x.astype(np.float64) @ w.T
    half_step = np.repeat(s16.astype(np.float64), 32, axis=1) / 2          # [N, K]
    bound = np.abs(x.astype(np.float64)) @ half_step.T + 1e-12 * (1 + B)
    assert np.all(np.abs(y - ref) <= bound)
    # the bound is tight: far below |y| and below what a dropped min would cost
    assert bound.max() < 0.05 * np.abs(ref).max()
    y_nomin, _ = oracle.gemv(x, codes, s16, np.zeros_like(m16))
    assert np.all(np.abs(y_nomin - ref).max(axis=1) > bound.max(axis=1))


def test_linearity_powers_of_two():
    M, N, K = 2, 17, 256
    _, codes, scale, mn = _rand(5, M, N, K)
    rng = np.random.default_rng(5)
    # small integers: every combination a*x1 + b*x2 below is exact in binary16
    x1 = rng.integers(-64, 65, size=(M, K)).astype(np.float16)
    x2 = rng.integers(-64, 65, size=(M, K)).astype(np.float16)
    a, b = 0.5, -2.0
    xc = (a * x1.astype(np.float64) + b * x2.astype(np.float64))
    xc16 = xc.astype(np.float16)
    assert np.array_equal(xc16.astype(np.float64), xc)   # combination stays exact
    y1, B1 = oracle.gemv(x1, codes, scale, mn)
    y2, B2 = oracle.gemv(x2, codes, scale, mn)
    yc, _ = oracle.gemv(xc16, codes, scale, mn)
    tol = 1e-13 * (abs(a) * B1 + abs(b) * B2) + 1e-300
    assert np.all(np.abs(yc - (a * y1 + b * y2)) <= tol)


def test_group_permutation_invariance():
    M, N, K = 3, 9, 320
    x, codes, scale, mn = _rand(7, M, N, K)
    G = K // 32
    perm = np.random.default_rng(0).permutation(G)
    xp = x.reshape(M, G, 32)[:, perm].reshape(M, K)
    cp = codes.reshape(N, G, 16)[:, perm].reshape(N, K // 2)
    y, B = oracle.gemv(x, codes, scale, mn)
    yp, Bp = oracle.gemv(xp, cp, scale[:, perm], mn[:, perm])
    np.testing.assert_allclose(yp, y, rtol=0, atol=1e-13 * B.max())
    np.testing.assert_allclose(Bp, B, rtol=1e-13)


def test_tolerance_scale_invariants():
    M, N, K = 4, 21, 192
    x, codes, scale, mn = _rand(8, M, N, K)
    y, B = oracle.gemv(x, codes, scale, mn)
    assert np.all(B >= np.abs(y) - 1e-12 * B)
    # with x >= 0 and w_hat >= 0 (min = 0), every product is >= 0 so B == y
    xp = np.abs(x)
    y0, B0 = oracle.gemv(xp, codes, scale, np.zeros_like(mn))
    np.testing.assert_allclose(y0, B0, rtol=1e-14)
    assert np.all(oracle.within_tolerance(y + 0.9 * oracle.tolerance(B), y, B))
    assert not np.any(oracle.within_tolerance(y + 1.1 * oracle.tolerance(B), y, B))


def test_row_blocks_and_threads_do_not_change_results():
    M, N, K = 2, 300, 256
    x, codes, scale, mn = _rand(9, M, N, K)
    y1, B1 = oracle.gemv(x, codes, scale, mn, row_block=N)
    y2, B2 = oracle.gemv(x, codes, scale, mn, row_block=7, threads=3)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(B1, B2)
    rows = [0, 17, 299]
    yr, Br = oracle.gemv_rows(x, codes, scale, mn, rows)
    np.testing.assert_array_equal(yr, y1[:, rows])
    np.testing.assert_array_equal(Br, B1[:, rows])


def test_rejects_bad_shapes():
    x, codes, scale, mn = _rand(10, 1, 4, 64)
    with pytest.raises(ValueError):
        oracle.gemv(x[:, :32], codes, scale, mn)
    with pytest.raises(ValueError):
        oracle.gemv(x, codes, scale[:, :1], mn)
