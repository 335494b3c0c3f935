"""Plain, slow, obviously correct fp64 reference for the W4A16 decode GEMV.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's CPU-baseline leg; never by the product path.

What is computed, and where it comes from
-----------------------------------------
The core-modules page (section 5.1, packer: quantisation bullet) puts decode
on the edge in the 4-bit-weight / 16-bit-activation regime, and its runtime
table (section 5.2) names the K-quant family (Q4_K_M) as llama.cpp's format;
the Magnitude page (section 4.2, model conversion) recommends q4_k_m as the
best size/accuracy balance. Neither page defines the format bit by bit, so
the reading used here (stated once, for every function below) is the plain
group-affine one:

* weights are unsigned 4-bit codes q in 0..15, two per byte, the LOW nibble
  holding the even k and the HIGH nibble the odd k of row n;
* every 32 consecutive k of one row form a group g = k // 32 with its own
  binary16 scale s[n, g] and binary16 min m[n, g];
* the dequantised weight is  w_hat[n, k] = s[n, g] * q[n, k] + m[n, g];
* the product is  y[m, n] = sum_k w_hat[n, k] * x[m, k]  (row n = output
  feature, the nn.Linear orientation), x binary16 [M, K], y returned in fp64.

Alongside y the oracle returns the tolerance scale
B[m, n] = sum_k |w_hat[n, k] * x[m, k]|; a result y' passes when
|y' - y| <= 1e-3 * B + 1e-5 element by element.

Every w_hat and every product w_hat * x is exact in fp64 (a binary16 scale has
11 significant bits, q has 4, a binary16 x has 11; the min is exactly
representable), so only the K-term summation rounds: the oracle is within
about K * 2**-53 * B of the real-valued result.

Parity status: the pages print no worked GEMV values, so no function here is
pinned to a page example. The pins are closed forms, a quantise/dequantise
round-trip bound checked against a library matmul of the unquantised weights,
exact rational brute force, hand-derived golden fixtures under tests/golden/,
and metamorphic identities (linearity, group permutation).
"""
from __future__ import annotations

import concurrent.futures as _cf

import numpy as np

GROUP = 32
RTOL = 1e-3
ATOL = 1e-5


def _check(codes, scale, mn):
    N, Kh = codes.shape
    K = 2 * Kh
    if codes.dtype != np.uint8:
        raise TypeError("codes must be uint8")
    if K % GROUP:
        raise ValueError("K must be a multiple of 32")
    if scale.shape != (N, K // GROUP) or mn.shape != (N, K // GROUP):
        raise ValueError("scale/min must be [N, K/32]")
    return N, K


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8[N, K/2] -> int64[N, K]; low nibble is the even k, high nibble the odd k."""
    N, Kh = codes.shape
    q = np.empty((N, 2 * Kh), dtype=np.int64)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    return q


def dequantise(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """w_hat[n, k] = scale[n, k // 32] * q[n, k] + min[n, k // 32], in fp64 (exact)."""
    _check(codes, scale, mn)
    q = unpack_codes(codes).astype(np.float64)
    s = np.repeat(scale.astype(np.float64), GROUP, axis=1)
    m = np.repeat(mn.astype(np.float64), GROUP, axis=1)
    return s * q + m


def _block(x64, ax64, codes, scale, mn):
    w = dequantise(codes, scale, mn)
    return x64 @ w.T, ax64 @ np.abs(w).T


def gemv(x, codes, scale, mn, row_block: int = 256, threads: int = 1):
    """(y, B) in fp64, both [M, N]: y = x @ w_hat.T and B = |x| @ |w_hat|.T.

    Rows of the weight matrix are processed in blocks of ``row_block`` so the
    fp64 copy of w_hat stays small; ``threads`` > 1 hands the blocks to a pool
    of threads (numpy releases the GIL inside its kernels). Blocking only
    splits the output columns; every output element is one plain dot product.
    """
    N, K = _check(codes, scale, mn)
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    x64 = x.astype(np.float64)
    ax64 = np.abs(x64)
    M = x.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    starts = range(0, N, row_block)

    def run(r0):
        r1 = min(N, r0 + row_block)
        yb, bb = _block(x64, ax64, codes[r0:r1], scale[r0:r1], mn[r0:r1])
        y[:, r0:r1] = yb
        B[:, r0:r1] = bb

    if threads <= 1:
        for r0 in starts:
            run(r0)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, starts))
    return y, B


def gemv_rows(x, codes, scale, mn, rows):
    """(y, B) for the selected output rows only: [M, len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    return gemv(x, codes[rows], scale[rows], mn[rows])


def tolerance(B: np.ndarray) -> np.ndarray:
    """Allowed |y' - y| per element: 1e-3 * B + 1e-5."""
    return RTOL * B + ATOL


def within_tolerance(y_test, y_ref, B) -> np.ndarray:
    """Element-wise pass mask of a result against the oracle."""
    return np.abs(np.asarray(y_test, dtype=np.float64) - y_ref) <= tolerance(B)


# ---------------------------------------------------------------------------
# Round-trip quantiser (test helper; not on the GEMV path).
#
# The plain min/max reading of "group scale and min" (same reading as above):
# for each 32-group of real weights w,
#   m16 = the binary16 value of min(w) rounded DOWN,
#   s16 = the binary16 value of (max(w) - m16) / 15 rounded UP,
#   q   = clamp(rint((w - m16) / s16), 0, 15)  (ties to even).
# Then every w lies in [m16, m16 + 15 * s16], so |w - (s16 * q + m16)| <= s16/2
# up to the fp64 rounding of the division. If all w of a group are equal and
# exactly representable, s16 = 0, q = 0 and w_hat = w.
# ---------------------------------------------------------------------------


def _f16_down(v: np.ndarray) -> np.ndarray:
    h = v.astype(np.float16)
    above = h.astype(np.float64) > v
    h[above] = np.nextafter(h[above], np.float16(-np.inf))
    return h


def _f16_up(v: np.ndarray) -> np.ndarray:
    h = v.astype(np.float16)
    below = h.astype(np.float64) < v
    h[below] = np.nextafter(h[below], np.float16(np.inf))
    return h


def quantise(w: np.ndarray):
    """float64[N, K] -> (codes uint8[N, K/2], scale float16[N, K/32], min float16[N, K/32])."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 32")
    wg = w.reshape(N, K // GROUP, GROUP)
    m16 = _f16_down(wg.min(axis=2))
    s16 = _f16_up((wg.max(axis=2) - m16.astype(np.float64)) / 15.0)
    s64 = s16.astype(np.float64)[:, :, None]
    m64 = m16.astype(np.float64)[:, :, None]
    safe = np.where(s64 > 0, s64, 1.0)
    q = np.where(s64 > 0, np.rint((wg - m64) / safe), 0.0)
    q = np.clip(q, 0, 15).astype(np.uint8).reshape(N, K)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, s16, m16
