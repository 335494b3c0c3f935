"""Plain fp64 reference for the weight-code variants of the decode GEMV.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by the bench's CPU-baseline
leg; never by the product path.

Where the variants come from
----------------------------
The Magnitude page (section 4.2, model conversion) compares three llama.cpp
quantisation types it measured: a plain symmetric 4-bit type (q4_0: smallest,
least accurate), the K-quant 4-bit type (q4_k_m: the group-affine code of
``w4a16_ref``) and a 5-bit K-quant (q5_k_m: more accurate, about a quarter
larger). The core-modules page puts edge weights at INT8 or INT4 (section 5.1,
packer: quantisation) and lists 4-bit and 8-bit weight quantisation among the
runtimes' specialities (section 5.2, runtime table). None of the pages defines
a bit format. The readings used here, one per codec, keep the group of 32
consecutive k of one row with binary16 parameters, as for the 4-bit code:

* ``q4``     ``w_hat = s * q + m``,   q unsigned 4-bit (0..15), codes
             ``uint8[N, K/2]`` (low nibble = even k): the ``w4a16_ref`` code.
* ``q4_sym`` ``w_hat = s * (q - 8)``, q unsigned 4-bit, same code bytes; a
             scale and no min (the symmetric type: codes centred on 8).
* ``q5``     ``w_hat = s * q + m``,   q unsigned 5-bit (0..31), codes
             ``uint8[N, K]`` one code per byte (the canonical form; packing
             into 5 bits is the library's business).
* ``q8_sym`` ``w_hat = s * q``,       q signed 8-bit (-128..127, two's
             complement), codes ``int8[N, K]`` (passed as their bytes).
* ``pal4``   ``w_hat = lut[n, q]``,   q unsigned 4-bit, same code bytes as
             ``q4``; a 16-entry binary16 palette per output row (Core ML's
             palettisation, named in the core-modules page's runtime table,
             section 5.2, read at per-channel granularity: one lookup table
             per row, since a table per group of 32 weights would cost more
             bytes than the weights it encodes).

s and m are binary16 ``[N, K/32]``; the symmetric codecs have no m. For
``pal4`` the ``scale`` argument carries the palettes, binary16 ``[N, 16]``,
and there is no m.

What is computed: y[m, n] = sum_k w_hat[n, k] * x[m, k] and the tolerance scale
B[m, n] = sum_k |w_hat[n, k] * x[m, k]|, in fp64, with the same pass rule
|y' - y| <= 1e-3 * B + 1e-5. Every w_hat (at most 8 + 11 significant bits) and
every product with a binary16 x is exact in fp64, so only the sum over k
rounds.

Parity status: the pages print no worked values for any codec. The pins are
exact rational brute force, hand-derived golden fixtures under tests/golden/,
closed forms, and special cases that reduce to the pinned 4-bit group-affine
oracle (q4_sym is q4 with m = -8 s; q5 with codes below 16 is q4; q8_sym with
codes 0..15 is q4 with m = 0; pal4 with an affine palette s*c + m is q4 with
that scale and min).
"""
from __future__ import annotations

import concurrent.futures as _cf

import numpy as np

GROUP = 32
CODECS = ("q4", "q4_sym", "q5", "q8_sym", "pal4")
SYMMETRIC = {"q4": False, "q4_sym": True, "q5": False, "q8_sym": True, "pal4": True}  # True: no min array
# code bytes per weight in the canonical (unpacked) layout
_CODE_BYTES_PER_K = {"q4": 0.5, "q4_sym": 0.5, "q5": 1.0, "q8_sym": 1.0, "pal4": 0.5}
PALETTE = 16


def code_shape(codec: str, N: int, K: int):
    """Shape of the canonical code array of an N x K matrix."""
    if codec not in CODECS:
        raise ValueError(f"unknown codec {codec!r}")
    return (N, int(K * _CODE_BYTES_PER_K[codec]))


def _check(codec, codes, scale, mn):
    if codec not in CODECS:
        raise ValueError(f"unknown codec {codec!r}")
    codes = np.asarray(codes)
    N = codes.shape[0]
    if codec in ("q4", "q4_sym", "pal4"):
        if codes.dtype != np.uint8:
            raise TypeError("4-bit codes must be uint8 [N, K/2]")
        K = 2 * codes.shape[1]
    elif codec == "q5":
        if codes.dtype != np.uint8:
            raise TypeError("5-bit codes must be uint8 [N, K]")
        if codes.size and int(codes.max()) > 31:
            raise ValueError("5-bit codes must be < 32")
        K = codes.shape[1]
    else:
        if codes.dtype != np.int8:
            raise TypeError("8-bit codes must be int8 [N, K]")
        K = codes.shape[1]
    if K % GROUP or K <= 0:
        raise ValueError("K must be a positive multiple of 32")
    if codec == "pal4":
        if np.asarray(scale).shape != (N, PALETTE):
            raise ValueError("the palettes must be [N, 16]")
        return N, K
    if np.asarray(scale).shape != (N, K // GROUP):
        raise ValueError("scale must be [N, K/32]")
    if not SYMMETRIC[codec] and (mn is None or np.asarray(mn).shape != (N, K // GROUP)):
        raise ValueError("min must be [N, K/32] for an affine codec")
    return N, K


def unpack(codec: str, codes) -> np.ndarray:
    """Canonical codes -> int64 [N, K] code values q (before the affine map)."""
    codes = np.asarray(codes)
    if codec in ("q4", "q4_sym", "pal4"):
        q = np.empty((codes.shape[0], 2 * codes.shape[1]), dtype=np.int64)
        q[:, 0::2] = codes & 0x0F
        q[:, 1::2] = codes >> 4
        return q
    if codec == "q5":
        return codes.astype(np.int64)
    if codec == "q8_sym":
        return codes.astype(np.int64)  # int8 -> signed values
    raise ValueError(f"unknown codec {codec!r}")


def dequantise(codec: str, codes, scale, mn=None) -> np.ndarray:
    """w_hat in fp64 (exact) for one of CODECS."""
    _check(codec, codes, scale, mn)
    if codec == "pal4":  # w_hat[n, k] = lut[n, q[n, k]]
        q = unpack(codec, codes)
        lut = np.asarray(scale).astype(np.float64)
        return np.take_along_axis(lut, q, axis=1)
    q = unpack(codec, codes).astype(np.float64)
    s = np.repeat(np.asarray(scale).astype(np.float64), GROUP, axis=1)
    if codec == "q4_sym":
        return s * (q - 8.0)
    if codec == "q8_sym":
        return s * q
    m = np.repeat(np.asarray(mn).astype(np.float64), GROUP, axis=1)
    return s * q + m


def gemv(codec: str, x, codes, scale, mn=None, row_block: int = 256, threads: int = 1):
    """(y, B) in fp64, both [M, N]: y = x @ w_hat.T, B = |x| @ |w_hat|.T.

    Rows are processed in blocks of ``row_block`` (optionally on a thread
    pool); blocking only splits the output columns, each element is one plain
    dot product.
    """
    N, K = _check(codec, codes, scale, mn)
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    x64 = x.astype(np.float64)
    ax64 = np.abs(x64)
    M = x.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    codes = np.asarray(codes)
    scale = np.asarray(scale)
    mn = None if SYMMETRIC[codec] else np.asarray(mn)

    def run(r0):
        r1 = min(N, r0 + row_block)
        w = dequantise(codec, codes[r0:r1], scale[r0:r1], None if mn is None else mn[r0:r1])
        y[:, r0:r1] = x64 @ w.T
        B[:, r0:r1] = ax64 @ np.abs(w).T

    starts = range(0, N, row_block)
    if threads <= 1:
        for r0 in starts:
            run(r0)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, starts))
    return y, B


def gemv_rows(codec: str, x, codes, scale, mn, rows):
    """(y, B) for the selected output rows only: [M, len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    codes = np.asarray(codes)
    return gemv(codec, x, codes[rows], np.asarray(scale)[rows], None if mn is None else np.asarray(mn)[rows])
