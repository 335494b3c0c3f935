"""The host repacker (w4a16_pack) against an independent decode of the layout.

`unpack_blob` below is written from the packed-layout text in include/w4a16.h
only (a 256-byte header, then: slot p of a 32-bit word holds i = 2p for p < 4
and 2(p-4)+1 otherwise; scale/min tiles of 4 rows); it shares no code with
the C++ repacker. Packing then decoding must give back the canonical arrays
bit for bit.
"""
import numpy as np
import pytest

import bit_weight_quantized_w4a16_amd as w4
import workload
from blob_header import HEADER_BYTES, strip_header


def _round_up(v, a):
    return (v + a - 1) // a * a


def unpack_blob(blob, N, K):
    blob = strip_header(blob, 0, N, K)
    G = K // 32
    S = _round_up(N * K // 2, 256)
    T = (N + 3) // 4
    assert blob.size >= S + T * G * 16
    words = blob[: N * K // 2].view("<u4").reshape(N, G, 4).astype(np.int64)
    q = np.empty((N, G, 4, 8), dtype=np.int64)             # [n, g, d, i]
    for p in range(8):
        i = 2 * p if p < 4 else 2 * (p - 4) + 1
        q[:, :, :, i] = (words >> (4 * p)) & 0xF
    q = q.reshape(N, K)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    tiles = blob[S: S + T * G * 16].view("<u2").reshape(T, G, 4, 2)   # [t, g, r, (scale, min)]
    scale_bits = tiles[:, :, :, 0].transpose(0, 2, 1).reshape(T * 4, G)
    min_bits = tiles[:, :, :, 1].transpose(0, 2, 1).reshape(T * 4, G)
    pad_codes = blob[N * K // 2: S]
    pad_rows = (scale_bits[N:], min_bits[N:])
    return codes, scale_bits[:N].view(np.float16), min_bits[:N].view(np.float16), pad_codes, pad_rows


@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (4, 96), (5, 128), (17, 2080), (64, 4096), (7, 14336)])
def test_pack_roundtrip_bit_exact(w4a16_lib, N, K):
    _, codes, scale, mn = workload.random_problem(N + K, 1, N, K)
    # make a few scale/min values special: -0, subnormal, max normal
    special = np.array([-0.0, 2.0 ** -24, 65504.0], dtype=np.float16)
    flat = scale.reshape(-1)
    flat[: min(3, flat.size)] = special[: min(3, flat.size)]
    blob = w4.w4a16_pack(codes, scale, mn)
    assert blob.size == w4.w4a16_packed_bytes(N, K)
    assert blob.size == HEADER_BYTES + _round_up(N * K // 2, 256) + ((N + 3) // 4) * (K // 32) * 16
    c2, s2, m2, pad_codes, pad_rows = unpack_blob(blob, N, K)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2.view(np.uint16), scale.view(np.uint16))
    np.testing.assert_array_equal(m2.view(np.uint16), mn.view(np.uint16))
    assert not pad_codes.any()
    assert not pad_rows[0].any() and not pad_rows[1].any()


def test_pack_slot_layout_by_hand(w4a16_lib):
    """One row, one group: k = 0..31 carries code k % 16; check the first word by hand."""
    q = np.arange(32) % 16
    codes = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)[None, :]
    scale = np.full((1, 1), 0.5, dtype=np.float16)
    mn = np.full((1, 1), -1.0, dtype=np.float16)
    blob = w4.w4a16_pack(codes, scale, mn)[HEADER_BYTES:]
    w0 = int(blob[:4].view("<u4")[0])
    # word 0 holds k = 0..7: even k (0,2,4,6) in the low half-word, odd (1,3,5,7) in the high
    assert w0 == (0 | 2 << 4 | 4 << 8 | 6 << 12) | ((1 | 3 << 4 | 5 << 8 | 7 << 12) << 16)
    w1 = int(blob[4:8].view("<u4")[0])     # k = 8..15
    assert w1 == (8 | 10 << 4 | 12 << 8 | 14 << 12) | ((9 | 11 << 4 | 13 << 8 | 15 << 12) << 16)
    sm = blob[256:256 + 16].view("<u2")
    assert sm[0] == np.float16(0.5).view(np.uint16) and sm[1] == np.float16(-1.0).view(np.uint16)
    assert not sm[2:].any()


def test_pack_large_uses_threads_and_matches(w4a16_lib):
    N, K = 1024, 8192        # 4 MiB of codes: large enough for the threaded path
    _, codes, scale, mn = workload.random_problem(77, 1, N, K)
    blob = w4.w4a16_pack(codes, scale, mn)
    c2, s2, m2, _, _ = unpack_blob(blob, N, K)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2.view(np.uint16), scale.view(np.uint16))
    np.testing.assert_array_equal(m2.view(np.uint16), mn.view(np.uint16))


def test_header_bytes_by_hand(w4a16_lib):
    """The header of a (3, 64) blob, byte by byte."""
    _, codes, scale, mn = workload.random_problem(5, 1, 3, 64)
    blob = w4.w4a16_pack(codes, scale, mn)
    total = blob.size
    assert total == 256 + 256 + 1 * 2 * 16
    want = bytearray(256)
    want[0:4] = b"W416"
    want[4:6] = (6).to_bytes(2, "little")
    want[6:8] = (0).to_bytes(2, "little")
    want[8:12] = (3).to_bytes(4, "little")
    want[12:16] = (64).to_bytes(4, "little")
    want[16:24] = total.to_bytes(8, "little")
    assert blob[:256].tobytes() == bytes(want)
    assert w4.w4a16_abi_version() == 6


def test_blob_check(w4a16_lib):
    """w4a16_blob_check accepts the blob of its own (codec, N, K) and refuses
    every other reading of it, including the transposed shape of the same size."""
    N, K = 64, 224
    _, codes, scale, mn = workload.random_problem(9, 1, N, K)
    blob = w4.w4a16_pack(codes, scale, mn)
    assert w4.w4a16_blob_check(blob, "q4", N, K) == w4.W4A16_OK
    assert w4.w4a16_blob_check(blob, "q4", K, N) == w4.W4A16_ERR_FORMAT       # transposed
    assert w4.w4a16_blob_check(blob, "q4", N, K + 32) == w4.W4A16_ERR_FORMAT
    assert w4.w4a16_blob_check(blob, "q4_sym", N, K) == w4.W4A16_ERR_FORMAT   # another codec
    assert w4.w4a16_blob_check(blob[:-1], "q4", N, K) == w4.W4A16_ERR_SIZE    # truncated
    assert w4.w4a16_blob_check(blob[:100], "q4", N, K) == w4.W4A16_ERR_SIZE
    assert w4.w4a16_blob_check(blob, 9, N, K) == w4.W4A16_ERR_SHAPE
    for byte in (0, 4, 6, 8, 12, 16, 100, 255):                              # any changed header byte
        bad = blob.copy()
        bad[byte] ^= 0x01
        assert w4.w4a16_blob_check(bad, "q4", N, K) == w4.W4A16_ERR_FORMAT, byte


def test_blob_check_same_size_shapes(w4a16_lib):
    """(4096, 14336) and (14336, 4096) blobs have the same size; the header
    tells them apart (checked on small stand-ins of equal size: (8, 64) and (16, 32))."""
    assert w4.w4a16_packed_bytes(4096, 14336) == w4.w4a16_packed_bytes(14336, 4096)
    assert w4.w4a16_packed_bytes(8, 64) == w4.w4a16_packed_bytes(16, 32)
    _, codes, scale, mn = workload.random_problem(3, 1, 8, 64)
    blob = w4.w4a16_pack(codes, scale, mn)
    assert w4.w4a16_blob_check(blob, "q4", 8, 64) == w4.W4A16_OK
    assert w4.w4a16_blob_check(blob, "q4", 16, 32) == w4.W4A16_ERR_FORMAT
