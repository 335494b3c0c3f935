"""The codec repacker (w4a16_codec_pack) against an independent decode of the
layouts in include/w4a16.h, plus its error paths. No GPU.

`decode_blob` is written from the header's layout text only: the 4-bit chunk
slots (slot p of a word holds i = 2p for p < 4, else 2(p-4)+1), the fifth-bit
word (bit 4j + d is the code of k = 8d + 2(j mod 4) + j/4), the 8-bit halves
(low halves of every group, then high halves; bytes 0..3 of word e hold
i = 0, 2, 1, 3, each q + 128), the 8- or 16-byte parameter tiles and the
palette tiles (entry c of row 4t + r at byte 8c + 2r of tile t). It shares
no code with the C++ repacker. Packing then decoding must give back the
canonical arrays bit for bit, and every padding byte must be zero.
"""
import numpy as np
import pytest

import bit_weight_quantized_w4a16_amd as w4
import workload
from blob_header import HEADER_BYTES, strip_header


def _round_up(v, a):
    return (v + a - 1) // a * a


def _nibble_codes(words, N, G):
    """4-bit chunk words [N, G, 4] -> per-k codes [N, 32 G]."""
    q = np.empty((N, G, 4, 8), dtype=np.int64)
    for p in range(8):
        i = 2 * p if p < 4 else 2 * (p - 4) + 1
        q[:, :, :, i] = (words >> (4 * p)) & 0xF
    return q.reshape(N, 32 * G)


def _tiles(blob, off, T, G, entry):
    """Parameter tiles -> per-row arrays of uint16 bits [4T, G, entry // 8]."""
    t = blob[off: off + T * G * entry].view("<u2").reshape(T, G, 4, entry // 8)
    return t.transpose(0, 2, 1, 3).reshape(4 * T, G, entry // 8)


def decode_blob(codec, blob, N, K):
    blob = strip_header(blob, w4.CODEC_IDS[codec], N, K)
    G, T = K // 32, (N + 3) // 4
    code_bytes = N * G * (32 if codec == "q8_sym" else 16)
    S = _round_up(code_bytes, 256)
    pads = [blob[code_bytes:S]]
    mn = None
    if codec == "pal4":  # canonical bytes, then per tile: entry c of row r at byte 8c + 2r
        codes = blob[:code_bytes].reshape(N, K // 2).copy()
        T = (N + 3) // 4
        assert blob.size == S + T * 128
        lut = blob[S: S + T * 128].view("<u2").reshape(T, 16, 4).transpose(0, 2, 1).reshape(4 * T, 16)
        pads.append(lut[N:])
        return codes, lut[:N].copy().view(np.float16), None, pads
    if codec in ("q4_sym", "q5"):
        words = blob[:code_bytes].view("<u4").reshape(N, G, 4).astype(np.int64)
        q = _nibble_codes(words, N, G)
    if codec == "q4_sym":
        codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
        par = _tiles(blob, S, T, G, 8)
        end = S + T * G * 8
    elif codec == "q5":
        hb = blob[S: S + T * G * 16].view("<u4").reshape(T, G, 4).transpose(0, 2, 1).reshape(4 * T, G)
        pads.append(hb[N:])
        hb = hb[:N].astype(np.int64)
        fifth = np.zeros((N, G, 32), dtype=np.int64)
        for b in range(32):
            j, d = b // 4, b % 4
            fifth[:, :, 8 * d + 2 * (j % 4) + j // 4] = (hb >> b) & 1
        codes = (q + 16 * fifth.reshape(N, K)).astype(np.uint8)
        par = _tiles(blob, S + T * G * 16, T, G, 16)
        end = S + 2 * T * G * 16
    else:
        raw = blob[:code_bytes].reshape(N, 2, G, 4, 4).astype(np.int64)   # [n, half, g, word e, byte slot]
        q = np.empty((N, G, 2, 4, 4), dtype=np.int64)                      # [n, g, half, e, i]
        for slot, i in enumerate((0, 2, 1, 3)):
            q[:, :, :, :, i] = raw[:, :, :, :, slot].transpose(0, 2, 1, 3)
        codes = (q.reshape(N, K) - 128).astype(np.int8)
        par = _tiles(blob, S, T, G, 8)
        end = S + T * G * 8
    assert blob.size == end
    scale = par[:N, :, 0].copy().view(np.float16)
    if codec == "q5":
        mn = par[:N, :, 1].copy().view(np.float16)
    pads.append(par[N:])
    return codes, scale, mn, pads


SHAPES = [(1, 32), (3, 64), (4, 96), (5, 128), (17, 2080), (9, 4096), (7, 14336)]


@pytest.mark.parametrize("codec", ["q4_sym", "q5", "q8_sym", "pal4"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_codec_pack_roundtrip_bit_exact(w4a16_lib, codec, N, K):
    codes, scale, mn = workload.codec_weights(codec, 77, N, K % 7, N, K)
    scale.reshape(-1)[: min(3, scale.size)] = np.array([-0.0, 2.0 ** -24, 65504.0], np.float16)[: min(3, scale.size)]
    blob = w4.w4a16_codec_pack(codec, codes, scale, mn)
    assert blob.size == w4.w4a16_codec_packed_bytes(codec, N, K)
    c2, s2, m2, pads = decode_blob(codec, blob, N, K)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2.view(np.uint16), scale.view(np.uint16))
    if codec == "q5":
        np.testing.assert_array_equal(m2.view(np.uint16), mn.view(np.uint16))
    for p in pads:
        assert not np.asarray(p).any()


def test_q5_fifth_bits_by_hand(w4a16_lib):
    """One row, one group: only k = 5 has the fifth bit; it is bit 4j + d with d = 0, j = 6."""
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 5] = 16
    blob = w4.w4a16_codec_pack("q5", codes, np.ones((1, 1), np.float16), np.zeros((1, 1), np.float16))
    body = blob[HEADER_BYTES:]
    word = int(body[256:260].view("<u4")[0])
    assert word == 1 << 24          # k = 5 = 8*0 + 2*(6 mod 4) + 6//4  ->  b = 4*6 + 0
    assert not body[:16].any()      # the low nibbles are all zero


def test_q8_bytes_by_hand(w4a16_lib):
    """k = 0..3 of the low half: bytes hold k = 0, 2, 1, 3 as q + 128."""
    codes = np.zeros((1, 32), np.int8)
    codes[0, :4] = [-128, 1, 2, 127]
    blob = w4.w4a16_codec_pack("q8_sym", codes, np.ones((1, 1), np.float16))[HEADER_BYTES:]
    assert list(blob[:4]) == [0, 130, 129, 255]
    assert list(blob[4:32]) == [128] * 28   # the rest of both halves: q = 0


def test_codec_q4_is_w4a16_pack(w4a16_lib):
    codes, scale, mn = workload.codec_weights("q4", 5, 0, 0, 13, 256)
    np.testing.assert_array_equal(w4.w4a16_codec_pack("q4", codes, scale, mn), w4.w4a16_pack(codes, scale, mn))
    assert w4.w4a16_codec_packed_bytes("q4", 13, 256) == w4.w4a16_packed_bytes(13, 256)


def test_codec_pack_errors(w4a16_lib):
    L = w4.lib()
    one = np.ones((2, 2), np.float16)
    out = np.zeros(4096, np.uint8)
    q5 = np.zeros((2, 64), np.uint8)
    # unknown codec, code above 31 (nothing written)
    assert L.w4a16_codec_pack(5, q5.ctypes.data, one.ctypes.data, one.ctypes.data, 2, 64, out.ctypes.data,
                              out.nbytes) == w4.W4A16_ERR_FORMAT
    bad = q5.copy()
    bad[1, 63] = 32
    out[:] = 0xAB
    assert L.w4a16_codec_pack(2, bad.ctypes.data, one.ctypes.data, one.ctypes.data, 2, 64, out.ctypes.data,
                              out.nbytes) == w4.W4A16_ERR_FORMAT
    assert (out == 0xAB).all()
    # an affine codec needs its min; a symmetric one does not
    assert L.w4a16_codec_pack(2, q5.ctypes.data, one.ctypes.data, None, 2, 64, out.ctypes.data,
                              out.nbytes) == w4.W4A16_ERR_NULL
    assert L.w4a16_codec_pack(3, q5.ctypes.data, one.ctypes.data, None, 2, 64, out.ctypes.data,
                              out.nbytes) == w4.W4A16_OK
    assert L.w4a16_codec_pack(1, q5.ctypes.data, one.ctypes.data, None, 2, 33, out.ctypes.data,
                              out.nbytes) == w4.W4A16_ERR_SHAPE
    need = w4.w4a16_codec_packed_bytes("q8_sym", 2, 64)
    assert L.w4a16_codec_pack(3, q5.ctypes.data, one.ctypes.data, None, 2, 64, out.ctypes.data,
                              need - 1) == w4.W4A16_ERR_SIZE
    assert w4.w4a16_codec_packed_bytes(9, 4, 64) == 0 and w4.w4a16_codec_packed_bytes(5, 4, 64) == 0 and w4.w4a16_codec_packed_bytes("q5", 4, 48) == 0


@pytest.mark.parametrize("codec,expect", [("q4_sym", 18 / 32), ("q5", 24 / 32), ("q8_sym", 34 / 32),
                                          ("pal4", 16 / 32 + 32 / 4096)])
def test_codec_bytes_per_weight(w4a16_lib, codec, expect):
    N, K = 4096, 4096
    assert w4.w4a16_codec_packed_bytes(codec, N, K) == HEADER_BYTES + N * K * expect


def test_codec_gemv_rejects_before_any_hip_call(w4a16_lib):
    L = w4.lib()
    x, p, y = 0x10000, 0x20000, 0x40000
    assert L.w4a16_codec_gemv(5, x, p, y, 1, 8, 64, None) == w4.W4A16_ERR_FORMAT
    assert L.w4a16_codec_gemv(-1, x, p, y, 1, 8, 64, None) == w4.W4A16_ERR_FORMAT
    assert L.w4a16_codec_gemv(2, None, p, y, 1, 8, 64, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_codec_gemv(2, x, p, y, 9, 8, 64, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_codec_gemv(3, x, p, y, 1, 8, 48, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_codec_gemv(1, x + 8, p, y, 1, 8, 64, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_codec_gemv(1, x, p + 16, y, 1, 8, 64, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_codec_gemv(2, x, p, p + 64, 1, 8, 64, None) == w4.W4A16_ERR_OVERLAP
    assert L.w4a16_codec_gemv_timed(2, x, p, y, 1, 8, 64, None, None, None) == w4.W4A16_ERR_NULL


def test_codec_launch_shapes(w4a16_lib):
    for codec, cid in (("q4_sym", 1), ("q5", 2), ("q8_sym", 3), ("pal4", 4)):
        s = w4.w4a16_codec_launch_shape(codec, 1, 4096, 4096)
        assert s["kernel"] == f"codec_kernel<{cid}, 1, 1, 1>" and s["waves"] == 2
        s = w4.w4a16_codec_launch_shape(codec, 1, 4096, 14336)
        assert s["kernel"] == f"codec_kernel<{cid}, 1, 1, 1>" and s["waves"] == 7
        s = w4.w4a16_codec_launch_shape(codec, 8, 37, 131072)
        assert s["k_passes"] > 1 and s["kernel"].endswith(", 2>")
    for shape in ((1, 4096, 4096), (4, 6144, 4096), (8, 37, 131072)):
        assert w4.w4a16_codec_launch_shape("q4", *shape) == w4.w4a16_launch_shape(*shape)
    out = (__import__("ctypes").c_int32 * 3)()
    assert w4.lib().w4a16_codec_launch_shape(7, 1, 8, 64, out) == w4.W4A16_ERR_FORMAT
    assert w4.lib().w4a16_codec_launch_shape(1, 0, 8, 64, out) == w4.W4A16_ERR_SHAPE
