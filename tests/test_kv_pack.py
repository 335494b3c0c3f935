"""The KV-cache repacker (w4a16_kv_pack) against an independent decode of the
layout in include/w4a16.h, and the host-side checks of the attention call.
No GPU.

`decode_cache` follows the header text only: records of R bytes per
(KV head, 64-token block); words of four 8-bit elements hold elements
(0, 2, 1, 3) in bytes 0..3 as q + 128, words of eight 4-bit elements hold
element i in byte (0, 2, 1, 3)[i % 4], low nibble for i < 4 and high nibble
for i >= 4; INT8 key chunks of 16 dims per token, INT4 key chunks of one group
per token, and value loads of 16 (INT8) or 32 (INT4) tokens of one dim per
lane, dims 64h + lane. It shares no code with the C++ packer.
"""
import numpy as np
import pytest

import bit_weight_quantized_w4a16_amd as w4
import workload

SLOT = (0, 2, 1, 3)  # byte of element i (mod 4) of a word


def _bytes4(words):
    """Words of four 8-bit elements [..., 4 bytes] -> elements [..., 4] (q + 128 removed)."""
    out = np.empty(words.shape, dtype=np.int64)
    for i in range(4):
        out[..., i] = words[..., SLOT[i]].astype(np.int64) - 128
    return out


def _nibbles8(words):
    """Words of eight 4-bit elements [..., 4 bytes] -> elements [..., 8]."""
    out = np.empty(words.shape[:-1] + (8,), dtype=np.int64)
    for i in range(8):
        out[..., i] = (words[..., SLOT[i % 4]].astype(np.int64) >> (4 * (i // 4))) & 0xF
    return out


def decode_cache(bits, blob, T, Hkv):
    nb = (T + 63) // 64
    R = 17408 if bits == 8 else 10240
    assert blob.size == Hkv * nb * R
    recs = blob.reshape(Hkv, nb, R)
    Tp = nb * 64
    if bits == 8:
        kb = recs[:, :, :8192].reshape(Hkv, nb, 8, 64, 4, 4)                  # [g, b, chunk c, slot, word e, byte]
        k = _bytes4(kb).transpose(0, 1, 3, 2, 4, 5).reshape(Hkv, nb, 64, 128)  # dim 16c + 4e + i
        ks = recs[:, :, 8192:8704].copy().view("<u2").reshape(Hkv, nb, 64, 4)
        vs = recs[:, :, 8704:9216].copy().view("<u2").reshape(Hkv, nb, 64, 4)
        vb = recs[:, :, 9216:].reshape(Hkv, nb, 2, 4, 64, 4, 4)              # [g, b, h, tq, lane, word e, byte]
        v = _bytes4(vb)                                                        # token 16tq + 4e + i, dim 64h + lane
        v = v.transpose(0, 1, 3, 5, 6, 2, 4).reshape(Hkv, nb, 64, 128)
        km = vm = None
        to_codes = lambda a: a.transpose(1, 2, 0, 3).reshape(Tp, Hkv, 128)[:T].astype(np.int8)  # noqa: E731
        k_codes, v_codes = to_codes(k), to_codes(v)
    else:
        kb = recs[:, :, :4096].reshape(Hkv, nb, 4, 64, 4, 4)                  # [g, b, group c, slot, word, byte]
        kq = _nibbles8(kb).transpose(0, 1, 3, 2, 4, 5).reshape(Hkv, nb, 64, 128)  # dim 32c + 8 word + i
        k_codes = (kq[..., 0::2] | (kq[..., 1::2] << 4)).transpose(1, 2, 0, 3).reshape(Tp, Hkv, 64)[:T].astype(np.uint8)
        kp = recs[:, :, 4096:5120].copy().view("<u2").reshape(Hkv, nb, 64, 4, 2)
        vp = recs[:, :, 5120:6144].copy().view("<u2").reshape(Hkv, nb, 64, 4, 2)
        ks, km, vs, vm = kp[..., 0], kp[..., 1], vp[..., 0], vp[..., 1]
        vb = recs[:, :, 6144:].reshape(Hkv, nb, 2, 2, 64, 4, 4)              # [g, b, h, th, lane, word w, byte]
        vq = _nibbles8(vb)                                                     # token 32th + 8w + i, dim 64h + lane
        vq = vq.transpose(0, 1, 3, 5, 6, 2, 4).reshape(Hkv, nb, 64, 128)
        v_codes = (vq[..., 0::2] | (vq[..., 1::2] << 4)).transpose(1, 2, 0, 3).reshape(Tp, Hkv, 64)[:T].astype(np.uint8)
    par = lambda a: None if a is None else a.transpose(1, 2, 0, 3).reshape(Tp, Hkv, 4)[:T].copy().view(np.float16)  # noqa: E731
    return k_codes, par(ks), par(km), v_codes, par(vs), par(vm)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T,Hkv", [(1, 1), (63, 2), (64, 1), (65, 3), (200, 8)])
def test_kv_pack_roundtrip_bit_exact(w4a16_lib, bits, T, Hkv):
    cache = workload.kv_cache(bits, 9, T, T, Hkv)
    blob = w4.w4a16_kv_pack(bits, *cache)
    assert blob.size == w4.w4a16_kv_packed_bytes(bits, T, Hkv)
    got = decode_cache(bits, blob, T, Hkv)
    for a, b in zip(got, cache):
        if b is None:
            assert a is None
        else:
            np.testing.assert_array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    # slots past T are zero bytes: the blob equals that of the cache padded to whole blocks with
    # parameters 0 and the codes whose bytes are 0 (INT8 stores q + 128, so q = -128)
    Tp = ((T + 63) // 64) * 64
    fill = [-128 if bits == 8 else 0, 0, 0] * 2
    padded = [None if c is None else np.concatenate([c, np.full((Tp - T,) + c.shape[1:], f, c.dtype)])
              for c, f in zip(cache, fill)]
    np.testing.assert_array_equal(w4.w4a16_kv_pack(bits, *padded), blob)


def test_kv_pack_by_hand(w4a16_lib):
    """INT8: key dims 0..3 of token 0 land in bytes 0..3 as dims 0, 2, 1, 3 (+128);
    value dim d of token 1 lands at lane d, word 0, byte 2 of load 0.
    INT4: key dims 0..7 of token 0 land in word 0 as bytes (e0|e4<<4, e2|e6<<4,
    e1|e5<<4, e3|e7<<4); value dim 70 of token 9 lands in the low nibble of byte
    2 of word 1 of lane 6, load 2 (dims 64..127, tokens 0..31)."""
    T, Hkv = 2, 1
    k = np.zeros((T, Hkv, 128), np.int8)
    k[0, 0, :4] = [-128, 1, 2, 127]
    v = np.zeros((T, Hkv, 128), np.int8)
    v[1, 0, 6:8] = [5, -5]
    s = np.ones((T, Hkv, 4), np.float16)
    blob = w4.w4a16_kv_pack(8, k, s, None, v, s, None)
    assert list(blob[:4]) == [0, 130, 129, 255]
    assert blob[9216 + 6 * 16 + 2] == 133 and blob[9216 + 7 * 16 + 2] == 123

    T = 10
    k4 = np.zeros((T, Hkv, 64), np.uint8)
    k4[0, 0, :4] = [0x21, 0x43, 0x65, 0x87]   # dims 0..7 = 1..8
    v4 = np.zeros((T, Hkv, 64), np.uint8)
    v4[9, 0, 35] = 0x0A                       # dim 70 (even: low nibble) of token 9
    s4 = np.ones((T, Hkv, 4), np.float16)
    m4 = np.zeros((T, Hkv, 4), np.float16)
    blob = w4.w4a16_kv_pack(4, k4, s4, m4, v4, s4, m4)
    assert list(blob[:4]) == [0x51, 0x73, 0x62, 0x84]
    at = 6144 + 2 * 1024 + 6 * 16 + 4 * 1 + 2
    assert blob[at] == 0x0A
    assert np.count_nonzero(blob[6144:]) == 1


def test_kv_pack_and_call_errors(w4a16_lib):
    L = w4.lib()
    c = np.zeros((4, 2, 128), np.int8)
    s = np.ones((4, 2, 4), np.float16)
    out = np.zeros(1 << 16, np.uint8)
    assert L.w4a16_kv_pack(5, c.ctypes.data, s.ctypes.data, None, c.ctypes.data, s.ctypes.data, None, 4, 2,
                           out.ctypes.data, out.nbytes) == w4.W4A16_ERR_FORMAT
    assert L.w4a16_kv_pack(4, c.ctypes.data, s.ctypes.data, None, c.ctypes.data, s.ctypes.data, None, 4, 2,
                           out.ctypes.data, out.nbytes) == w4.W4A16_ERR_NULL
    assert L.w4a16_kv_pack(8, c.ctypes.data, s.ctypes.data, None, c.ctypes.data, s.ctypes.data, None, 0, 2,
                           out.ctypes.data, out.nbytes) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_kv_pack(8, c.ctypes.data, s.ctypes.data, None, c.ctypes.data, s.ctypes.data, None, 4, 2,
                           out.ctypes.data, 100) == w4.W4A16_ERR_SIZE
    assert w4.w4a16_kv_packed_bytes(8, 64, 8) == 8 * 17408 and w4.w4a16_kv_packed_bytes(4, 65, 8) == 16 * 10240
    assert w4.w4a16_kv_packed_bytes(6, 64, 8) == 0 and w4.w4a16_kv_workspace_bytes(0, 32) == 0
    # attention: host-side checks before anything is enqueued
    q, kv, o, ws = 0x10000, 0x100000, 0x200000, 0x300000
    nb = w4.w4a16_kv_workspace_bytes(1000, 32)
    assert L.w4a16_kv_attention(8, None, kv, o, 1000, 32, 8, ws, nb, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_kv_attention(8, q, kv, o, 1000, 32, 3, ws, nb, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_kv_attention(8, q, kv, o, 1000, 48, 3, ws, nb, None) == w4.W4A16_ERR_SHAPE   # 16 heads per KV head
    assert L.w4a16_kv_attention(5, q, kv, o, 1000, 32, 8, ws, nb, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_kv_attention(8, q + 8, kv, o, 1000, 32, 8, ws, nb, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_kv_attention(8, q, kv + 64, o, 1000, 32, 8, ws, nb, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_kv_attention(8, q, kv, o, 1000, 32, 8, ws, nb - 4, None) == w4.W4A16_ERR_SIZE
    assert L.w4a16_kv_attention(8, q, kv, kv + 256, 1000, 32, 8, ws, nb, None) == w4.W4A16_ERR_OVERLAP
    assert L.w4a16_kv_attention(8, q, kv, o, 1000, 32, 8, o + 1024, nb, None) == w4.W4A16_ERR_OVERLAP
    assert L.w4a16_kv_attention_timed(8, q, kv, o, 1000, 32, 8, ws, nb, None, None, None) == w4.W4A16_ERR_NULL


def test_kv_launch_shape(w4a16_lib):
    s = w4.w4a16_kv_launch_shape(8, 38863, 32, 8)
    assert s["heads_per_kv_head"] == 4 and s["blocks_per_workgroup"] % 4 == 0
    assert s["kernel"] == "kv_attn_kernel<8, 4>"
    nb = (38863 + 63) // 64
    assert s["workgroups_per_kv_head"] == -(-nb // s["blocks_per_workgroup"])
    # the workspace bound holds for the launch on any device
    assert w4.w4a16_kv_workspace_bytes(38863, 32) >= 32 * s["workgroups_per_kv_head"] * 130 * 4
