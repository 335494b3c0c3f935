"""Decode of the 256-byte header that starts every packed weight blob,
written from the header text in include/w4a16.h (little endian: uint32 magic
at byte 0, uint16 layout version at 4, uint16 codec at 6, int32 N at 8, int32
K at 12, uint64 blob bytes at 16, zeros to byte 256). Shares no code with the
C++ packer."""
import numpy as np

HEADER_BYTES = 256
MAGIC = b"W416"
LAYOUT_VERSION = 6


def read_header(blob):
    """(magic bytes, version, codec, N, K, total bytes, tail is all zero)."""
    h = np.asarray(blob[:HEADER_BYTES], dtype=np.uint8)
    assert h.size == HEADER_BYTES
    raw = h.tobytes()
    return (raw[0:4], int.from_bytes(raw[4:6], "little"), int.from_bytes(raw[6:8], "little"),
            int.from_bytes(raw[8:12], "little", signed=True), int.from_bytes(raw[12:16], "little", signed=True),
            int.from_bytes(raw[16:24], "little"), not any(raw[24:]))


def strip_header(blob, codec, N, K):
    """Check the header against (codec, N, K, blob size) and return the bytes after it."""
    magic, version, cid, n, k, total, zero_tail = read_header(blob)
    assert magic == MAGIC
    assert version == LAYOUT_VERSION
    assert (cid, n, k) == (codec, N, K)
    assert total == blob.size
    assert zero_tail
    return blob[HEADER_BYTES:]
