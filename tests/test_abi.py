"""The C-ABI library without a GPU: exported symbols and host-side error paths.

Every w4a16_gemv call here is rejected by argument validation before the
library touches the HIP runtime, so no compute is attempted. The pointers are
fake addresses that are never dereferenced.
"""
import os
import re
import subprocess

import numpy as np
import pytest

import bit_weight_quantized_w4a16_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(w4a16_\w+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported(w4a16_lib):
    declared = _declared_symbols()
    assert declared == set(w4.EXPORTS)
    for name in declared:
        assert hasattr(w4a16_lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", w4.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (w4a16_\w+)", out))
    assert declared <= exported


def test_version_and_strings(w4a16_lib):
    assert w4.w4a16_abi_version() == 1
    for st in range(7):
        assert w4.w4a16_status_string(st)
    assert w4.w4a16_status_string(99) == "unknown status"
    assert w4.w4a16_max_k(0) == 0 and w4.w4a16_max_k(9) == 0
    assert w4.w4a16_max_k(1) >= 131072 and w4.w4a16_max_k(8) >= 32768


def test_packed_bytes_rules(w4a16_lib):
    assert w4.w4a16_packed_bytes(0, 64) == 0
    assert w4.w4a16_packed_bytes(4, 16) == 0
    assert w4.w4a16_packed_bytes(4, 48) == 0
    assert w4.w4a16_packed_bytes(-1, 64) == 0
    assert w4.w4a16_packed_bytes(2**31 - 1, 2**16) == 0          # chunk index would overflow
    assert w4.w4a16_packed_bytes(4096, 4096) == 4096 * 2048 + 1024 * 128 * 16
    assert w4.w4a16_packed_bytes(3, 32) == 256 + 16


def test_pack_errors(w4a16_lib):
    L = w4a16_lib
    codes = np.zeros((4, 32), np.uint8)
    sc = np.zeros((4, 2), np.float16)
    out = np.full(w4.w4a16_packed_bytes(4, 64), 0xAB, np.uint8)
    c, s, o = codes.ctypes.data, sc.ctypes.data, out.ctypes.data
    assert L.w4a16_pack(None, s, s, 4, 64, o, out.nbytes) == w4.W4A16_ERR_NULL
    assert L.w4a16_pack(c, None, s, 4, 64, o, out.nbytes) == w4.W4A16_ERR_NULL
    assert L.w4a16_pack(c, s, None, 4, 64, o, out.nbytes) == w4.W4A16_ERR_NULL
    assert L.w4a16_pack(c, s, s, 4, 64, None, out.nbytes) == w4.W4A16_ERR_NULL
    assert L.w4a16_pack(c, s, s, 4, 63, o, out.nbytes) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_pack(c, s, s, 0, 64, o, out.nbytes) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_pack(c, s, s, 4, 64, o, out.nbytes - 1) == w4.W4A16_ERR_SIZE
    assert (out == 0xAB).all()           # nothing written on error
    assert L.w4a16_pack(c, s, s, 4, 64, o, out.nbytes) == w4.W4A16_OK


BASE = 0x7F0000000000   # fake, never dereferenced


@pytest.mark.parametrize("args,status", [
    ((0, BASE, BASE + 2**30, 1, 64, 64), w4.W4A16_ERR_NULL),
    ((BASE, 0, BASE + 2**30, 1, 64, 64), w4.W4A16_ERR_NULL),
    ((BASE, BASE + 2**20, 0, 1, 64, 64), w4.W4A16_ERR_NULL),
    ((BASE, BASE + 2**20, BASE + 2**30, 0, 64, 64), w4.W4A16_ERR_SHAPE),
    ((BASE, BASE + 2**20, BASE + 2**30, 9, 64, 64), w4.W4A16_ERR_SHAPE),
    ((BASE, BASE + 2**20, BASE + 2**30, 1, 0, 64), w4.W4A16_ERR_SHAPE),
    ((BASE, BASE + 2**20, BASE + 2**30, 1, 64, 0), w4.W4A16_ERR_SHAPE),
    ((BASE, BASE + 2**20, BASE + 2**30, 1, 64, 16), w4.W4A16_ERR_SHAPE),
    ((BASE, BASE + 2**20, BASE + 2**30, 1, 64, 48), w4.W4A16_ERR_SHAPE),
    ((BASE, BASE + 2**20, BASE + 2**30, 1, 64, 2**21), w4.W4A16_ERR_SHAPE),
    ((BASE + 2, BASE + 2**20, BASE + 2**30, 1, 64, 64), w4.W4A16_ERR_ALIGN),
    ((BASE + 8, BASE + 2**20, BASE + 2**30, 1, 64, 64), w4.W4A16_ERR_ALIGN),
    ((BASE, BASE + 2**20 + 128, BASE + 2**30, 1, 64, 64), w4.W4A16_ERR_ALIGN),
    ((BASE, BASE + 2**20, BASE + 2**30 + 2, 1, 64, 64), w4.W4A16_ERR_ALIGN),
    ((BASE, BASE + 2**20, BASE + 64, 1, 64, 64), w4.W4A16_ERR_OVERLAP),          # y inside x
    ((BASE, BASE + 2**20, BASE + 2**20 + 1024, 1, 64, 64), w4.W4A16_ERR_OVERLAP),  # y inside packed
    ((BASE + 256, BASE + 2**20, BASE, 2, 64, 64), w4.W4A16_ERR_OVERLAP),          # y runs into x
])
def test_gemv_rejects_before_any_hip_call(w4a16_lib, args, status):
    x, p, y, M, N, K = args
    assert w4a16_lib.w4a16_gemv(x or None, p or None, y or None, M, N, K, None) == status


def test_binding_checks(w4a16_lib):
    torch = pytest.importorskip("torch")
    x = torch.zeros(2, 64, dtype=torch.float32)
    y = torch.zeros(2, 4, dtype=torch.float32)
    with pytest.raises(TypeError):
        w4.w4a16_gemv(x, torch.zeros(1, dtype=torch.uint8), y)
    x = torch.zeros(2, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        w4.w4a16_gemv(x, torch.zeros(16, dtype=torch.uint8), y)   # blob too small
    with pytest.raises(ValueError):
        w4.w4a16_gemv(x, torch.zeros(10**6, dtype=torch.uint8), torch.zeros(3, 4))


def test_launch_shape_host_logic(w4a16_lib):
    shp = w4.w4a16_launch_shape
    a = shp(1, 6144, 4096)
    assert a["groups_per_lane"] * 64 * a["waves"] >= 4096 // 32 and a["k_passes"] == 1
    b = shp(8, 8192, 28672)
    per_pass = b["groups_per_lane"] * 64 * b["waves"]
    assert per_pass * b["k_passes"] >= 28672 // 32
    for M in range(1, 9):
        for K in (32, 96, 4096, 14336, 28672, 131072):
            s = shp(M, 5, K)
            assert s["groups_per_lane"] in (1, 2, 4) and 1 <= s["waves"] <= 16
            assert s["groups_per_lane"] * 64 * s["waves"] * s["k_passes"] >= K // 32
    with pytest.raises(w4.W4A16Error):
        shp(9, 5, 64)
    assert w4a16_lib.w4a16_launch_shape(1, 1, 64, None) == w4.W4A16_ERR_NULL
