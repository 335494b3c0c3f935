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


def test_python_constants_match_header():
    """Every numeric #define and enum value of include/w4a16.h that the binding
    mirrors has the same value there."""
    text = open(os.path.join(ROOT, "include", "w4a16.h")).read()
    defines = {m.group(1): int(m.group(2), 0) for m in re.finditer(r"#define (W4A16_\w+) (0x[0-9A-Fa-f]+|\d+)u?\b", text)}
    enums = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(W4A16_\w+) = (\d+)", text)}
    mirrored = {k: getattr(w4, k) for k in list(defines) + list(enums) if hasattr(w4, k)}
    assert len(mirrored) >= 15
    for k, v in mirrored.items():
        assert v == defines.get(k, enums.get(k)), k
    for name, cid in w4.CODEC_IDS.items():
        assert enums["W4A16_CODEC_" + name.upper()] == cid


def test_version_and_strings(w4a16_lib):
    assert w4.w4a16_abi_version() == 6
    for st in range(9):
        assert w4.w4a16_status_string(st) != "unknown status"
    assert w4.w4a16_status_string(99) == "unknown status"
    assert w4.w4a16_max_k(0) == 0 and w4.w4a16_max_k(9) == 0
    assert w4.w4a16_max_k(1) >= 131072 and w4.w4a16_max_k(8) >= 32768


def test_packed_bytes_rules(w4a16_lib):
    assert w4.w4a16_packed_bytes(0, 64) == 0
    assert w4.w4a16_packed_bytes(4, 16) == 0
    assert w4.w4a16_packed_bytes(4, 48) == 0
    assert w4.w4a16_packed_bytes(-1, 64) == 0
    assert w4.w4a16_packed_bytes(2**31 - 1, 2**16) == 0          # chunk index would overflow
    assert w4.w4a16_packed_bytes(4096, 4096) == 256 + 4096 * 2048 + 1024 * 128 * 16
    assert w4.w4a16_packed_bytes(3, 32) == 256 + 256 + 16


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
    # the timed variant validates the same way (fake event handles, never used on error)
    assert w4a16_lib.w4a16_gemv_timed(x or None, p or None, y or None, M, N, K, None, BASE, BASE) == status


def test_timed_entry_points_need_both_events(w4a16_lib):
    L = w4a16_lib
    good = (BASE, BASE + 2**20, BASE + 2**30, 1, 64, 64)
    assert L.w4a16_gemv_timed(*good, None, None, BASE) == w4.W4A16_ERR_NULL
    assert L.w4a16_gemv_timed(*good, None, BASE, None) == w4.W4A16_ERR_NULL
    ws = w4.W4A16_CHAIN_WORKSPACE_BYTES
    assert L.w4a16_gemv_chain_timed(BASE, 1, 1, BASE, ws, None, None, BASE) == w4.W4A16_ERR_NULL
    assert L.w4a16_gemv_chain_timed(BASE, 1, 1, BASE, ws, None, BASE, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_gemv_chain_timed(BASE, 0, 1, BASE, ws, None, BASE, BASE) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemv_chain_timed(BASE, 1, 1, BASE, ws - 4, None, BASE, BASE) == w4.W4A16_ERR_SIZE


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
    # the kernel name carries the mode: one wave per tile / waves split K / passes over K
    assert shp(1, 4096, 2048)["kernel"] == "gemv_kernel<1, 1, 0>"
    assert shp(1, 6144, 4096)["kernel"] == "gemv_kernel<1, 1, 1>"
    assert shp(1, 4096, 14336)["kernel"] == "gemv_kernel<1, 1, 1>"
    assert shp(1, 64, 2**20)["kernel"].endswith(", 2>")


def test_chain_launch_shape(w4a16_lib):
    for M in range(1, 9):
        s = w4.chain_launch_shape(M)
        assert s["M"] == M and s["ring"] % 8 == 0 and s["compute_waves"] == 8
        assert s["kernel"] == f"chain_kernel<{M}, {s['ring']}, {s['compute_waves']}>"
        plan = w4.w4a16_chain_plan([(0x7F0000000000, 0x7F0001000000, 0x7F0040000000, 64, 64)], M)
        hdr = plan[:64].view("<i4")
        assert (hdr[4], hdr[5]) == (s["ring"], s["compute_waves"])    # the plan is made for that kernel
    for M in (0, 9):
        with pytest.raises(w4.W4A16Error):
            w4.chain_launch_shape(M)
    assert w4a16_lib.w4a16_chain_launch_shape(1, None) == w4.W4A16_ERR_NULL


# ------------------------------------------------------------ decode-step chain

def _plan_fields(plan, count):
    hdr = plan[:64].view("<u4")
    ents = []
    for i in range(count):
        raw = plan[64 + 64 * i: 128 + 64 * i]
        ptrs = raw[:32].view("<u8")
        ints = raw[32:56].view("<i4")
        blob = raw[56:64].view("<u8")
        ents.append((*[int(p) for p in ptrs], *[int(v) for v in ints], int(blob[0])))
    return hdr, ents


def test_chain_plan_layout(w4a16_lib):
    B = 0x7F0000000000
    entries = [
        (B, B + 2**24, B + 2**30, 6144, 4096),                    # two segments of 64 groups
        (B + 2**20, B + 2**26, B + 2**30 + 2**20, 4096, 14336),   # seven segments, one LDS pass
        (B + 2**21, B + 2**28, B + 2**30 + 2**21, 10, 28672),     # fourteen segments, two passes
        (B + 2**30 + 2**20, B + 2**29, B + 2**31, 64, 64),        # x is the second entry's y
    ]
    plan = w4.w4a16_chain_plan(entries, 1)
    assert plan.size == w4.w4a16_chain_plan_bytes(4) == 64 + 4 * 64
    hdr, ents = _plan_fields(plan, 4)
    shape = w4.chain_launch_shape(1)
    assert (hdr[0], hdr[1], hdr[2], hdr[3]) == (0x48433457, 5, 4, 1)
    assert (hdr[4], hdr[5]) == (shape["ring"], shape["compute_waves"]) == (24, 8)
    for (x, p, y, N, K), e in zip(entries, ents):
        ex, ecodes, esm, ey, eN, eG, eT, S, passes, xcoh, pad = e
        assert (ex, ecodes, ey, eN, eG, eT) == (x, p + 256, y, N, K // 32, (N + 3) // 4)
        assert esm == p + 256 + (N * K // 2 + 255) // 256 * 256
        assert S * 64 >= K // 32 > (S - 1) * 64               # segments of 64 groups, one per lane
    assert all(e[10] == 0 for e in ents)                   # padding
    # M = 1: 8 segments of activations per LDS pass; only the last x is written by an earlier entry
    assert [e[7:10] for e in ents] == [(2, 1, 0), (7, 1, 0), (14, 2, 0), (1, 1, 1)]
    plan8 = w4.w4a16_chain_plan(entries[:2], 8)
    hdr8, e8 = _plan_fields(plan8, 2)
    assert (hdr8[3], hdr8[4]) == (8, w4.chain_launch_shape(8)["ring"])
    # M = 8: one segment of 8 activation rows per pass
    assert [e[7:10] for e in e8] == [(2, 2, 0), (7, 7, 0)]


def test_chain_plan_errors(w4a16_lib):
    L = w4a16_lib
    B = 0x7F0000000000
    good = (B, B + 2**24, B + 2**30, 64, 64)
    buf = np.zeros(4096, np.uint8)

    def plan(entries, M=1, nbytes=None):
        arr = (w4.ChainEntry * len(entries))(*[w4.ChainEntry(*e) for e in entries])
        return L.w4a16_chain_plan(arr, len(entries), M, buf.ctypes.data, buf.nbytes if nbytes is None else nbytes)

    assert plan([good]) == w4.W4A16_OK
    assert L.w4a16_chain_plan(None, 1, 1, buf.ctypes.data, buf.nbytes) == w4.W4A16_ERR_NULL
    assert plan([(0, B + 2**24, B + 2**30, 64, 64)]) == w4.W4A16_ERR_NULL
    assert plan([good], M=0) == w4.W4A16_ERR_SHAPE
    assert plan([good], M=9) == w4.W4A16_ERR_SHAPE
    assert plan([(B, B + 2**24, B + 2**30, 64, 48)]) == w4.W4A16_ERR_SHAPE
    assert plan([(B, B + 2**24, B + 2**30, 0, 64)]) == w4.W4A16_ERR_SHAPE
    assert plan([(B + 8, B + 2**24, B + 2**30, 64, 64)]) == w4.W4A16_ERR_ALIGN
    assert plan([(B, B + 2**24 + 16, B + 2**30, 64, 64)]) == w4.W4A16_ERR_ALIGN
    assert plan([good], nbytes=127) == w4.W4A16_ERR_SIZE
    assert plan([(B, B + 2**24, B + 32, 64, 64)]) == w4.W4A16_ERR_OVERLAP          # y over its own x
    # a later entry's y lands inside an earlier entry's weights
    assert plan([good, (B + 2**20, B + 2**25, B + 2**24 + 512, 64, 64)]) == w4.W4A16_ERR_OVERLAP
    # a later entry reading an earlier entry's y is the allowed dependency
    assert plan([good, (B + 2**30, B + 2**25, B + 2**31, 64, 64)]) == w4.W4A16_OK
    assert L.w4a16_chain_plan_bytes(0) == 0 and L.w4a16_chain_plan_bytes(-3) == 0
    assert L.w4a16_chain_plan_bytes(2**20) == 64 + 2**20 * 64 and L.w4a16_chain_plan_bytes(2**20 + 1) == 0


def test_chain_call_rejects_before_any_hip_call(w4a16_lib):
    L = w4a16_lib
    B = 0x7F0000000000
    W = w4.W4A16_CHAIN_WORKSPACE_BYTES
    assert L.w4a16_gemv_chain(None, 1, 1, B, W, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_gemv_chain(B, 1, 1, None, W, None) == w4.W4A16_ERR_NULL
    assert L.w4a16_gemv_chain(B, 0, 1, B + 4096, W, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemv_chain(B, 1, 9, B + 4096, W, None) == w4.W4A16_ERR_SHAPE
    assert L.w4a16_gemv_chain(B + 8, 1, 1, B + 4096, W, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_gemv_chain(B, 1, 1, B + 4100, W, None) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_gemv_chain(B, 1, 1, B + 4096, W - 1, None) == w4.W4A16_ERR_SIZE
    assert L.w4a16_gemv_chain(B, 1, 1, B + 4096, 256, None) == w4.W4A16_ERR_SIZE


def test_chain_status_rejects_before_any_hip_call(w4a16_lib):
    import ctypes

    L = w4a16_lib
    B = 0x7F0000000000
    W = w4.W4A16_CHAIN_WORKSPACE_BYTES
    bits = ctypes.c_uint32(77)
    assert L.w4a16_chain_status(None, W, None, ctypes.byref(bits), 0) == w4.W4A16_ERR_NULL
    assert L.w4a16_chain_status(B, W, None, None, 0) == w4.W4A16_ERR_NULL
    assert bits.value == 77                                  # untouched on NULL
    assert L.w4a16_chain_status(B + 4, W, None, ctypes.byref(bits), 1) == w4.W4A16_ERR_ALIGN
    assert L.w4a16_chain_status(B, W - 1, None, ctypes.byref(bits), 1) == w4.W4A16_ERR_SIZE
    assert L.w4a16_chain_status(B, 256, None, ctypes.byref(bits), 0) == w4.W4A16_ERR_SIZE


# ------------------------------------------------------ binding argument checks
def test_binding_refuses_host_and_strided_tensors_before_any_gpu_call(w4a16_lib):
    """The library takes bare device addresses: the binding refuses host
    tensors, non-tensors and mismatched byte buffers with ValueError before
    anything reaches it (these run on a machine without a GPU)."""
    torch = pytest.importorskip("torch")
    M, N, K = 1, 8, 64
    x = torch.zeros((M, K), dtype=torch.float16)
    y = torch.zeros((M, N), dtype=torch.float32)
    packed = torch.zeros(w4.w4a16_packed_bytes(N, K), dtype=torch.uint8)
    with pytest.raises(ValueError, match="not on a GPU"):
        w4.w4a16_gemv(x, packed, y)
    with pytest.raises(ValueError, match="torch tensor"):
        w4._device_tensors("w4a16_gemv", packed=packed.numpy())
    with pytest.raises(ValueError, match="not on a GPU"):
        w4.w4a16_codec_gemv("q8_sym", x, packed, y)
    with pytest.raises(ValueError, match="not on a GPU"):
        w4.w4a16_gemv_chain(packed, 1, 1, torch.zeros(16, dtype=torch.int32))
    with pytest.raises(ValueError, match="not on a GPU"):
        w4.w4a16_chain_status(torch.zeros(16, dtype=torch.int32))
    q = torch.zeros((4, 128), dtype=torch.float16)
    o = torch.zeros((4, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="not on a GPU"):
        w4.w4a16_kv_attention(8, q, packed, o, 1, 1, torch.zeros(16))
    # the per-tensor rules, checked directly (no GPU needed to build the fakes)

    class Fake:
        def __init__(self, device="cuda:0", contiguous=True, dtype="torch.uint8"):
            self.is_cuda, self.device, self.dtype, self._c = True, device, dtype, contiguous

        def is_contiguous(self):
            return self._c

        def data_ptr(self):
            return 0x7F0000000000

    w4._device_tensors("t", x=Fake(dtype="torch.float16"), packed=Fake())
    with pytest.raises(ValueError, match="contiguous"):
        w4._device_tensors("t", x=Fake(), packed=Fake(contiguous=False))
    with pytest.raises(ValueError, match="uint8"):
        w4._device_tensors("t", packed=Fake(dtype="torch.int32"))
    with pytest.raises(ValueError, match="other tensors"):
        w4._device_tensors("t", x=Fake(device="cuda:0"), y=Fake(device="cuda:1"))
