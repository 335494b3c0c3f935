"""Thin ctypes binding of libw4a16 (the C ABI in include/w4a16.h).

Argument marshalling only: every step of the product runs in the library's
host repacker and gfx950 kernels. PyTorch, when used, only supplies device
memory and the current stream. If the library is not built this module
raises; it never falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libw4a16.so")

W4A16_OK = 0
W4A16_ERR_NULL = 1
W4A16_ERR_SHAPE = 2
W4A16_ERR_ALIGN = 3
W4A16_ERR_SIZE = 4
W4A16_ERR_OVERLAP = 5
W4A16_ERR_HIP = 6
W4A16_ERR_FORMAT = 7
W4A16_ERR_WAIT = 8

# weight-code variants (enum w4a16_codec)
CODEC_IDS = {"q4": 0, "q4_sym": 1, "q5": 2, "q8_sym": 3, "pal4": 4}

# every symbol include/w4a16.h declares
EXPORTS = (
    "w4a16_abi_version",
    "w4a16_max_k",
    "w4a16_packed_bytes",
    "w4a16_pack",
    "w4a16_gemv",
    "w4a16_launch_shape",
    "w4a16_chain_plan_bytes",
    "w4a16_chain_plan",
    "w4a16_chain_launch_shape",
    "w4a16_gemv_timed",
    "w4a16_gemv_chain_timed",
    "w4a16_gemv_chain",
    "w4a16_status_string",
    "w4a16_codec_packed_bytes",
    "w4a16_codec_pack",
    "w4a16_codec_gemv",
    "w4a16_codec_gemv_timed",
    "w4a16_codec_launch_shape",
    "w4a16_kv_packed_bytes",
    "w4a16_kv_pack",
    "w4a16_kv_workspace_bytes",
    "w4a16_kv_attention",
    "w4a16_kv_attention_timed",
    "w4a16_kv_launch_shape",
    "w4a16_blob_check",
    "w4a16_blob_mismatches",
    "w4a16_kv_attention_static",
    "w4a16_chain_status",
)

W4A16_CHAIN_WORKSPACE_BYTES = 69632
W4A16_CHAIN_MAX_ENTRIES = 1048576
W4A16_CHAIN_ERROR_OFFSET = 256  # uint32 error word of the chain workspace, a set of these bits:
W4A16_CHAIN_ERR_WAIT = 1        # an ordering wait gave up
W4A16_CHAIN_ERR_PLAN = 2        # the plan header does not match (count, M)
W4A16_CHAIN_ERR_BLOB = 4        # an entry's blob header does not match its (N, K)

W4A16_BLOB_MAGIC = 0x36313457   # first four bytes of every packed weight blob
W4A16_LAYOUT_VERSION = 6
W4A16_BLOB_HEADER_BYTES = 256
W4A16_KV_STATIC_WORKSPACE_BYTES = 8 << 20


class ChainEntry(ctypes.Structure):
    """struct w4a16_chain_entry of include/w4a16.h."""
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32)]

_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {w4a16_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libw4a16.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    c_i32, c_sz, c_vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    L.w4a16_abi_version.restype = c_i32
    L.w4a16_abi_version.argtypes = []
    L.w4a16_max_k.restype = c_i32
    L.w4a16_max_k.argtypes = [c_i32]
    L.w4a16_packed_bytes.restype = c_sz
    L.w4a16_packed_bytes.argtypes = [c_i32, c_i32]
    L.w4a16_pack.restype = c_i32
    L.w4a16_pack.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_sz]
    L.w4a16_gemv.restype = c_i32
    L.w4a16_gemv.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp]
    L.w4a16_launch_shape.restype = c_i32
    L.w4a16_launch_shape.argtypes = [c_i32, c_i32, c_i32, ctypes.POINTER(c_i32)]
    L.w4a16_chain_plan_bytes.restype = c_sz
    L.w4a16_chain_plan_bytes.argtypes = [c_i32]
    L.w4a16_chain_plan.restype = c_i32
    L.w4a16_chain_plan.argtypes = [ctypes.POINTER(ChainEntry), c_i32, c_i32, c_vp, c_sz]
    L.w4a16_chain_launch_shape.restype = c_i32
    L.w4a16_chain_launch_shape.argtypes = [c_i32, ctypes.POINTER(c_i32)]
    L.w4a16_gemv_timed.restype = c_i32
    L.w4a16_gemv_timed.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
    L.w4a16_gemv_chain_timed.restype = c_i32
    L.w4a16_gemv_chain_timed.argtypes = [c_vp, c_i32, c_i32, c_vp, c_sz, c_vp, c_vp, c_vp]
    L.w4a16_gemv_chain.restype = c_i32
    L.w4a16_gemv_chain.argtypes = [c_vp, c_i32, c_i32, c_vp, c_sz, c_vp]
    L.w4a16_chain_status.restype = c_i32
    L.w4a16_chain_status.argtypes = [c_vp, c_sz, c_vp, ctypes.POINTER(ctypes.c_uint32), c_i32]
    L.w4a16_codec_packed_bytes.restype = c_sz
    L.w4a16_codec_packed_bytes.argtypes = [c_i32, c_i32, c_i32]
    L.w4a16_codec_pack.restype = c_i32
    L.w4a16_codec_pack.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_sz]
    L.w4a16_codec_gemv.restype = c_i32
    L.w4a16_codec_gemv.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp]
    L.w4a16_codec_gemv_timed.restype = c_i32
    L.w4a16_codec_gemv_timed.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
    L.w4a16_codec_launch_shape.restype = c_i32
    L.w4a16_codec_launch_shape.argtypes = [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_i32)]
    L.w4a16_kv_packed_bytes.restype = c_sz
    L.w4a16_kv_packed_bytes.argtypes = [c_i32, c_i32, c_i32]
    L.w4a16_kv_pack.restype = c_i32
    L.w4a16_kv_pack.argtypes = [c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_sz]
    L.w4a16_kv_workspace_bytes.restype = c_sz
    L.w4a16_kv_workspace_bytes.argtypes = [c_i32, c_i32]
    L.w4a16_kv_attention.restype = c_i32
    L.w4a16_kv_attention.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp]
    L.w4a16_kv_attention_timed.restype = c_i32
    L.w4a16_kv_attention_timed.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp, c_vp, c_vp]
    L.w4a16_kv_launch_shape.restype = c_i32
    L.w4a16_kv_launch_shape.argtypes = [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_i32)]
    L.w4a16_status_string.restype = ctypes.c_char_p
    L.w4a16_status_string.argtypes = [c_i32]
    L.w4a16_blob_check.restype = c_i32
    L.w4a16_blob_check.argtypes = [c_vp, c_sz, c_i32, c_i32, c_i32]
    L.w4a16_kv_attention_static.restype = c_i32
    L.w4a16_kv_attention_static.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp]
    L.w4a16_blob_mismatches.restype = c_i32
    L.w4a16_blob_mismatches.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    _lib = L
    return L


def w4a16_abi_version() -> int:
    return int(lib().w4a16_abi_version())


def w4a16_max_k(M: int) -> int:
    return int(lib().w4a16_max_k(M))


def w4a16_status_string(status: int) -> str:
    return lib().w4a16_status_string(int(status)).decode()


def w4a16_packed_bytes(N: int, K: int) -> int:
    return int(lib().w4a16_packed_bytes(int(N), int(K)))


def w4a16_blob_check(blob: np.ndarray, codec, N: int, K: int) -> int:
    """Status of w4a16_blob_check on a host blob (W4A16_OK if it is a blob of
    this layout for (codec, N, K) and holds all of its bytes)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    if blob.nbytes < W4A16_BLOB_HEADER_BYTES:
        return W4A16_ERR_SIZE
    return int(lib().w4a16_blob_check(blob.ctypes.data, blob.nbytes, codec_id(codec), int(N), int(K)))


def w4a16_blob_mismatches() -> int:
    """Launches on the current device since the last call whose blob header
    did not match their call (they wrote nothing); resets the count."""
    out = ctypes.c_uint32(0)
    st = lib().w4a16_blob_mismatches(ctypes.byref(out))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_blob_mismatches")
    return int(out.value)


def w4a16_pack(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Host repack: codes uint8[N, K/2], scale/min float16[N, K/32] -> uint8 blob."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float16)
    mn = np.ascontiguousarray(mn, dtype=np.float16)
    N, Kh = codes.shape
    K = 2 * Kh
    nbytes = w4a16_packed_bytes(N, K)
    if out is None:
        out = np.empty(max(nbytes, 1), dtype=np.uint8)
    if scale.shape != (N, K // 32) or mn.shape != (N, K // 32):
        raise ValueError("scale and min must be [N, K/32]")
    st = lib().w4a16_pack(codes.ctypes.data, scale.ctypes.data, mn.ctypes.data, N, K,
                          out.ctypes.data, out.nbytes)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_pack")
    return out


def w4a16_launch_shape(M: int, N: int, K: int) -> dict:
    """(groups per lane, waves per workgroup, passes over K) w4a16_gemv would use."""
    out = (ctypes.c_int32 * 3)()
    st = lib().w4a16_launch_shape(M, N, K, out)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_launch_shape")
    mode = 2 if out[2] > 1 else 1 if out[1] > 1 else 0     # direct / block / multi-pass kernel
    return {"groups_per_lane": out[0], "waves": out[1], "k_passes": out[2],
            "kernel": f"gemv_kernel<{M}, {out[0]}, {mode}>"}


def chain_launch_shape(M: int) -> dict:
    """Template arguments of the kernel w4a16_gemv_chain launches for M."""
    out = (ctypes.c_int32 * 3)()
    st = lib().w4a16_chain_launch_shape(M, out)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_chain_launch_shape")
    return {"M": out[0], "ring": out[1], "compute_waves": out[2],
            "kernel": f"chain_kernel<{out[0]}, {out[1]}, {out[2]}>"}


def _ptr(t) -> int:
    return int(t.data_ptr()) if hasattr(t, "data_ptr") else int(t)


def _device_tensors(where: str, **tensors) -> None:
    """Raise ValueError unless every named tensor is a contiguous GPU tensor
    and all of them sit on the same device: the library receives bare device
    addresses, so a host tensor or a strided view would be read as garbage
    (or fault the GPU) rather than refused. Byte buffers (packed blobs,
    plans) must be uint8. Nothing here touches the GPU."""
    device = None
    for name, t in tensors.items():
        if not hasattr(t, "is_cuda") or not hasattr(t, "data_ptr"):
            raise ValueError(f"{where}: {name} must be a torch tensor on the GPU")
        if not t.is_cuda:
            raise ValueError(f"{where}: {name} is on {t.device}, not on a GPU")
        if not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{where}: {name} is on {t.device}, the other tensors on {device}")
        if name in ("packed", "kv", "plan") and str(t.dtype) != "torch.uint8":
            raise ValueError(f"{where}: {name} must be a uint8 byte buffer, not {t.dtype}")


def w4a16_gemv_raw(x_ptr: int, packed_ptr: int, y_ptr: int, M: int, N: int, K: int, stream: int = 0) -> int:
    """Direct C call with raw pointers; returns the status code."""
    return int(lib().w4a16_gemv(x_ptr, packed_ptr, y_ptr, M, N, K, stream))


def w4a16_gemv_timed_raw(x_ptr: int, packed_ptr: int, y_ptr: int, M: int, N: int, K: int, stream: int,
                         start_event: int, stop_event: int) -> int:
    """w4a16_gemv_timed with raw pointers and hipEvent_t handles; returns the status code."""
    return int(lib().w4a16_gemv_timed(x_ptr, packed_ptr, y_ptr, M, N, K, stream, start_event, stop_event))


def w4a16_gemv(x, packed, y, stream=None) -> None:
    """y[M, N] = x[M, K] @ w_hat.T on the GPU, enqueued on `stream`.

    x: device float16 [M, K]; packed: device uint8 blob from w4a16_pack;
    y: device float32 [M, N], overwritten. `stream` is a torch stream, a raw
    hipStream_t integer, or None for torch's current stream.
    """
    if str(x.dtype) != "torch.float16" or str(y.dtype) != "torch.float32":
        raise TypeError("x must be float16 and y float32")
    if x.dim() != 2 or y.dim() != 2:
        raise ValueError("x must be [M, K] and y [M, N]")
    _device_tensors("w4a16_gemv", x=x, packed=packed, y=y)
    M, K = int(x.shape[0]), int(x.shape[1])
    N = int(y.shape[-1])
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N] with the same M as x")
    need = w4a16_packed_bytes(N, K)
    if need == 0:
        raise W4A16Error(W4A16_ERR_SHAPE, "w4a16_gemv")
    if packed.numel() * packed.element_size() < need:
        raise ValueError(f"packed blob has {packed.numel() * packed.element_size()} bytes, needs {need}")
    if stream is None:
        import torch  # only for the current stream handle

        s = torch.cuda.current_stream(x.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        s = stream.cuda_stream
    else:
        s = int(stream)
    st = w4a16_gemv_raw(_ptr(x), _ptr(packed), _ptr(y), M, N, K, s)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemv")


def upload_packed(blob: np.ndarray, device="cuda"):
    """Copy a host blob from w4a16_pack to a 256-byte-aligned device uint8 tensor."""
    import torch

    host = torch.from_numpy(np.ascontiguousarray(blob, dtype=np.uint8))
    dev = torch.empty(host.numel() + 256, dtype=torch.uint8, device=device)
    off = (-dev.data_ptr()) % 256
    view = dev[off:off + host.numel()]
    view.copy_(host)
    return view


def w4a16_chain_plan_bytes(count: int) -> int:
    return int(lib().w4a16_chain_plan_bytes(int(count)))


def w4a16_chain_plan(entries, M: int) -> np.ndarray:
    """Host plan for w4a16_gemv_chain.

    entries: sequence of (x, packed, y, N, K) where x/packed/y are device
    tensors or raw device addresses. Returns the plan as a host uint8 array;
    copy it to device memory (16-byte aligned) before calling the chain.
    """
    n = len(entries)
    arr = (ChainEntry * max(n, 1))()
    for i, (x, packed, y, N, K) in enumerate(entries):
        arr[i] = ChainEntry(_ptr(x), _ptr(packed), _ptr(y), int(N), int(K))
    nbytes = w4a16_chain_plan_bytes(n)
    out = np.zeros(max(nbytes, 1), dtype=np.uint8)
    st = lib().w4a16_chain_plan(arr, n, int(M), out.ctypes.data, out.nbytes if nbytes else 0)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_chain_plan")
    return out


def w4a16_gemv_chain_raw(plan_ptr: int, count: int, M: int, workspace_ptr: int, workspace_bytes: int,
                         stream: int = 0) -> int:
    """Direct C call with raw pointers; returns the status code."""
    return int(lib().w4a16_gemv_chain(plan_ptr, int(count), int(M), workspace_ptr, int(workspace_bytes), stream))


def w4a16_gemv_chain_timed_raw(plan_ptr: int, count: int, M: int, workspace_ptr: int, workspace_bytes: int,
                               stream: int, start_event: int, stop_event: int) -> int:
    """w4a16_gemv_chain_timed with raw pointers and hipEvent_t handles; returns the status code."""
    return int(lib().w4a16_gemv_chain_timed(plan_ptr, int(count), int(M), workspace_ptr, int(workspace_bytes),
                                            stream, start_event, stop_event))


def _stream_handle(stream) -> int:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def w4a16_gemv_chain(plan, count: int, M: int, workspace, stream=None, check: bool = False) -> None:
    """Enqueue a planned decode-step chain (plan and workspace are device tensors).

    check=True waits for the call and raises W4A16Error (W4A16_ERR_WAIT or
    W4A16_ERR_FORMAT) if it raised a bit of the workspace's error word; the
    word is then cleared with the rest of the workspace."""
    _device_tensors("w4a16_gemv_chain", plan=plan, workspace=workspace)
    s = _stream_handle(stream)
    st = w4a16_gemv_chain_raw(_ptr(plan), count, M, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), s)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemv_chain")
    if check:
        st, bits = w4a16_chain_status_raw(_ptr(workspace), workspace.numel() * workspace.element_size(), s, True)
        if st != W4A16_OK:
            raise W4A16Error(st, f"w4a16_gemv_chain (error word {bits:#x})")


def w4a16_chain_status_raw(workspace_ptr: int, workspace_bytes: int, stream: int, clear: bool) -> tuple:
    """w4a16_chain_status with raw pointers; returns (status code, error bits)."""
    bits = ctypes.c_uint32(0)
    st = int(lib().w4a16_chain_status(workspace_ptr, int(workspace_bytes), stream, ctypes.byref(bits), int(bool(clear))))
    return st, int(bits.value)


def w4a16_chain_status(workspace, stream=None, clear: bool = False) -> int:
    """Wait for the chain calls enqueued on `stream` and return the error bits
    of their workspace (0: every result valid); clear=True zero-fills the
    workspace again when a bit was set. Raises W4A16Error on host errors."""
    _device_tensors("w4a16_chain_status", workspace=workspace)
    st, bits = w4a16_chain_status_raw(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream_handle(stream), clear)
    if st not in (W4A16_OK, W4A16_ERR_WAIT, W4A16_ERR_FORMAT):
        raise W4A16Error(st, "w4a16_chain_status")
    return bits


# ---------------------------------------------------------------------------
# weight-code variants
# ---------------------------------------------------------------------------


def codec_id(codec) -> int:
    """Codec name ("q4", "q4_sym", "q5", "q8_sym") or id -> the C enum value."""
    if isinstance(codec, str):
        if codec not in CODEC_IDS:
            raise ValueError(f"unknown codec {codec!r}")
        return CODEC_IDS[codec]
    return int(codec)


def w4a16_codec_packed_bytes(codec, N: int, K: int) -> int:
    return int(lib().w4a16_codec_packed_bytes(codec_id(codec), int(N), int(K)))


def w4a16_codec_pack(codec, codes: np.ndarray, scale: np.ndarray, mn: np.ndarray | None = None) -> np.ndarray:
    """Host repack of one codec's canonical arrays into a uint8 blob.

    codes: uint8[N, K/2] for the 4-bit codecs, uint8[N, K] (values < 32) for
    "q5", int8[N, K] for "q8_sym"; scale (and min, affine codecs only)
    float16[N, K/32]; for "pal4" scale carries the palettes, float16[N, 16].
    """
    cid = codec_id(codec)
    codes = np.ascontiguousarray(codes)
    if codes.dtype not in (np.uint8, np.int8):
        raise TypeError("codes must be uint8 or int8")
    N = codes.shape[0]
    K = codes.shape[1] * (2 if cid in (0, 1, 4) else 1)
    scale = np.ascontiguousarray(scale, dtype=np.float16)
    if scale.shape != ((N, 16) if cid == 4 else (N, K // 32)):
        raise ValueError("scale must be [N, K/32] ([N, 16] palettes for pal4)")
    mp = None
    if mn is not None:
        mn = np.ascontiguousarray(mn, dtype=np.float16)
        if mn.shape != (N, K // 32):
            raise ValueError("min must be [N, K/32]")
        mp = mn.ctypes.data
    nbytes = w4a16_codec_packed_bytes(cid, N, K)
    out = np.empty(max(nbytes, 1), dtype=np.uint8)
    st = lib().w4a16_codec_pack(cid, codes.ctypes.data, scale.ctypes.data, mp, N, K, out.ctypes.data, out.nbytes)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_codec_pack")
    return out


def w4a16_codec_launch_shape(codec, M: int, N: int, K: int) -> dict:
    """(groups per lane, waves, passes over K) and the kernel name w4a16_codec_gemv would use."""
    cid = codec_id(codec)
    out = (ctypes.c_int32 * 3)()
    st = lib().w4a16_codec_launch_shape(cid, M, N, K, out)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_codec_launch_shape")
    mode = 2 if out[2] > 1 else 1 if out[1] > 1 else 0
    name = (f"gemv_kernel<{M}, {out[0]}, {mode}>" if cid == 0 else f"codec_kernel<{cid}, {M}, {out[0]}, {mode}>")
    return {"groups_per_lane": out[0], "waves": out[1], "k_passes": out[2], "kernel": name}


def w4a16_codec_gemv_raw(codec, x_ptr: int, packed_ptr: int, y_ptr: int, M: int, N: int, K: int,
                         stream: int = 0) -> int:
    """Direct C call with raw pointers; returns the status code."""
    return int(lib().w4a16_codec_gemv(codec_id(codec), x_ptr, packed_ptr, y_ptr, M, N, K, stream))


def w4a16_codec_gemv_timed_raw(codec, x_ptr: int, packed_ptr: int, y_ptr: int, M: int, N: int, K: int,
                               stream: int, start_event: int, stop_event: int) -> int:
    """w4a16_codec_gemv_timed with raw pointers and hipEvent_t handles; returns the status code."""
    return int(lib().w4a16_codec_gemv_timed(codec_id(codec), x_ptr, packed_ptr, y_ptr, M, N, K, stream,
                                            start_event, stop_event))


def w4a16_codec_gemv(codec, x, packed, y, stream=None) -> None:
    """y[M, N] = x[M, K] @ w_hat.T for a blob from w4a16_codec_pack (device tensors)."""
    if str(x.dtype) != "torch.float16" or str(y.dtype) != "torch.float32":
        raise TypeError("x must be float16 and y float32")
    if x.dim() != 2 or y.dim() != 2 or int(y.shape[0]) != int(x.shape[0]):
        raise ValueError("x must be [M, K] and y [M, N]")
    _device_tensors("w4a16_codec_gemv", x=x, packed=packed, y=y)
    M, K, N = int(x.shape[0]), int(x.shape[1]), int(y.shape[1])
    need = w4a16_codec_packed_bytes(codec, N, K)
    if need == 0:
        raise W4A16Error(W4A16_ERR_SHAPE, "w4a16_codec_gemv")
    if packed.numel() * packed.element_size() < need:
        raise ValueError(f"packed blob has {packed.numel() * packed.element_size()} bytes, needs {need}")
    if stream is None:
        import torch

        s = torch.cuda.current_stream(x.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        s = stream.cuda_stream
    else:
        s = int(stream)
    st = w4a16_codec_gemv_raw(codec, _ptr(x), _ptr(packed), _ptr(y), M, N, K, s)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_codec_gemv")


# ---------------------------------------------------------------------------
# decode attention over a quantised KV cache
# ---------------------------------------------------------------------------


def w4a16_kv_packed_bytes(bits: int, T: int, Hkv: int) -> int:
    return int(lib().w4a16_kv_packed_bytes(int(bits), int(T), int(Hkv)))


def w4a16_kv_workspace_bytes(T: int, Hq: int) -> int:
    return int(lib().w4a16_kv_workspace_bytes(int(T), int(Hq)))


def w4a16_kv_pack(bits: int, k_codes, k_scale, k_min, v_codes, v_scale, v_min) -> np.ndarray:
    """Host repack of one layer's canonical cache (see include/w4a16.h) into a uint8 blob."""
    k_codes = np.ascontiguousarray(k_codes)
    v_codes = np.ascontiguousarray(v_codes)
    T, Hkv = int(k_codes.shape[0]), int(k_codes.shape[1])
    want = (T, Hkv, 128 if bits == 8 else 64)
    if k_codes.shape != want or v_codes.shape != want:
        raise ValueError(f"codes must be {want}")
    arrs = []
    for a in (k_scale, k_min, v_scale, v_min):
        if a is None:
            arrs.append(None)
            continue
        a = np.ascontiguousarray(a, dtype=np.float16)
        if a.shape != (T, Hkv, 4):
            raise ValueError("scales and mins must be [T, Hkv, 4]")
        arrs.append(a)
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    nbytes = w4a16_kv_packed_bytes(bits, T, Hkv)
    out = np.empty(max(nbytes, 1), dtype=np.uint8)
    st = lib().w4a16_kv_pack(int(bits), k_codes.ctypes.data, ptr(arrs[0]), ptr(arrs[1]), v_codes.ctypes.data,
                             ptr(arrs[2]), ptr(arrs[3]), T, Hkv, out.ctypes.data, out.nbytes)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_kv_pack")
    return out


def w4a16_kv_launch_shape(bits: int, T: int, Hq: int, Hkv: int) -> dict:
    out = (ctypes.c_int32 * 3)()
    st = lib().w4a16_kv_launch_shape(int(bits), int(T), int(Hq), int(Hkv), out)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_kv_launch_shape")
    return {"heads_per_kv_head": out[0], "blocks_per_workgroup": out[1], "workgroups_per_kv_head": out[2],
            "kernel": f"kv_attn_kernel<{int(bits)}, {out[0]}>", "merge_kernel": f"kv_combine_kernel<{out[0]}>"}


def w4a16_kv_attention_raw(bits: int, q_ptr: int, kv_ptr: int, o_ptr: int, T: int, Hq: int, Hkv: int,
                           ws_ptr: int, ws_bytes: int, stream: int = 0) -> int:
    """Direct C call with raw pointers; returns the status code."""
    return int(lib().w4a16_kv_attention(int(bits), q_ptr, kv_ptr, o_ptr, int(T), int(Hq), int(Hkv), ws_ptr,
                                        int(ws_bytes), stream))


def w4a16_kv_attention_timed_raw(bits: int, q_ptr: int, kv_ptr: int, o_ptr: int, T: int, Hq: int, Hkv: int,
                                 ws_ptr: int, ws_bytes: int, stream: int, start_event: int, stop_event: int) -> int:
    return int(lib().w4a16_kv_attention_timed(int(bits), q_ptr, kv_ptr, o_ptr, int(T), int(Hq), int(Hkv), ws_ptr,
                                              int(ws_bytes), stream, start_event, stop_event))


def w4a16_kv_attention_static_raw(bits: int, q_ptr: int, kv_ptr: int, o_ptr: int, T: int, Hq: int, Hkv: int,
                                  stream: int = 0) -> int:
    """w4a16_kv_attention_static with raw device pointers; returns the status code."""
    return int(lib().w4a16_kv_attention_static(int(bits), q_ptr, kv_ptr, o_ptr, int(T), int(Hq), int(Hkv), stream))


def w4a16_kv_attention(bits: int, q, kv, o, T: int, Hkv: int, workspace, stream=None) -> None:
    """o[Hq, 128] for one layer (device tensors: q float16 [Hq, 128], kv the
    uploaded packed cache, o float32 [Hq, 128], workspace any device buffer of
    w4a16_kv_workspace_bytes(T, Hq) bytes)."""
    if str(q.dtype) != "torch.float16" or str(o.dtype) != "torch.float32":
        raise TypeError("q must be float16 and o float32")
    if q.dim() != 2 or tuple(o.shape) != tuple(q.shape) or int(q.shape[1]) != 128:
        raise ValueError("q and o must be [Hq, 128]")
    _device_tensors("w4a16_kv_attention", q=q, kv=kv, o=o, workspace=workspace)
    Hq = int(q.shape[0])
    need = w4a16_kv_packed_bytes(bits, T, Hkv)
    if need == 0 or kv.numel() * kv.element_size() < need:
        raise ValueError(f"packed cache too small or bad shape (needs {need} bytes)")
    if stream is None:
        import torch

        s = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        s = stream.cuda_stream
    else:
        s = int(stream)
    st = w4a16_kv_attention_raw(bits, _ptr(q), _ptr(kv), _ptr(o), T, Hq, Hkv, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), s)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_kv_attention")
