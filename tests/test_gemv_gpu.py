"""GPU parity: the gfx950 kernels through the C ABI against the fp64 oracle.

Pass rule per element: |y_gpu - y_ref| <= 1e-3 * B + 1e-5, B = sum_k |w_hat x|.
Small shapes are compared in full; the named Llama-shaped workloads are run at
their full sizes with the same launch the bench uses, and compared in full
where the oracle is fast enough, otherwise on sampled rows (first, last and a
seeded random set, so every tile position and the ragged tail are hit).
"""
import numpy as np
import pytest

import bit_weight_quantized_w4a16_amd as w4
import oracle
import workload
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _device_inputs(x, codes, scale, mn):
    blob = w4.w4a16_pack(codes, scale, mn)
    packed = w4.upload_packed(blob, DEV)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return xd, packed


def run_gpu(x, codes, scale, mn, stream=None):
    xd, packed = _device_inputs(x, codes, scale, mn)
    M, N = x.shape[0], codes.shape[0]
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    w4.w4a16_gemv(xd, packed, y, stream)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def sample_rows(N, seed, count=384):
    rng = np.random.default_rng(seed)
    rows = set(range(min(N, 8))) | set(range(max(0, N - 8), N))
    rows |= set(rng.choice(N, size=min(N, count), replace=False).tolist())
    return np.array(sorted(rows))


# ---------------------------------------------------------------- small shapes

SMALL = [
    (1, 1, 32), (1, 3, 64), (1, 4, 96), (1, 5, 160), (2, 17, 2080), (3, 33, 4096),
    (4, 7, 4128), (5, 9, 8192), (6, 65, 2048), (7, 12, 6176), (8, 4097, 256),
    (1, 4097, 4096), (8, 13, 14336), (1, 9, 16416), (2, 11, 65536), (8, 6, 16416),
]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_shapes_full(w4a16_lib, M, N, K):
    print(f"[shape] M={M} N={N} K={K}", flush=True)
    x, codes, scale, mn = workload.random_problem(M * 131 + N * 7 + K, M, N, K, outliers=(K >= 1000))
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn)
    check(y, y_ref, B, f"M={M} N={N} K={K}", inputs=(x, codes, scale, mn))


# Enough tiles that a workgroup walks several of them (two load buffers
# alternating, then a tail of one or two tiles) at 5..8 activation rows, with
# ragged N and, at K = 4128, a ragged K slot of a three-wave split.
SEVERAL_TILES = [(5, 24579, 2080), (6, 16387, 2080), (7, 12291, 4128), (8, 8195, 2080)]


@pytest.mark.parametrize("M,N,K", SEVERAL_TILES)
def test_several_tiles_per_workgroup_full(w4a16_lib, M, N, K):
    print(f"[shape] M={M} N={N} K={K}", flush=True)
    x, codes, scale, mn = workload.random_problem(M * 977 + N, M, N, K, outliers=True)
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn, threads=8)
    check(y, y_ref, B, f"M={M} N={N} K={K}", inputs=(x, codes, scale, mn))


@pytest.mark.parametrize("M,K", [(1, 131072), (1, 131104), (8, 32800), (4, 32768)])
def test_long_k_multi_pass(w4a16_lib, M, K):
    """K beyond one pass of a workgroup: partial sums carried across passes."""
    N = 37
    print(f"[shape] M={M} N={N} K={K}", flush=True)
    x, codes, scale, mn = workload.random_problem(K + M, M, N, K, outliers=True)
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn)
    check(y, y_ref, B, f"M={M} N={N} K={K}", inputs=(x, codes, scale, mn))


# --------------------------------------------------------- closed forms, edges

@pytest.mark.parametrize("M,N,K", [(1, 64, 4096), (8, 21, 14336)])
def test_zero_weights_give_exact_zero(w4a16_lib, M, N, K):
    x, codes, scale, _ = workload.random_problem(11, M, N, K, outliers=True)
    codes[:] = 0
    mn = np.zeros_like(scale)
    y = run_gpu(x, codes, scale, mn)
    assert np.array_equal(y, np.zeros_like(y))


def test_zero_codes_closed_form(w4a16_lib):
    M, N, K = 3, 100, 4096
    x, codes, scale, mn = workload.random_problem(12, M, N, K)
    codes[:] = 0
    y = run_gpu(x, codes, scale, mn)
    xs = x.astype(np.float64).reshape(M, K // 32, 32).sum(axis=2)
    expect = xs @ mn.astype(np.float64).T
    _, B = oracle.gemv(x, codes, scale, mn)
    check(y, expect, B, "zero codes", inputs=(x, codes, scale, mn))


def test_one_hot_x_picks_weights(w4a16_lib):
    N, K = 24, 256
    _, codes, scale, mn = workload.random_problem(13, 1, N, K)
    w_hat = oracle.dequantise(codes, scale, mn)
    xd, packed = _device_inputs(np.zeros((1, K), np.float16), codes, scale, mn)
    for k in [0, 1, 2, 3, 5, 8, 31, 32, 33, 100, 255]:
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        xd.copy_(torch.from_numpy(x))
        y = torch.empty((1, N), dtype=torch.float32, device=DEV)
        w4.w4a16_gemv(xd, packed, y)
        torch.cuda.synchronize()
        got = y.cpu().numpy()[0].astype(np.float64)
        # a single nonzero product: exact up to one fp32 rounding of w_hat
        np.testing.assert_allclose(got, w_hat[:, k], rtol=2 ** -23, atol=1e-30)


def test_zero_x_gives_zero(w4a16_lib):
    _, codes, scale, mn = workload.random_problem(14, 2, 40, 512)
    y = run_gpu(np.zeros((2, 512), np.float16), codes, scale, mn)
    assert np.array_equal(y, np.zeros_like(y))


def test_bitwise_repeatable_and_stream_ordered(w4a16_lib):
    M, N, K = 1, 6144, 4096
    x, codes, scale, mn = workload.random_problem(15, M, N, K, outliers=True)
    xd, packed = _device_inputs(x, codes, scale, mn)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())  # the uploads ran on the current stream
    ys = []
    with torch.cuda.stream(s):
        for _ in range(3):
            y = torch.empty((M, N), dtype=torch.float32, device=DEV)
            w4.w4a16_gemv(xd, packed, y, s)
            ys.append(y)
    s.synchronize()
    a = ys[0].cpu().numpy()
    for y in ys[1:]:
        assert np.array_equal(a.view(np.uint32), y.cpu().numpy().view(np.uint32))
    y_ref, B = oracle.gemv(x, codes, scale, mn)
    check(a.astype(np.float64), y_ref, B, "stream", inputs=(x, codes, scale, mn))


def test_timed_launch_matches_and_times_the_kernel(w4a16_lib):
    M, N, K = 1, 4096, 14336
    x, codes, scale, mn = workload.random_problem(16, M, N, K, outliers=True)
    xd, packed = _device_inputs(x, codes, scale, mn)
    s = torch.cuda.Stream(device=DEV)
    y0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.wait_stream(torch.cuda.current_stream())  # the uploads and the NaN fill ran on the current stream
    with torch.cuda.stream(s):
        a.record(s)
        b.record(s)
        w4.w4a16_gemv(xd, packed, y0, s)
        st = w4.w4a16_gemv_timed_raw(xd.data_ptr(), packed.data_ptr(), y1.data_ptr(), M, N, K, s.cuda_stream,
                                     a.cuda_event, b.cuda_event)
    assert st == w4.W4A16_OK
    s.synchronize()
    assert torch.equal(y0, y1)
    assert 0.0 < a.elapsed_time(b) < 100.0        # ms: the kernel itself, a few microseconds


def test_y_is_overwritten_not_accumulated(w4a16_lib):
    M, N, K = 2, 50, 1024
    x, codes, scale, mn = workload.random_problem(16, M, N, K)
    xd, packed = _device_inputs(x, codes, scale, mn)
    y = torch.full((M, N), 1e6, dtype=torch.float32, device=DEV)
    w4.w4a16_gemv(xd, packed, y)
    torch.cuda.synchronize()
    y_ref, B = oracle.gemv(x, codes, scale, mn)
    check(y.cpu().numpy().astype(np.float64), y_ref, B, "overwrite", inputs=(x, codes, scale, mn))


def test_fp16_extremes_in_x(w4a16_lib):
    M, N, K = 2, 30, 512
    x, codes, scale, mn = workload.random_problem(17, M, N, K)
    x[0, :8] = np.array([65504, -65504, 2 ** -24, -(2 ** -24), 2 ** -14, 0.0, -0.0, 1000], dtype=np.float16)
    x[1, ::3] = np.float16(2 ** -20)          # many subnormals
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn)
    check(y, y_ref, B, "fp16 extremes", inputs=(x, codes, scale, mn))


def test_beyond_4gib_of_weights_sampled(w4a16_lib):
    """A 5.4 GB packed matrix (ragged N = 262,147 rows at K = 32,768): the last
    rows' code chunks lie more than 2^32 bytes into the blob, so every load
    address is formed in 64 bits. Compared on sampled rows, the last eight
    included."""
    M, N, K = 1, 262147, 32768
    print(f"[shape] M={M} N={N} K={K} ({w4.w4a16_packed_bytes(N, K) / 1e9:.2f} GB packed)", flush=True)
    # seeded, non-periodic bytes drawn directly (the workload recipe's fp64
    # draws take most of a minute at this size): codes are uniform bytes,
    # scale and min uniform binary16 bit patterns in [0.001, 0.01] and [-0.08, 0]
    rng = np.random.default_rng(0x4D415847)
    codes = np.frombuffer(rng.bytes(N * K // 2), dtype=np.uint8).reshape(N, K // 2)
    lo, hi = np.float16(0.001).view(np.uint16), np.float16(0.01).view(np.uint16)
    scale = rng.integers(lo, hi + 1, size=(N, K // 32), dtype=np.uint16).view(np.float16)
    mn = (rng.integers(0, np.float16(0.08).view(np.uint16) + 1, size=(N, K // 32), dtype=np.uint16)
          | np.uint16(0x8000)).view(np.float16)
    x = workload.activations(77, 0, 0, M, K, True)
    assert codes.nbytes > 2**32
    y = run_gpu(x, codes, scale, mn)
    rows = sample_rows(N, 77, count=256)
    y_ref, B = oracle.gemv_rows(x, codes, scale, mn, rows)
    check(y[:, rows], y_ref, B, f"M={M} N={N} K={K}", inputs=(x, codes, scale, mn), rows=rows)


# ------------------------------------------------------ named Llama workloads

def test_gemv4096_full(w4a16_lib):
    x, codes, scale, mn = workload.gemv_inputs("gemv4096", 0, 0, 1)
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn)
    check(y, y_ref, B, "gemv4096", inputs=(x, codes, scale, mn))


@pytest.mark.parametrize("proj", [0, 1, 2, 3])
def test_llama8b_layer_full(w4a16_lib, proj):
    x, codes, scale, mn = workload.gemv_inputs("llama8b_layer", 0, proj, 1)
    print(f"[shape] llama8b_layer proj={proj} N={codes.shape[0]} K={x.shape[1]}", flush=True)
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn, threads=8)
    check(y, y_ref, B, f"llama8b_layer proj {proj}", inputs=(x, codes, scale, mn))


@pytest.mark.parametrize("M", [4, 8])
@pytest.mark.parametrize("proj", [0, 1, 2, 3])
def test_llama8b_verify_full(w4a16_lib, M, proj):
    x, codes, scale, mn = workload.gemv_inputs("llama8b_verify", 0, proj, M)
    print(f"[shape] llama8b_verify M={M} proj={proj} N={codes.shape[0]} K={x.shape[1]}", flush=True)
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn, threads=8)
    check(y, y_ref, B, f"llama8b_verify M={M} proj {proj}", inputs=(x, codes, scale, mn))


@pytest.mark.parametrize("layer", [0, 31])
@pytest.mark.parametrize("proj", [0, 1, 2, 3])
def test_llama8b_step_sampled(w4a16_lib, layer, proj):
    x, codes, scale, mn = workload.gemv_inputs("llama8b_step", layer, proj, 1)
    print(f"[shape] llama8b_step layer={layer} proj={proj} N={codes.shape[0]} K={x.shape[1]}", flush=True)
    y = run_gpu(x, codes, scale, mn)
    rows = sample_rows(codes.shape[0], layer * 4 + proj)
    y_ref, B = oracle.gemv_rows(x, codes, scale, mn, rows)
    check(y[:, rows], y_ref, B, f"llama8b_step layer {layer} proj {proj}", inputs=(x, codes, scale, mn), rows=rows)


@pytest.mark.parametrize("layer", [0, 79])
@pytest.mark.parametrize("proj", [0, 1, 2, 3])
def test_llama70b_tp8_shard(w4a16_lib, layer, proj):
    """One GPU's share of the 70B layer at 8-way tensor parallelism, in the
    launch the bench times: o's K of 1024 is 32 groups, half a wave's lanes."""
    x, codes, scale, mn = workload.gemv_inputs("llama70b_tp8", layer, proj, 1)
    print(f"[shape] llama70b_tp8 layer={layer} proj={proj} N={codes.shape[0]} K={x.shape[1]}", flush=True)
    y = run_gpu(x, codes, scale, mn)
    y_ref, B = oracle.gemv(x, codes, scale, mn, threads=8)
    check(y, y_ref, B, f"llama70b_tp8 layer {layer} proj {proj}", inputs=(x, codes, scale, mn))


@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("proj", [0, 1, 2, 3])
def test_llama70b_sampled(w4a16_lib, M, proj):
    layer = 79 if M == 8 else 0
    x, codes, scale, mn = workload.gemv_inputs("llama70b_step", layer, proj, M)
    print(f"[shape] llama70b_step M={M} layer={layer} proj={proj} N={codes.shape[0]} K={x.shape[1]}",
          flush=True)
    y = run_gpu(x, codes, scale, mn)
    rows = sample_rows(codes.shape[0], 100 + proj)
    y_ref, B = oracle.gemv_rows(x, codes, scale, mn, rows)
    check(y[:, rows], y_ref, B, f"llama70b M={M} proj {proj}", inputs=(x, codes, scale, mn), rows=rows)
