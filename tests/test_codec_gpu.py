"""GPU parity of the weight-code variants through the C ABI against the fp64
codec oracle, element by element, with the same pass rule as the 4-bit code:
|y_gpu - y_ref| <= 1e-3 * B + 1e-5.

Small and ragged shapes are compared in full; the Llama-3-8B layer shapes run
at full size in the bench's launch and are compared on sampled rows (first,
last and a seeded random set).
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
CODECS = ["q4_sym", "q5", "q8_sym", "pal4"]
C = oracle.codecs_ref


def run_codec(codec, x, codes, scale, mn):
    packed = w4.upload_packed(w4.w4a16_codec_pack(codec, codes, scale, mn), DEV)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    y = torch.full((x.shape[0], codes.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    w4.w4a16_codec_gemv(codec, xd, packed, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


SMALL = [
    (1, 1, 32), (1, 5, 160), (2, 17, 2080), (3, 33, 4096), (4, 7, 4128), (5, 9, 8192),
    (6, 65, 2048), (7, 12, 6176), (8, 4097, 256), (1, 4097, 4096), (8, 13, 14336), (1, 9, 16416),
]


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_codec_small_shapes_full(w4a16_lib, codec, M, N, K):
    print(f"[codec shape] {codec} M={M} N={N} K={K}", flush=True)
    x, codes, scale, mn = workload.random_codec_problem(codec, M * 131 + N * 7 + K, M, N, K, outliers=(K >= 1000))
    y = run_codec(codec, x, codes, scale, mn)
    y_ref, B = C.gemv(codec, x, codes, scale, mn)
    check(y, y_ref, B, f"{codec} M={M} N={N} K={K}", inputs=(x, codes, scale, mn), codec=codec)


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("M,K", [(1, 131072), (8, 32800)])
def test_codec_long_k_multi_pass(w4a16_lib, codec, M, K):
    N = 37
    print(f"[codec shape] {codec} M={M} N={N} K={K}", flush=True)
    x, codes, scale, mn = workload.random_codec_problem(codec, K + M, M, N, K, outliers=True)
    y = run_codec(codec, x, codes, scale, mn)
    y_ref, B = C.gemv(codec, x, codes, scale, mn)
    check(y, y_ref, B, f"{codec} M={M} K={K}", inputs=(x, codes, scale, mn), codec=codec)


def _sample_rows(N, seed, count=256):
    rng = np.random.default_rng(seed)
    rows = set(range(min(N, 8))) | set(range(max(0, N - 8), N))
    rows |= set(rng.choice(N, size=min(N, count), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("M", [1, 4, 8])
def test_codec_llama8b_layer_sampled(w4a16_lib, codec, M):
    name = "llama8b_layer" if M == 1 else "llama8b_verify"
    for pi, p in enumerate(workload.WORKLOADS[name].shapes):
        print(f"[codec 8b] {codec} M={M} {p.name} N={p.N} K={p.K}", flush=True)
        x, codes, scale, mn = workload.codec_gemv_inputs(codec, name, 0, pi, M)
        y = run_codec(codec, x, codes, scale, mn)
        rows = _sample_rows(p.N, pi)
        y_ref, B = C.gemv_rows(codec, x, codes, scale, mn, rows)
        check(y[:, rows], y_ref, B, f"{codec} M={M} {p.name}", inputs=(x, codes, scale, mn), rows=rows, codec=codec)


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("M,N,K", [(5, 24579, 2080), (8, 8195, 2080)])
def test_codec_several_tiles_per_workgroup_sampled(w4a16_lib, codec, M, N, K):
    """Workgroups walk several tiles (alternating load buffers and their tail) at M > 4."""
    print(f"[codec shape] {codec} M={M} N={N} K={K}", flush=True)
    x, codes, scale, mn = workload.random_codec_problem(codec, M * 977 + N, M, N, K, outliers=True)
    y = run_codec(codec, x, codes, scale, mn)
    rows = _sample_rows(N, M)
    y_ref, B = C.gemv_rows(codec, x, codes, scale, mn, rows)
    check(y[:, rows], y_ref, B, f"{codec} M={M} N={N} K={K}", inputs=(x, codes, scale, mn), rows=rows, codec=codec)


@pytest.mark.parametrize("codec", CODECS)
def test_codec_bitwise_repeatable(w4a16_lib, codec):
    x, codes, scale, mn = workload.random_codec_problem(codec, 3, 2, 1000, 4096, outliers=True)
    a = run_codec(codec, x, codes, scale, mn)
    b = run_codec(codec, x, codes, scale, mn)
    np.testing.assert_array_equal(a, b)


def test_q4_sym_kernel_equals_q4_kernel_with_min_minus_eight_scales(w4a16_lib):
    """Same fold, same order: the symmetric kernel with s matches the affine
    kernel with m = -8 s (exact in binary16) bit for bit."""
    x, codes, scale, _ = workload.random_codec_problem("q4_sym", 4, 3, 515, 6176, outliers=True)
    mn = (-8.0 * scale.astype(np.float64)).astype(np.float16)
    ys = run_codec("q4_sym", x, codes, scale, None)
    ya = run_codec("q4", x, codes, scale, mn)
    np.testing.assert_array_equal(ys, ya)


def test_pal4_kernel_with_an_affine_palette_matches_the_q4_kernel(w4a16_lib):
    """An affine palette lut[n][c] = s_n * c + m_n: the palette kernel and the
    4-bit group-affine kernel compute the same product (within tolerance; the
    two sum in different orders)."""
    M, N, K = 2, 300, 4096
    x, codes, _, _ = workload.random_codec_problem("pal4", 13, M, N, K)
    rng = np.random.default_rng(5)
    s = rng.integers(1, 8, size=N).astype(np.float64) / 512.0
    m = -rng.integers(0, 32, size=N).astype(np.float64) / 256.0
    lut = (s[:, None] * np.arange(16)[None, :] + m[:, None]).astype(np.float16)
    G = K // 32
    yp = run_codec("pal4", x, codes, lut, None)
    ya = run_codec("q4", x, codes, np.repeat(s[:, None], G, 1).astype(np.float16),
                   np.repeat(m[:, None], G, 1).astype(np.float16))
    y_ref, B = C.gemv("pal4", x, codes, lut)
    check(yp, y_ref, B, "pal4 affine palette", inputs=(x, codes, lut, None), codec="pal4")
    check(ya, y_ref, B, "q4 with the palette's scale and min",
          inputs=(x, codes, np.repeat(s[:, None], G, 1).astype(np.float16),
                  np.repeat(m[:, None], G, 1).astype(np.float16)))


def test_codec_q4_is_w4a16_gemv(w4a16_lib):
    x, codes, scale, mn = workload.random_problem(11, 2, 300, 4096)
    packed = w4.upload_packed(w4.w4a16_pack(codes, scale, mn), DEV)
    xd = torch.from_numpy(x).to(DEV)
    y0 = torch.empty((2, 300), dtype=torch.float32, device=DEV)
    y1 = torch.empty_like(y0)
    w4.w4a16_gemv(xd, packed, y0)
    w4.w4a16_codec_gemv("q4", xd, packed, y1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("codec", CODECS)
def test_codec_timed_matches_untimed(w4a16_lib, codec):
    M, N, K = 1, 2048, 4096
    x, codes, scale, mn = workload.random_codec_problem(codec, 12, M, N, K)
    packed = w4.upload_packed(w4.w4a16_codec_pack(codec, codes, scale, mn), DEV)
    xd = torch.from_numpy(x).to(DEV)
    s = torch.cuda.Stream(device=DEV)
    y0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.wait_stream(torch.cuda.current_stream())  # the uploads and the NaN fill ran on the current stream
    with torch.cuda.stream(s):
        a.record(s)      # creates the events before their handles are passed on
        b.record(s)
        w4.w4a16_codec_gemv(codec, xd, packed, y0, s)
        st = w4.w4a16_codec_gemv_timed_raw(codec, xd.data_ptr(), packed.data_ptr(), y1.data_ptr(), M, N, K,
                                           s.cuda_stream, a.cuda_event, b.cuda_event)
    assert st == w4.W4A16_OK
    s.synchronize()
    assert torch.equal(y0, y1)
    assert 0.0 < a.elapsed_time(b) < 100.0
