"""GPU parity across launch grids: many tile counts per launch shape.

The GEMV kernels walk 4-row tiles in blocks of one or more tiles per
workgroup, with the workgroup count chosen on the host from the tile count
and the device's occupancy, and pass both to the kernel in one argument. These
cases sweep the tile count (N = 1 .. 65537 at small K, so the oracle stays
fast) at each launch shape of M = 1, 3 and 8, plus two larger K, so that one
tile per workgroup, several tiles per workgroup, more blocks than resident
workgroups and the ragged last block all occur. Every element is compared
with the fp64 oracle (pass rule and sensitivity bound of parity.check).
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

CASES = [(M, N, K) for M in (1, 3, 8) for N, K in
         ((1, 64), (257, 64), (4099, 64), (30001, 64), (65537, 96), (1025, 4128), (6145, 4128), (511, 14336))]


def _run(M, N, K, codec):
    x, codes, scale, mn = (workload.random_problem(M * 977 + N * 13 + K, M, N, K) if codec == "q4" else
                           workload.random_codec_problem(codec, M * 977 + N * 13 + K, M, N, K))
    blob = w4.w4a16_pack(codes, scale, mn) if codec == "q4" else w4.w4a16_codec_pack(codec, codes, scale, mn)
    packed = w4.upload_packed(blob, DEV)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    if codec == "q4":
        w4.w4a16_gemv(xd, packed, y)
    else:
        w4.w4a16_codec_gemv(codec, xd, packed, y)
    torch.cuda.synchronize()
    y_ref, B = oracle.gemv(x, codes, scale, mn) if codec == "q4" else oracle.codecs_ref.gemv(codec, x, codes, scale, mn)
    check(y.cpu().numpy().astype(np.float64), y_ref, B, f"{codec} M={M} N={N} K={K}", inputs=(x, codes, scale, mn),
          codec=codec)


@pytest.mark.parametrize("M,N,K", CASES)
def test_gemv_across_tile_counts(w4a16_lib, M, N, K):
    print(f"[grid] q4 M={M} N={N} K={K} {w4.w4a16_launch_shape(M, N, K)['kernel']}", flush=True)
    _run(M, N, K, "q4")


@pytest.mark.parametrize("codec", ["q5", "pal4"])
@pytest.mark.parametrize("M,N,K", [(1, 65537, 96), (8, 30001, 64), (3, 6145, 4128)])
def test_codec_across_tile_counts(w4a16_lib, codec, M, N, K):
    print(f"[grid] {codec} M={M} N={N} K={K}", flush=True)
    _run(M, N, K, codec)
