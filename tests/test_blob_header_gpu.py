"""GPU tests of the blob-header check: a launch whose packed blob's header
does not match the call (another shape of the same size, another codec, a
changed layout version) writes nothing to y and is counted, and a chain
naming such a blob writes nothing and raises its blob bit. Every mismatched
blob is chosen so that all of the kernel's reads stay inside the blob's
allocation: the same total size, or a layout the call reads less of."""
import numpy as np
import pytest

import bit_weight_quantized_w4a16_amd as w4
import oracle
import workload
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FILL = -7.0


def _x(M, K, seed):
    x = workload.random_problem(seed, M, 4, K)[0]
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_transposed_blob_writes_nothing(w4a16_lib, M):
    """A blob of the 8B down projection (N = 4096, K = 14336) handed to a call
    for gate's shape (N = 14336, K = 4096): both blobs have the same size."""
    N, K = 4096, 14336
    assert w4.w4a16_packed_bytes(N, K) == w4.w4a16_packed_bytes(K, N)
    _, codes, scale, mn = workload.random_problem(41 + M, 1, N, K)
    packed = w4.upload_packed(w4.w4a16_pack(codes, scale, mn), DEV)
    w4.w4a16_blob_mismatches()                              # reset the device's count
    x = _x(M, N, 5 + M)                                      # the call's K is 4096
    y = torch.full((M, K), FILL, dtype=torch.float32, device=DEV)
    print(f"[blob] transposed M={M}: call (N={K}, K={N}) on a blob of (N={N}, K={K})", flush=True)
    w4.w4a16_gemv(x, packed, y)
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == FILL).all()
    assert w4.w4a16_blob_mismatches() == 1
    assert w4.w4a16_blob_mismatches() == 0                   # the query reset it


def test_matching_blob_is_not_counted(w4a16_lib):
    x, codes, scale, mn = workload.random_problem(3, 2, 130, 4096)
    packed = w4.upload_packed(w4.w4a16_pack(codes, scale, mn), DEV)
    w4.w4a16_blob_mismatches()
    y = torch.full((2, 130), FILL, dtype=torch.float32, device=DEV)
    w4.w4a16_gemv(torch.from_numpy(x).to(DEV), packed, y)
    torch.cuda.synchronize()
    y_ref, B = oracle.gemv(x, codes, scale, mn)
    check(y.cpu().numpy().astype(np.float64), y_ref, B, "matching header", inputs=(x, codes, scale, mn))
    assert w4.w4a16_blob_mismatches() == 0


def test_changed_version_writes_nothing(w4a16_lib):
    """A blob whose layout-version field differs (an older or newer packer)."""
    x, codes, scale, mn = workload.random_problem(7, 1, 300, 2048)
    blob = w4.w4a16_pack(codes, scale, mn)
    blob[4] ^= 0x03                                          # version 6 -> 5
    packed = w4.upload_packed(blob, DEV)
    w4.w4a16_blob_mismatches()
    y = torch.full((1, 300), FILL, dtype=torch.float32, device=DEV)
    w4.w4a16_gemv(torch.from_numpy(x).to(DEV), packed, y)
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == FILL).all()
    assert w4.w4a16_blob_mismatches() == 1


@pytest.mark.parametrize("codec", ["q4_sym", "pal4"])
def test_codec_blob_of_another_codec_writes_nothing(w4a16_lib, codec):
    """A 4-bit group-affine blob handed to a codec call: the q4_sym and pal4
    layouts of the same (N, K) are no larger, so every read stays inside it."""
    N, K = 1000, 4096
    assert w4.w4a16_codec_packed_bytes(codec, N, K) <= w4.w4a16_packed_bytes(N, K)
    x, codes, scale, mn = workload.random_problem(11, 2, N, K)
    packed = w4.upload_packed(w4.w4a16_pack(codes, scale, mn), DEV)
    w4.w4a16_blob_mismatches()
    y = torch.full((2, N), FILL, dtype=torch.float32, device=DEV)
    w4.w4a16_codec_gemv(codec, torch.from_numpy(x).to(DEV), packed, y)
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == FILL).all()
    assert w4.w4a16_blob_mismatches() == 1


@pytest.mark.parametrize("bad_at", [0, 1, 2])
def test_chain_with_a_mismatched_blob_writes_nothing(w4a16_lib, bad_at):
    """One entry's blob is packed for (8, 64) but the entry says (16, 32) (the
    same size): the launch writes no y at all, raises the blob bit and
    resets every counter; the plan without that entry then runs as usual."""
    M = 1
    p0 = workload.random_problem(21, M, 517, 4096)
    p2 = workload.random_problem(23, M, 64, 8192)
    _, c1, s1, m1 = workload.random_problem(22, M, 8, 64)
    assert w4.w4a16_packed_bytes(8, 64) == w4.w4a16_packed_bytes(16, 32)
    items = []
    for x, codes, scale, mn in (p0, p2):
        items.append(dict(x=torch.from_numpy(x).to(DEV), packed=w4.upload_packed(w4.w4a16_pack(codes, scale, mn), DEV),
                          y=torch.full((M, codes.shape[0]), FILL, dtype=torch.float32, device=DEV),
                          N=codes.shape[0], K=codes.shape[1] * 2))
    bad = dict(x=_x(M, 32, 9), packed=w4.upload_packed(w4.w4a16_pack(c1, s1, m1), DEV),
               y=torch.full((M, 16), FILL, dtype=torch.float32, device=DEV), N=16, K=32)
    order = [items[0], items[1]]
    order.insert(bad_at, bad)

    def run(entries):
        plan = torch.from_numpy(w4.w4a16_chain_plan([(it["x"], it["packed"], it["y"], it["N"], it["K"])
                                                     for it in entries], M)).to(DEV)
        ws = torch.zeros(w4.W4A16_CHAIN_WORKSPACE_BYTES // 4, dtype=torch.int32, device=DEV)
        w4.w4a16_gemv_chain(plan, len(entries), M, ws)
        torch.cuda.synchronize()
        return ws.cpu().numpy(), w4.w4a16_chain_status_raw(ws.data_ptr(), ws.numel() * 4, 0, False)

    print(f"[blob] chain of 3, entry {bad_at} mismatched", flush=True)
    w, status = run(order)
    for it in order:
        assert (it["y"].cpu().numpy() == FILL).all()
    assert w[w4.W4A16_CHAIN_ERROR_OFFSET // 4] == w4.W4A16_CHAIN_ERR_BLOB
    assert status == (w4.W4A16_ERR_FORMAT, w4.W4A16_CHAIN_ERR_BLOB)
    w[w4.W4A16_CHAIN_ERROR_OFFSET // 4] = 0
    assert not w.any()
    w, status = run(items)
    assert not w.any() and status == (w4.W4A16_OK, 0)
    for it, (x, codes, scale, mn) in zip(items, (p0, p2)):
        y_ref, B = oracle.gemv(x, codes, scale, mn)
        check(it["y"].cpu().numpy().astype(np.float64), y_ref, B, f"chain entry N={it['N']}",
              inputs=(x, codes, scale, mn))
