"""GPU tests of the decode-step chain (w4a16_gemv_chain) through the C ABI.

* parity with the fp64 oracle on mixed shapes, every M, and on one full
  8B-shaped layer (sampled rows);
* a real dependency: product 1 reads product 0's fp32 output as its binary16
  input, so running it before product 0 finished would read stale memory;
* agreement with separate w4a16_gemv launches (bitwise where the launch
  shapes coincide);
* the workspace is left zeroed and error-free after every call;
* a plan whose header does not match the call writes nothing and raises the
  plan bit of the error word, which w4a16_chain_status reports (and clears);
* w4a16_chain_status maps each error bit to its status;
* the chain captured in a HIP graph and replayed, with eager work and
  synchronisation between replays, matches the eager result every time.
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


class Chain:
    """Device buffers and plan for a list of (x, codes, scale, min) problems."""

    def __init__(self, problems, M, y_fill=float("nan")):
        self.M = M
        self.items = []
        for x, codes, scale, mn in problems:
            packed = w4.upload_packed(w4.w4a16_pack(codes, scale, mn), DEV)
            xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if x is not None else None
            y = torch.full((M, codes.shape[0]), y_fill, dtype=torch.float32, device=DEV)
            self.items.append(dict(x=xd, packed=packed, y=y, N=codes.shape[0], K=codes.shape[1] * 2))
        self.workspace = torch.zeros(w4.W4A16_CHAIN_WORKSPACE_BYTES // 4, dtype=torch.int32, device=DEV)

    def plan(self, M=None):
        entries = [(it["x"], it["packed"], it["y"], it["N"], it["K"]) for it in self.items]
        host = w4.w4a16_chain_plan(entries, self.M if M is None else M)
        self.plan_dev = torch.from_numpy(host).to(DEV)
        return self.plan_dev

    def run(self, stream=None, M=None, check=False):
        w4.w4a16_gemv_chain(self.plan_dev, len(self.items), self.M if M is None else M, self.workspace, stream,
                            check=check)


def assert_workspace_clean(ch):
    ws = ch.workspace.cpu().numpy()
    assert ws[w4.W4A16_CHAIN_ERROR_OFFSET // 4] == 0, "the error word is raised"
    assert not ws.any(), f"counters or flags not reset: {np.flatnonzero(ws)[:8]}"


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_chain_mixed_shapes_vs_oracle(w4a16_lib, M):
    shapes = [(4097, 4096), (3, 64), (130, 14336), (64, 8192), (21, 28672), (517, 96)]
    problems = [workload.random_problem(300 + i * 7 + M, M, N, K, outliers=True) for i, (N, K) in enumerate(shapes)]
    print(f"[chain] M={M} shapes={shapes}", flush=True)
    ch = Chain(problems, M)
    ch.plan()
    ch.run()
    torch.cuda.synchronize()
    for it, (x, codes, scale, mn) in zip(ch.items, problems):
        y_ref, B = oracle.gemv(x, codes, scale, mn)
        check(it["y"].cpu().numpy().astype(np.float64), y_ref, B, f"M={M} N={it['N']} K={it['K']}",
              inputs=(x, codes, scale, mn))
    assert_workspace_clean(ch)


def test_chain_llama8b_layer_sampled(w4a16_lib):
    """One 8B-shaped layer (qkv, o, gate_up, down at their full sizes, M = 1)
    through the chain kernel the bench times, compared on sampled rows."""
    problems = [workload.gemv_inputs("llama8b_layer", 0, proj, 1) for proj in range(4)]
    print(f"[chain] llama8b_layer M=1 {w4.chain_launch_shape(1)}", flush=True)
    ch = Chain(problems, 1)
    ch.plan()
    ch.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    for it, (x, codes, scale, mn) in zip(ch.items, problems):
        N = it["N"]
        rows = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N), rng.choice(N, 256, replace=False)]))
        y_ref, B = oracle.gemv_rows(x, codes, scale, mn, rows)
        check(it["y"].cpu().numpy().astype(np.float64)[:, rows], y_ref, B, f"llama8b_layer N={N} K={it['K']}",
              inputs=(x, codes, scale, mn), rows=rows)
    assert_workspace_clean(ch)


def _dependent_problems(seed):
    """Product 0 gives small non-negative integers y0 (< 256, so their fp32 low
    halves are zero); product 1 reads y0's bytes as 2*N0 binary16 values."""
    rng = np.random.default_rng(seed)
    N0, K0 = 96, 64
    x0 = np.ones((1, K0), np.float16)
    q0 = rng.integers(0, 8, size=(N0, K0))                  # sum of 64 codes < 8*64 = 512
    q0[:, 32:] = 0                                          # keep y0 <= 7*32 = 224 < 256
    codes0 = (q0[:, 0::2] | (q0[:, 1::2] << 4)).astype(np.uint8)
    scale0 = np.ones((N0, K0 // 32), np.float16)
    min0 = np.zeros((N0, K0 // 32), np.float16)
    y0 = q0.sum(axis=1).astype(np.float32)[None, :]         # exact
    x1 = y0.view(np.float16)                                # [1, 2*N0] = [1, 192]
    K1 = x1.shape[1]
    _, codes1, scale1, min1 = workload.random_problem(seed + 1, 1, 77, K1)
    return (x0, codes0, scale0, min0), (x1, codes1, scale1, min1), y0


def test_chain_honours_read_after_write(w4a16_lib):
    p0, p1, y0_exact = _dependent_problems(5)
    # product 1's x is product 0's y: build the chain by hand so that entry 1
    # points its x at entry 0's output buffer; that buffer starts as garbage
    ch = Chain([p0, (None, p1[1], p1[2], p1[3])], 1, y_fill=3.0)
    ch.items[1]["x"] = ch.items[0]["y"]
    ch.plan()
    for rep in range(3):
        ch.items[0]["y"].fill_(3.0)           # stale contents: 3.0f reads as binary16 (0, 2.125)
        ch.items[1]["y"].fill_(float("nan"))
        ch.run()
        torch.cuda.synchronize()
        y0 = ch.items[0]["y"].cpu().numpy()
        assert np.array_equal(y0, y0_exact)
        y_ref, B = oracle.gemv(p1[0], p1[1], p1[2], p1[3])
        check(ch.items[1]["y"].cpu().numpy().astype(np.float64), y_ref, B, f"dependent product, rep {rep}",
              inputs=(p1[0], p1[1], p1[2], p1[3]))
        assert_workspace_clean(ch)


@pytest.mark.parametrize("M", [1, 2])
def test_chain_matches_separate_launches(w4a16_lib, M):
    shapes = [(6144, 4096), (4096, 4096), (2048, 14336), (1000, 4096)]
    problems = [workload.random_problem(400 + i, M, N, K, outliers=True) for i, (N, K) in enumerate(shapes)]
    ch = Chain(problems, M)
    ch.plan()
    ch.run()
    torch.cuda.synchronize()
    for it, (x, codes, scale, mn) in zip(ch.items, problems):
        y = torch.empty_like(it["y"])
        w4.w4a16_gemv(it["x"], it["packed"], y)
        torch.cuda.synchronize()
        a, b = it["y"].cpu().numpy(), y.cpu().numpy()
        if M == 2:
            # both split K into 64-group segments and add the segments' wave
            # sums in order: the same bits
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"N={it['N']} K={it['K']}"
        else:
            # different segment widths: only the fp32 summation order differs
            _, B = oracle.gemv(x, codes, scale, mn)
            assert (np.abs(a.astype(np.float64) - b) <= 1e-5 * B + 1e-6).all(), f"N={it['N']} K={it['K']}"


def test_chain_header_mismatch_writes_nothing(w4a16_lib):
    problems = [workload.random_problem(500, 1, 40, 128)]
    ch = Chain(problems, 1, y_fill=-7.0)
    ch.plan(M=1)
    ch.run(M=2)                                             # plan says M = 1
    torch.cuda.synchronize()
    assert (ch.items[0]["y"].cpu().numpy() == -7.0).all()
    ws = ch.workspace.cpu().numpy()
    assert ws[w4.W4A16_CHAIN_ERROR_OFFSET // 4] == w4.W4A16_CHAIN_ERR_PLAN
    ws[w4.W4A16_CHAIN_ERROR_OFFSET // 4] = 0
    assert not ws.any()                                     # no counter was touched
    ws_bytes = ch.workspace.numel() * 4
    st, bits = w4.w4a16_chain_status_raw(ch.workspace.data_ptr(), ws_bytes, 0, False)
    assert (st, bits) == (w4.W4A16_ERR_FORMAT, w4.W4A16_CHAIN_ERR_PLAN)
    assert w4.w4a16_chain_status(ch.workspace) == w4.W4A16_CHAIN_ERR_PLAN   # sticky until cleared
    assert w4.w4a16_chain_status(ch.workspace, clear=True) == w4.W4A16_CHAIN_ERR_PLAN
    assert not ch.workspace.cpu().numpy().any()
    with pytest.raises(w4.W4A16Error) as e:
        ch.run(M=2, check=True)
    assert e.value.status == w4.W4A16_ERR_FORMAT
    assert not ch.workspace.cpu().numpy().any()             # check=True cleared it
    ch.run(M=1, check=True)                                 # the matching call still works
    assert np.isfinite(ch.items[0]["y"].cpu().numpy()).all() and (ch.items[0]["y"].cpu().numpy() != -7.0).any()
    assert_workspace_clean(ch)
    assert w4.w4a16_chain_status_raw(ch.workspace.data_ptr(), ws_bytes, 0, True) == (w4.W4A16_OK, 0)


def test_chain_status_maps_each_bit(w4a16_lib):
    """The error word is the only input of w4a16_chain_status: set from the
    host, each combination of bits maps to its status (the wait bit wins), and
    clearing zero-fills the whole workspace. No chain kernel is launched."""
    ws = torch.zeros(w4.W4A16_CHAIN_WORKSPACE_BYTES // 4 + 8, dtype=torch.int32, device=DEV)
    at = w4.W4A16_CHAIN_ERROR_OFFSET // 4
    cases = [(0, w4.W4A16_OK), (w4.W4A16_CHAIN_ERR_WAIT, w4.W4A16_ERR_WAIT),
             (w4.W4A16_CHAIN_ERR_PLAN, w4.W4A16_ERR_FORMAT), (w4.W4A16_CHAIN_ERR_BLOB, w4.W4A16_ERR_FORMAT),
             (w4.W4A16_CHAIN_ERR_WAIT | w4.W4A16_CHAIN_ERR_BLOB, w4.W4A16_ERR_WAIT)]
    s = torch.cuda.Stream()
    for word, status in cases:
        ws.fill_(0)
        ws[at] = word
        ws[1] = 5                                           # a stale counter beside the word
        ws[-1] = 9                                          # past the workspace: never touched
        torch.cuda.synchronize()
        st, bits = w4.w4a16_chain_status_raw(ws.data_ptr(), ws.numel() * 4, s.cuda_stream, True)
        assert (st, bits) == (status, word), word
        h = ws.cpu().numpy()
        assert h[-1] == 9
        if word:
            assert not h[:-8].any(), word                   # cleared: counters too
        else:
            assert h[1] == 5                                # nothing set: nothing cleared


def test_chain_graph_replays_match_eager(w4a16_lib):
    shapes = [(1024, 4096), (512, 14336), (300, 4096)]
    problems = [workload.random_problem(600 + i, 1, N, K, outliers=True) for i, (N, K) in enumerate(shapes)]
    ch = Chain(problems, 1)
    ch.plan()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())  # the plan and workspace uploads ran on the current stream
    with torch.cuda.stream(s):
        ch.run(s)
    s.synchronize()
    eager = [it["y"].clone() for it in ch.items]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ch.run(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for it in ch.items:
            it["y"].fill_(float("nan"))                     # eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        for it, e in zip(ch.items, eager):
            assert torch.equal(it["y"], e), f"replay {rep} differs"
        assert_workspace_clean(ch)
