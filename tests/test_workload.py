"""The seeded input recipe: determinism, ranges and the outlier count."""
import numpy as np
import pytest

import workload


def test_deterministic_and_keyed():
    a = workload.weights(1, 0, 0, 8, 64)
    b = workload.weights(1, 0, 0, 8, 64)
    c = workload.weights(1, 1, 0, 8, 64)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert not np.array_equal(a[0], c[0])
    x1 = workload.activations(1, 0, 0, 2, 4096, True)
    x2 = workload.activations(1, 0, 0, 2, 4096, True)
    assert np.array_equal(x1, x2)


def test_ranges_and_dtypes():
    codes, scale, mn = workload.weights(0, 0, 0, 64, 4096)
    assert codes.dtype == np.uint8 and codes.shape == (64, 2048)
    assert scale.dtype == np.float16 and scale.shape == (64, 128)
    assert mn.dtype == np.float16 and mn.shape == (64, 128)
    s = scale.astype(np.float64)
    m = mn.astype(np.float64)
    assert s.min() >= np.float16(0.001) and s.max() <= np.float16(0.01)
    assert m.min() >= np.float16(-0.08) and m.max() <= 0.0
    lo, hi = codes & 0xF, codes >> 4
    # both nibbles cover 0..15 and look uniform
    for nib in (lo, hi):
        counts = np.bincount(nib.reshape(-1), minlength=16)
        assert counts.min() > 0.9 * nib.size / 16 and counts.max() < 1.1 * nib.size / 16


@pytest.mark.parametrize("K", [4096, 8192, 14336, 28672])
def test_outlier_count_per_row(K):
    assert workload.n_outliers(K) == {4096: 4, 8192: 8, 14336: 14, 28672: 29}[K]
    plain = workload._rng(5, 0, 0, workload._T_X).standard_normal(size=(3, K))
    x = workload.activations(5, 0, 0, 3, K, True)
    for m in range(3):
        changed = x[m] != plain[m].astype(np.float16)
        assert changed.sum() == workload.n_outliers(K)
        np.testing.assert_array_equal(x[m][changed], (20.0 * plain[m][changed]).astype(np.float16))
    no = workload.activations(5, 0, 0, 3, K, False)
    assert np.array_equal(no, plain.astype(np.float16))


def test_named_workloads():
    names = list(workload.WORKLOADS)
    assert names == ["gemv4096", "llama8b_layer", "llama8b_step", "llama8b_verify", "llama70b_step", "llama70b_tp8"]
    step = list(workload.workload_gemvs("llama8b_step"))
    assert len(step) == 128
    nweights = sum(p.N * p.K for _, _, p, _ in step)
    assert nweights == 6_979_321_856
    big = list(workload.workload_gemvs("llama70b_step", M=1))
    assert len(big) == 320
    assert sum(p.N * p.K for _, _, p, _ in big) == 68_451_041_280
    # 8-way tensor parallelism: every matrix of the 70B layer is split eight ways,
    # qkv and gate_up along N, o and down along K
    shard = list(workload.workload_gemvs("llama70b_tp8", M=1))
    assert len(shard) == 320
    assert sum(p.N * p.K for _, _, p, _ in shard) * 8 == 68_451_041_280
    for full, part in zip(workload.LLAMA70B_LAYER, workload.LLAMA70B_TP8_SHARD):
        assert full.name == part.name
        assert (part.N * 8, part.K) == (full.N, full.K) or (part.N, part.K * 8) == (full.N, full.K)


def test_gemv_inputs_shapes():
    x, codes, scale, mn = workload.gemv_inputs("llama8b_verify", 0, 3, 8)
    assert x.shape == (8, 14336) and codes.shape == (4096, 7168)
    assert scale.shape == (4096, 448) and mn.shape == (4096, 448)
