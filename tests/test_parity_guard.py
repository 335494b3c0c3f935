"""The sensitivity bound of the GPU parity checks (tests/parity.py), on the CPU.

* It catches what the pass rule misses: dropping one group of 32 weights from
  one output of the 8B down projection (K = 14336) breaks the bound for nearly
  every output, while the pass rule lets most of them through.
* It is not tighter than fp32 arithmetic allows: fp32 sums over the kernels'
  split of each weight into a code part and an offset part, in sequential and
  in shuffled order, stay inside it.
"""
import numpy as np

import oracle
import parity
import workload


def test_dropped_group_fails_the_bound_but_not_the_pass_rule():
    x, codes, scale, mn = workload.gemv_inputs("llama8b_layer", 0, 3, 1)   # down projection, K = 14336
    rows = np.arange(0, codes.shape[0], 32)                                  # 128 outputs
    y_ref, B = oracle.gemv_rows(x, codes, scale, mn, rows)
    bound = parity.sensitivity_bound("q4", x, codes, scale, mn, rows)[0]
    w = oracle.w4a16_ref.dequantise(codes[rows], scale[rows], mn[rows])
    contrib = (w * x[0].astype(np.float64)).reshape(len(rows), -1, 32).sum(axis=2)   # [rows, groups]
    groups = np.arange(0, contrib.shape[1], 7)
    caught_bound = np.abs(contrib[:, groups]) > bound[:, None]
    caught_rule = np.abs(contrib[:, groups]) > oracle.tolerance(B[0])[:, None]
    print(f"dropped group: outside the bound {caught_bound.mean():.3f}, outside the pass rule {caught_rule.mean():.3f}")
    assert caught_bound.mean() >= 0.95
    assert caught_rule.mean() <= 0.5


def _fp32_sum(terms, order):
    acc = np.float32(0)
    for t in terms[order]:
        acc = np.float32(acc + np.float32(t))
    return float(acc)


def test_fp32_sums_stay_inside_the_bound():
    rng = np.random.default_rng(3)
    for K in (32, 256, 4096):
        x, codes, scale, mn = workload.random_problem(K, 1, 6, K, outliers=True)
        y_ref, _ = oracle.gemv(x, codes, scale, mn)
        bound = parity.sensitivity_bound("q4", x, codes, scale, mn)[0]
        q = parity._nibbles(codes)
        s = np.repeat(scale.astype(np.float64), 32, axis=1)
        m = np.repeat(mn.astype(np.float64), 32, axis=1)
        xf = x[0].astype(np.float64)
        for n in range(codes.shape[0]):
            terms = np.concatenate([s[n] * q[n] * xf, m[n] * xf])    # code parts, offset parts
            for order in (np.arange(2 * K), rng.permutation(2 * K)):
                assert abs(_fp32_sum(terms, order) - y_ref[0, n]) <= bound[n]


def test_weight_parts_of_each_codec():
    codes = np.array([[0x10, 0xF7]], np.uint8)          # k = 0..3: q = 0, 1, 7, 15
    s = np.full((1, 1), 0.5, np.float16)
    m = np.full((1, 1), -0.25, np.float16)
    pad = lambda a: np.pad(a, ((0, 0), (0, 14)))        # noqa: E731  (K = 32)
    p = parity.weight_parts("q4", pad(codes), s, m)
    np.testing.assert_array_equal(p[0, :4], [0.25, 0.75, 3.75, 7.75])
    p = parity.weight_parts("q4_sym", pad(codes), s)
    np.testing.assert_array_equal(p[0, :4], [4.0, 4.5, 7.5, 11.5])
    q8 = np.zeros((1, 32), np.int8)
    q8[0, :3] = [-128, 0, 127]
    p = parity.weight_parts("q8_sym", q8.view(np.uint8), s)
    np.testing.assert_array_equal(p[0, :3], [64.0, 128.0, 191.5])
    lut = np.arange(16, dtype=np.float16)[None, :] - 8
    p = parity.weight_parts("pal4", pad(codes), lut)
    np.testing.assert_array_equal(p[0, :4], [8.0, 7.0, 1.0, 7.0])
