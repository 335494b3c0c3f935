"""Seeded synthetic inputs for the W4A16 decode GEMV.

This module is shared by the oracle side (tests, CPU baseline) and the HIP side
(tests, bench, smoke). It holds only random draws and shapes: no dequantisation,
no dot products, no packing. Everything the method computes lives elsewhere.

Recipe (per GEMV, all draws from numpy's PCG64 keyed by
``SeedSequence(ROOT_SEED, spawn_key=(workload, layer, projection, tensor))``):

* codes: uniform random bytes ``uint8[N, K/2]``; a byte is two independent
  uniform 4-bit codes (low nibble = even k, high nibble = odd k).
* scale: uniform on [0.001, 0.01] in float64, rounded to IEEE binary16.
* min:   uniform on [-0.08, 0] in float64, rounded to IEEE binary16.
* x:     standard normal in float64; for the "outlier" workloads exactly
  ``round(0.001 * K)`` distinct positions per activation row (uniform, without
  replacement) are multiplied by 20; then rounded to binary16.

Layer shapes are the public Llama-3-8B and Llama-3-70B decoder projections with
the query/key/value and gate/up matrices fused, the fusion the core-modules
page lists among the packer's operator rewrites (section 5.1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROOT_SEED = 0x57A4A16
GROUP = 32

# tensor ids inside a seed key
_T_CODES, _T_SCALE, _T_MIN, _T_X, _T_OUTLIER = range(5)


@dataclass(frozen=True)
class Proj:
    name: str
    K: int  # input features (reduction length)
    N: int  # output features (rows of the weight matrix)


LLAMA8B_LAYER = (
    Proj("qkv", 4096, 6144),
    Proj("o", 4096, 4096),
    Proj("gate_up", 4096, 28672),
    Proj("down", 14336, 4096),
)

LLAMA70B_LAYER = (
    Proj("qkv", 8192, 10240),
    Proj("o", 8192, 8192),
    Proj("gate_up", 8192, 57344),
    Proj("down", 28672, 8192),
)


# One GPU's share of the 70B layer under 8-way tensor parallelism: the fused
# qkv and gate_up matrices split along their output rows (column-parallel),
# o and down along their input features (row-parallel, each GPU a 1/8 slice
# of K, summed across GPUs afterwards).
LLAMA70B_TP8_SHARD = (
    Proj("qkv", 8192, 1280),
    Proj("o", 1024, 8192),
    Proj("gate_up", 8192, 7168),
    Proj("down", 3584, 8192),
)


@dataclass(frozen=True)
class Workload:
    wid: int             # numeric id used in the seed key
    name: str
    layers: int
    shapes: tuple        # tuple[Proj, ...] per layer
    ms: tuple            # activation-row counts M exercised
    outliers: bool       # 0.1 % x20 activation outliers


WORKLOADS = {
    # single 4096 x 4096 GEMV, M = 1, plain N(0,1) activations
    "gemv4096": Workload(0, "gemv4096", 1, (Proj("square", 4096, 4096),), (1,), False),
    # one Llama-3-8B-shaped decoder layer at M = 1, with activation outliers
    "llama8b_layer": Workload(1, "llama8b_layer", 1, LLAMA8B_LAYER, (1,), True),
    # 32 such layers with independent weights: one decode step, M = 1
    "llama8b_step": Workload(2, "llama8b_step", 32, LLAMA8B_LAYER, (1,), True),
    # speculative-verify batches on the 8B layer shapes, M = 4 and M = 8
    "llama8b_verify": Workload(3, "llama8b_verify", 1, LLAMA8B_LAYER, (4, 8), False),
    # 80 Llama-3-70B-shaped layers, M = 1 and M = 8, with activation outliers
    "llama70b_step": Workload(4, "llama70b_step", 80, LLAMA70B_LAYER, (1, 8), True),
    # one GPU's share of that step under 8-way tensor parallelism, M = 1
    "llama70b_tp8": Workload(5, "llama70b_tp8", 80, LLAMA70B_TP8_SHARD, (1,), True),
}


def _rng(wid: int, layer: int, proj: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=(wid, layer, proj, tensor))
    return np.random.Generator(np.random.PCG64(ss))


def n_outliers(K: int) -> int:
    """Outlier positions per activation row: round(0.001 * K)."""
    return int(round(0.001 * K))


def weights(wid: int, layer: int, proj: int, N: int, K: int):
    """Seeded codes uint8[N, K/2], scale and min float16[N, K/32]."""
    if K % GROUP or K <= 0 or N <= 0:
        raise ValueError(f"bad shape N={N} K={K}")
    codes = _rng(wid, layer, proj, _T_CODES).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scale = _rng(wid, layer, proj, _T_SCALE).uniform(0.001, 0.01, size=(N, K // GROUP)).astype(np.float16)
    mn = _rng(wid, layer, proj, _T_MIN).uniform(-0.08, 0.0, size=(N, K // GROUP)).astype(np.float16)
    return codes, scale, mn


def activations(wid: int, layer: int, proj: int, M: int, K: int, outliers: bool) -> np.ndarray:
    """Seeded x float16[M, K]: N(0,1), optionally with round(0.001 K) x20 outliers per row."""
    x = _rng(wid, layer, proj, _T_X).standard_normal(size=(M, K))
    if outliers:
        r = _rng(wid, layer, proj, _T_OUTLIER)
        cnt = n_outliers(K)
        for m in range(M):
            pos = r.choice(K, size=cnt, replace=False)
            x[m, pos] *= 20.0
    return x.astype(np.float16)


def workload_gemvs(name: str, M: int | None = None):
    """Yield (layer, proj_index, Proj, M) for every GEMV of a named workload."""
    w = WORKLOADS[name]
    ms = w.ms if M is None else (M,)
    for m in ms:
        for layer in range(w.layers):
            for pi, p in enumerate(w.shapes):
                yield layer, pi, p, m


def gemv_inputs(name: str, layer: int, proj: int, M: int):
    """All seeded inputs of one GEMV of a named workload: (x, codes, scale, min)."""
    w = WORKLOADS[name]
    p = w.shapes[proj]
    codes, scale, mn = weights(w.wid, layer, proj, p.N, p.K)
    # x seeds also depend on M so that the M = 4 and M = 8 batches are distinct
    x = activations(w.wid, layer, proj + 16 * M, M, p.K, w.outliers)
    return x, codes, scale, mn


# Weight-code variants (see the codec definitions in the library header): the
# canonical code array per codec is
#   "q4", "q4_sym": uniform random bytes uint8[N, K/2] (two uniform 4-bit codes);
#   "q5":           uniform integers 0..31, uint8[N, K] (one code per byte);
#   "q8_sym":       uniform integers -128..127, int8[N, K];
#   "pal4":         uniform random bytes uint8[N, K/2], and per row a palette
#                   of 16 values U[-0.08, 0.07] sorted, -> binary16 [N, 16]
#                   (passed in the place of the scales).
# Scale and min are the same draws as for the 4-bit code; the symmetric codecs
# take no min (None). Codes of the variants use their own seed keys.
CODECS = ("q4", "q4_sym", "q5", "q8_sym", "pal4")


def codec_weights(codec: str, wid: int, layer: int, proj: int, N: int, K: int):
    """Seeded (codes, scale, min-or-None) of one matrix in a codec's canonical layout."""
    if codec not in CODECS:
        raise ValueError(f"unknown codec {codec!r}")
    codes, scale, mn = weights(wid, layer, proj, N, K)
    ci = CODECS.index(codec)
    r = _rng(wid, layer, proj, _T_CODES + 8 * ci)
    if codec == "q5":
        codes = r.integers(0, 32, size=(N, K), dtype=np.uint8)
    elif codec == "q8_sym":
        codes = r.integers(-128, 128, size=(N, K), dtype=np.int8)
    elif codec in ("q4_sym", "pal4"):
        codes = r.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    if codec == "pal4":
        lut = np.sort(_rng(wid, layer, proj, _T_SCALE + 8 * ci).uniform(-0.08, 0.07, size=(N, 16)), axis=1)
        return codes, lut.astype(np.float16), None
    return codes, scale, (None if codec in ("q4_sym", "q8_sym") else mn)


def codec_gemv_inputs(codec: str, name: str, layer: int, proj: int, M: int):
    """Seeded (x, codes, scale, min-or-None) of one GEMV of a named workload in a codec."""
    w = WORKLOADS[name]
    p = w.shapes[proj]
    codes, scale, mn = codec_weights(codec, w.wid, layer, proj, p.N, p.K)
    x = activations(w.wid, layer, proj + 16 * M, M, p.K, w.outliers)
    return x, codes, scale, mn


def random_codec_problem(codec: str, seed: int, M: int, N: int, K: int, outliers: bool = False):
    """Seeded codec inputs for an arbitrary (M, N, K), used by edge-shape tests."""
    codes, scale, mn = codec_weights(codec, 1000 + seed, 0, 0, N, K)
    x = activations(1000 + seed, 0, 0, M, K, outliers)
    return x, codes, scale, mn


# Decode attention over a quantised KV cache (one layer per call): the
# Llama-3-8B attention shape (32 query heads, 8 KV heads, head size 128,
# 32 layers). The context lengths are the core-modules page's maximum contexts
# for a 2.37 GiB KV budget (section 5.4): 38,863 tokens with INT8 values and
# 77,726 with INT4. Recipe per layer (own seed keys):
#   INT8: codes uniform -128..127, scale U[0.004, 0.012] -> binary16;
#   INT4: codes uniform bytes (two uniform nibbles), scale U[0.08, 0.16] and
#         min U[-1.2, -0.6] -> binary16;
#   q:    N(0, 1) -> binary16, [Hq, 128].
KV_HQ, KV_HKV, KV_D, KV_LAYERS = 32, 8, 128, 32
KV_CONTEXT = {8: 38863, 4: 77726}
_T_KV = 40  # first tensor id of the KV draws


def kv_cache(bits: int, wid: int, layer: int, T: int, Hkv: int = KV_HKV):
    """Seeded (k_codes, k_scale, k_min, v_codes, v_scale, v_min) of one layer's
    cache; the mins are None for INT8."""
    if bits not in (8, 4) or T < 1 or Hkv < 1:
        raise ValueError("bits must be 8 or 4, T and Hkv positive")
    out = []
    for which in range(2):  # keys, then values
        base = _T_KV + 4 * which
        r = _rng(wid, layer, 0, base)
        if bits == 8:
            codes = r.integers(-128, 128, size=(T, Hkv, KV_D), dtype=np.int8)
            scale = _rng(wid, layer, 0, base + 1).uniform(0.004, 0.012, size=(T, Hkv, KV_D // GROUP))
            out += [codes, scale.astype(np.float16), None]
        else:
            codes = r.integers(0, 256, size=(T, Hkv, KV_D // 2), dtype=np.uint8)
            scale = _rng(wid, layer, 0, base + 1).uniform(0.08, 0.16, size=(T, Hkv, KV_D // GROUP))
            mn = _rng(wid, layer, 0, base + 2).uniform(-1.2, -0.6, size=(T, Hkv, KV_D // GROUP))
            out += [codes, scale.astype(np.float16), mn.astype(np.float16)]
    return tuple(out)


KV_BLOCK = 64  # tokens per block of the sentinel recipe (the kernel's unit of work)
KV_SENTINEL_CODE = 3  # the one nonzero value code of the sentinel cache


def kv_sentinel_channel(b: int, Hkv: int) -> tuple:
    """(KV head, dim) that token block b of the sentinel cache marks: block b
    marks channel b mod (Hkv * 128), so a channel is marked by at most
    ceil(blocks / (Hkv * 128)) blocks."""
    ch = b % (Hkv * KV_D)
    return ch // KV_D, ch % KV_D


def kv_sentinel_cache(bits: int, T: int, Hkv: int = KV_HKV):
    """A cache in which every block of 64 tokens is visible on its own: all
    keys are zero (so every token gets the same attention weight), all values
    are zero except that each token of block b holds KV_SENTINEL_CODE in the
    one channel kv_sentinel_channel(b) marks. Scales 0.25, mins 0 (binary16)."""
    if bits not in (8, 4) or T < 1 or Hkv < 1:
        raise ValueError("bits must be 8 or 4, T and Hkv positive")
    G = KV_D // GROUP
    if bits == 8:
        kc = np.zeros((T, Hkv, KV_D), np.int8)
        vc = np.zeros((T, Hkv, KV_D), np.int8)
    else:
        kc = np.zeros((T, Hkv, KV_D // 2), np.uint8)
        vc = np.zeros((T, Hkv, KV_D // 2), np.uint8)
    for b in range(-(-T // KV_BLOCK)):
        g, d = kv_sentinel_channel(b, Hkv)
        t0, t1 = b * KV_BLOCK, min(T, (b + 1) * KV_BLOCK)
        if bits == 8:
            vc[t0:t1, g, d] = KV_SENTINEL_CODE
        else:
            vc[t0:t1, g, d // 2] = KV_SENTINEL_CODE << (4 * (d % 2))
    scale = np.full((T, Hkv, G), 0.25, np.float16)
    mn = None if bits == 8 else np.zeros((T, Hkv, G), np.float16)
    return kc, scale, mn, vc, scale.copy(), None if mn is None else mn.copy()


def kv_query(wid: int, layer: int, Hq: int = KV_HQ) -> np.ndarray:
    """Seeded query q binary16 [Hq, 128]."""
    return _rng(wid, layer, 0, _T_KV + 9).standard_normal(size=(Hq, KV_D)).astype(np.float16)


def random_problem(seed: int, M: int, N: int, K: int, outliers: bool = False):
    """Seeded inputs for an arbitrary (M, N, K), used by edge-shape tests."""
    codes, scale, mn = weights(1000 + seed, 0, 0, N, K)
    x = activations(1000 + seed, 0, 0, M, K, outliers)
    return x, codes, scale, mn
