// gfx950 kernels and C-ABI entry points of decode attention over a quantised
// KV cache (INT8 symmetric or INT4 affine values; formats in include/w4a16.h).
//
// The core-modules page (section 5.4, memory manager: KV budget) sizes the KV
// cache of an 8B grouped-query model at 131,072 bytes per token in fp16,
// halved with INT8 and quartered with INT4 values. At a decode step the whole
// cache of every layer is read once per generated token, so, like the weight
// GEMVs, the operation is a streaming kernel: every cache byte is loaded once
// with 128-bit non-temporal loads, and the arithmetic per byte is small.
//
// Work decomposition (split-T "flash decoding"):
// * The cache of a KV head is a run of 64-token blocks. A workgroup of four
//   waves takes a contiguous range of a head's blocks; its waves take the
//   blocks round-robin. All GQ query heads that share the KV head are served
//   by the same pass over the block, so the cache is read once for all of them.
// * Phase 1 of a block, one lane per token: the key codes of its token (eight
//   or four 16-byte chunks laid out so that each load instruction reads 1 KiB
//   contiguously) are turned into binary16 subnormal pairs by masking and
//   dotted with the query pairs, which come from scalar loads (the query is
//   uniform across the wave); the group scale folds them into the score. An
//   online softmax across the wave keeps the running maximum per query head,
//   and each lane writes its token's weights p * s_v (and p * m_v) to LDS.
// * Phase 2 of a block, one lane per two head dimensions: the value codes
//   (16 bytes per lane per load, eight or sixteen tokens of its two dims) are
//   converted to fp32 and accumulated with the token weights read back from
//   LDS.
// * The four waves' partial results are merged through LDS in a fixed order
//   and each workgroup writes one partial (maximum, sum of weights, 128
//   weighted values per query head) to the caller's workspace; a second
//   kernel merges the partials of each query head, again in a fixed order.
//   Results are bitwise repeatable; no atomics are used.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "w4a16.h"
#include "w4a16_device.h"
#include "w4a16_host.h"

using namespace w4a16_dev;

namespace {

constexpr int kD = 128;          // head size
constexpr int kBlockTokens = 64;  // tokens per block (one per lane in phase 1)
constexpr int kWaves = 4;         // waves per workgroup
constexpr int kPartFloats = kD + 2;  // one partial: 128 weighted values, maximum, weight sum

// Bytes of one (KV head, block) record, and offsets inside it.
template <int BITS>
struct Rec;
template <>
struct Rec<8> {
  static constexpr int kKCodes = 0;        // 8 chunks x 64 tokens x 16 B
  static constexpr int kKPar = 8192;       // 64 tokens x 4 scales (binary16)
  static constexpr int kVPar = 8704;       // 64 tokens x 4 scales
  static constexpr int kVCodes = 9216;     // 8 loads x 64 lanes x 16 B
  static constexpr int kBytes = 17408;
  static constexpr int kKChunks = 8;
  static constexpr int kVLoads = 8;        // 8 tokens per load
};
template <>
struct Rec<4> {
  static constexpr int kKCodes = 0;        // 4 chunks x 64 tokens x 16 B
  static constexpr int kKPar = 4096;       // 64 tokens x 4 (scale, min)
  static constexpr int kVPar = 5120;       // 64 tokens x 4 (scale, min)
  static constexpr int kVCodes = 6144;     // 4 loads x 64 lanes x 16 B
  static constexpr int kBytes = 10240;
  static constexpr int kKChunks = 4;
  static constexpr int kVLoads = 4;        // 16 tokens per load
};

typedef const __attribute__((address_space(4))) uint32_t* QPtr;  // read through scalar loads
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float half_lo(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xFFFFu))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16))); }
__device__ __forceinline__ float byte_f(uint32_t w, int i) { return float((w >> (8 * i)) & 0xFFu); }

// Score of this lane's token against query head h (in units of the raw dot
// product, before 1/sqrt(D)): the key chunks kc, the token's group
// parameters kp (INT8: 4 scales in 2 words; INT4: (scale, min) x 4 in 4
// words) and the query's per-group sums qsum.
template <int BITS>
__device__ __forceinline__ float key_score(const u32x4 (&kc)[Rec<BITS>::kKChunks], const u32x4& kp, QPtr qh,
                                           const float (&qsum)[4]) {
  float score = 0.f;
  if constexpr (BITS == 8) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      float dot = 0.f;
#pragma unroll
      for (int c = 2 * grp; c < 2 * grp + 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = elem(kc[c], e);
          dot = dot2(w & 0x00FF00FFu, qh[8 * c + 2 * e], dot);
          dot = dot2((w >> 8) & 0x00FF00FFu, qh[8 * c + 2 * e + 1], dot);
        }
      const float s = (grp & 1) ? half_hi(elem(kp, grp >> 1)) : half_lo(elem(kp, grp >> 1));
      score = __builtin_fmaf(s * 0x1p24f, dot, score);
      score = __builtin_fmaf(-128.f * s, qsum[grp], score);
    }
  } else {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      float lo = 0.f, hi = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t w = elem(kc[grp], wd), w8 = w >> 8;
        const int qd = 16 * grp + 4 * wd;
        lo = dot2(w & 0x000F000Fu, qh[qd], lo);
        hi = dot2(w & 0x00F000F0u, qh[qd + 1], hi);
        lo = dot2(w8 & 0x000F000Fu, qh[qd + 2], lo);
        hi = dot2(w8 & 0x00F000F0u, qh[qd + 3], hi);
      }
      const uint32_t par = elem(kp, grp);
      score = __builtin_fmaf(half_lo(par) * 0x1p20f, __builtin_fmaf(lo, 16.f, hi), score);
      score = __builtin_fmaf(half_hi(par), qsum[grp], score);
    }
  }
  return score;
}

template <int BITS, int GQ>
__global__ void __launch_bounds__(64 * kWaves)
kv_attn_kernel(const uint32_t* __restrict__ q_pairs, const uint8_t* __restrict__ kv, float* __restrict__ part, int T,
               int nb, int bpw, float scale_log2) {
  using R = Rec<BITS>;
  // the query (binary16 pairs [Hq][64]) is read through the constant address
  // space: uniform, so the compiler loads it with scalar loads
  const QPtr q = (QPtr)(reinterpret_cast<uintptr_t>(q_pairs));
  constexpr int kKPar = BITS == 8 ? 8 : 16;  // parameter bytes per token
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.y;           // KV head
  const int split = blockIdx.x;
  const int S = gridDim.x;
  const int b0 = split * bpw;
  const int b1 = min(b0 + bpw, nb);

  // binary16 token weights p * s_v * 2^E per (wave, head, value group, slot)
  __shared__ __attribute__((aligned(16))) _Float16 wh[kWaves][GQ][4][kBlockTokens];
  __shared__ float comb[kWaves][GQ][kPartFloats];

  // Per-group sums of each query head (the offset / min terms of the
  // score). The GQ heads' rows are GQ * 16 chunks of 16 bytes; lane i of load
  // c takes chunk 64c + i (head i / 16, group (i / 4) % 4), issued before the
  // first block's loads and summed after them, so the two latencies overlap
  // (scalar loads of the 16 groups one after another would put 16 cache
  // round trips in front of the first block).
  constexpr int kQLoads = (GQ * 16 + 63) / 64;
  u32x4 qv[kQLoads];
#pragma unroll
  for (int c = 0; c < kQLoads; ++c) {
    const int i = 64 * c + lane;
    qv[c] = reinterpret_cast<const u32x4*>(q_pairs + size_t(g) * GQ * (kD / 2))[i < GQ * 16 ? i : 0];
  }
  float qsum[GQ][4];
#pragma unroll
  for (int j = 0; j < GQ; ++j)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) qsum[j][grp] = 0.f;

  // Running state per query head j: the maximum m (uniform, exp2 domain) and,
  // in real units, l (the weight sum of this lane's tokens), acc (the weighted
  // values of this lane's two dims) and off[grp] (the offset / min term of
  // this lane's tokens for value group grp).
  float m[GQ], l[GQ], acc[GQ][2], off[GQ][4];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    m[j] = -__builtin_inff();
    l[j] = 0.f;
    acc[j][0] = acc[j][1] = 0.f;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) off[j][grp] = 0.f;
  }
  const int vgrp = lane >> 4;  // group of this lane's two dims in phase 2
  // slot of this lane's token in a row of binary16 weights: INT8 keeps token
  // order (dword k = tokens 2k, 2k+1, the pair a value word forms); INT4
  // stores each 4-token group as (t0, t2, t1, t3), the pairs its value bytes
  // form under the nibble masks
  const int wpos = BITS == 8 ? lane : (lane & ~3) | ((lane & 1) << 1) | ((lane >> 1) & 1);

  for (int b = b0 + wave; b < b1; b += kWaves) {
    const uint8_t* rec = kv + (size_t(g) * nb + b) * R::kBytes;
    // every load of the block first
    u32x4 kc[R::kKChunks], vc[R::kVLoads], kp, vp;
#pragma unroll
    for (int c = 0; c < R::kKChunks; ++c)
      kc[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + R::kKCodes + c * 1024) + lane);
    if constexpr (BITS == 8) {
      const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rec + R::kKPar) + lane);
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rec + R::kVPar) + lane);
      kp = u32x4{a.x, a.y, 0u, 0u};
      vp = u32x4{v.x, v.y, 0u, 0u};
    } else {
      kp = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + R::kKPar) + lane);
      vp = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + R::kVPar) + lane);
    }
    if (b == b0 + wave) {  // this wave's first block: its loads are out, form the query sums
      float qs[kQLoads];
#pragma unroll
      for (int c = 0; c < kQLoads; ++c) {
        asm volatile("" : "+v"(qv[c]));  // keeps the sums here, after the block's loads
        float t = dot2(qv[c].x, kOnes, 0.f);
        t = dot2(qv[c].y, kOnes, t);
        t = dot2(qv[c].z, kOnes, t);
        t = dot2(qv[c].w, kOnes, t);
        t += dpp<0xB1>(t);  // quad_perm [1,0,3,2]
        qs[c] = t + dpp<0x4E>(t);  // quad_perm [2,3,0,1]: the group's sum in each lane of its quad
      }
#pragma unroll
      for (int gi = 0; gi < GQ * 4; ++gi)
        qsum[gi / 4][gi % 4] =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qs[gi / 16]), 4 * (gi % 16)));
    }
    static_assert(kKPar * kBlockTokens == 512 || kKPar * kBlockTokens == 1024, "parameter layout");
    float vs[4], vm[4];  // this lane's token's value scales (and mins)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      if constexpr (BITS == 8) {
        vs[grp] = (grp & 1) ? half_hi(elem(vp, grp >> 1)) : half_lo(elem(vp, grp >> 1));
        vm[grp] = 0.f;
      } else {
        vs[grp] = half_lo(elem(vp, grp));
        vm[grp] = half_hi(elem(vp, grp));
      }
    }
    // block scale 2^E: every |p * s_v| * 2^E stays below 2^14, so the binary16
    // weights are normal numbers down to 2^-28 of the block's largest scale
    float smax = fmaxf(fmaxf(fabsf(vs[0]), fabsf(vs[1])), fmaxf(fabsf(vs[2]), fabsf(vs[3])));
    smax = uniform(wave_max(smax));
    const int E = __builtin_amdgcn_readfirstlane(14 - (smax > 0.f ? __builtin_amdgcn_frexp_expf(smax) : 0));

    // phase 1: one lane per token
    const bool valid = b * kBlockTokens + lane < T;
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
      const float sc = valid ? key_score<BITS>(kc, kp, q + (g * GQ + j) * (kD / 2), qsum[j]) * scale_log2
                             : -__builtin_inff();
      const float m_new = uniform(fmaxf(m[j], wave_max(sc)));  // finite: every block has a valid token
      const float corr = __builtin_amdgcn_exp2f(m[j] - m_new);
      const float p = __builtin_amdgcn_exp2f(sc - m_new);
      m[j] = m_new;
      l[j] = __builtin_fmaf(l[j], corr, p);
      acc[j][0] *= corr;
      acc[j][1] *= corr;
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        // the token's weight p * s_v, rounded to binary16 at scale 2^E; the
        // offset / min term is formed from the same rounded weight, so the
        // rounding only perturbs each token's weight by 2^-11 relative
        const float ps = p * vs[grp];
        const _Float16 h = _Float16(__builtin_ldexpf(ps, E));
        const float wr = __builtin_ldexpf(float(h), -E);
        if constexpr (BITS == 8) {
          off[j][grp] = __builtin_fmaf(off[j][grp], corr, -128.f * wr);
        } else {
          const float fix = vs[grp] != 0.f ? (wr - ps) * (vm[grp] * __builtin_amdgcn_rcpf(vs[grp])) : 0.f;
          off[j][grp] = __builtin_fmaf(off[j][grp], corr, __builtin_fmaf(p, vm[grp], fix));
        }
        wh[wave][j][grp][wpos] = h;
      }
    }
    // the value codes are loaded only now: their registers are live in
    // phase 2 only, which keeps the kernel at more waves per SIMD
#pragma unroll
    for (int c = 0; c < R::kVLoads; ++c)
      vc[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + R::kVCodes + c * 1024) + lane);
    wave_lds_sync();  // phase 2 reads the weights other lanes wrote

    // phase 2: one lane per two dims (2*lane, 2*lane + 1); the value codes are
    // binary16 subnormal pairs over two tokens, dotted with the weight pairs
    if constexpr (BITS == 8) {
      float blk[GQ][2];
#pragma unroll
      for (int j = 0; j < GQ; ++j) blk[j][0] = blk[j][1] = 0.f;
#pragma unroll
      for (int c = 0; c < R::kVLoads; ++c) {  // tokens 8c .. 8c+7; word wd = tokens 8c+2wd, +1
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
          const u32x4 wp = *reinterpret_cast<const u32x4*>(&wh[wave][j][vgrp][8 * c]);
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) {
            const uint32_t w = elem(vc[c], wd);  // bytes (t0 d0, t0 d1, t1 d0, t1 d1), each q + 128
            blk[j][0] = dot2(w & 0x00FF00FFu, elem(wp, wd), blk[j][0]);
            blk[j][1] = dot2((w >> 8) & 0x00FF00FFu, elem(wp, wd), blk[j][1]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < GQ; ++j) {  // codes were q + 128 times 2^-24, weights times 2^E
        acc[j][0] = __builtin_fmaf(blk[j][0], __builtin_ldexpf(1.f, 24 - E), acc[j][0]);
        acc[j][1] = __builtin_fmaf(blk[j][1], __builtin_ldexpf(1.f, 24 - E), acc[j][1]);
      }
    } else {
      float lo[GQ], hi[GQ];
#pragma unroll
      for (int j = 0; j < GQ; ++j) lo[j] = hi[j] = 0.f;
#pragma unroll
      for (int c = 0; c < R::kVLoads; ++c) {  // tokens 16c .. 16c+15
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
          const u32x4 wa = *reinterpret_cast<const u32x4*>(&wh[wave][j][vgrp][16 * c]);
          const u32x4 wb = *reinterpret_cast<const u32x4*>(&wh[wave][j][vgrp][16 * c + 8]);
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) {  // tokens 16c + 4wd + i in byte i: (low nibble d0, high nibble d1)
            const uint32_t w = elem(vc[c], wd), w8 = w >> 8;
            const uint32_t p02 = wd < 2 ? elem(wa, 2 * wd) : elem(wb, 2 * wd - 4);      // weights (t0, t2)
            const uint32_t p13 = wd < 2 ? elem(wa, 2 * wd + 1) : elem(wb, 2 * wd - 3);  // weights (t1, t3)
            lo[j] = dot2(w & 0x000F000Fu, p02, lo[j]);
            hi[j] = dot2(w & 0x00F000F0u, p02, hi[j]);
            lo[j] = dot2(w8 & 0x000F000Fu, p13, lo[j]);
            hi[j] = dot2(w8 & 0x00F000F0u, p13, hi[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < GQ; ++j) {  // dim d0 in units of 2^-24, d1 of 2^-20, weights times 2^E
        acc[j][0] = __builtin_fmaf(lo[j], __builtin_ldexpf(1.f, 24 - E), acc[j][0]);
        acc[j][1] = __builtin_fmaf(hi[j], __builtin_ldexpf(1.f, 20 - E), acc[j][1]);
      }
    }
    wave_lds_sync();  // the next block's phase 1 overwrites the weights just read
  }

  // this wave's partial: maximum (uniform), weight sum, weighted values; the
  // offset / min terms of the value groups are summed over the wave's tokens
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float lsum = wave_sum(l[j]);
    float o4[4];
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) o4[grp] = wave_sum(off[j][grp]);
    const float oq = vgrp == 0 ? o4[0] : vgrp == 1 ? o4[1] : vgrp == 2 ? o4[2] : o4[3];
    comb[wave][j][2 * lane] = acc[j][0] + oq;
    comb[wave][j][2 * lane + 1] = acc[j][1] + oq;
    if (lane == 0) {
      comb[wave][j][kD] = m[j];
      comb[wave][j][kD + 1] = lsum;
    }
  }
  __syncthreads();
  // merge the waves in order 0..3 (a wave without blocks has maximum -inf and
  // weight 0; wave 0 always has a block)
  for (int i = threadIdx.x; i < GQ * kD; i += 64 * kWaves) {
    const int j = i / kD, d = i % kD;
    float mx = comb[0][j][kD];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, comb[w][j][kD]);
    float a = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(comb[w][j][kD] - mx);
      a = __builtin_fmaf(f, comb[w][j][d], a);
      ls = __builtin_fmaf(f, comb[w][j][kD + 1], ls);
    }
    float* out = part + (size_t(g * S + split) * GQ + j) * kPartFloats;
    out[d] = a;
    if (d == 0) {
      out[kD] = mx;
      out[kD + 1] = ls;
    }
  }
}

// One workgroup of 512 threads per query head h: merge the S partials of h's
// KV head. The maximum is a reduction over all threads; the weighted sums are
// split into 4 fixed slices of the partials (slice k takes s = k, k+4, ...),
// each thread summing one dim of one slice with its loads issued 8 at a
// time, and the slices are added in order 0..3: a fixed summation order.
constexpr int kMergeThreads = 512, kMergeSlices = kMergeThreads / kD, kMergeUnroll = 8;
static_assert(kMergeSlices == 4, "the final sum below adds four slices");

template <int GQ>
__global__ void __launch_bounds__(kMergeThreads) kv_combine_kernel(const float* __restrict__ part, float* __restrict__ o,
                                                                  int S) {
  const int h = blockIdx.x;
  const int g = h / GQ, j = h % GQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = tid % kD, k = tid / kD;
  const float* p = part + (size_t(g * S) * GQ + j) * kPartFloats;
  const size_t stride = size_t(GQ) * kPartFloats;
  __shared__ float red[kMergeThreads / 64];
  __shared__ float accs[kMergeSlices][kD];
  __shared__ float lss[kMergeSlices];

  float mx = -__builtin_inff();
  for (int s = tid; s < S; s += kMergeThreads) mx = fmaxf(mx, p[s * stride + kD]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w]);

  float a = 0.f, ls = 0.f;
  for (int s0 = k; s0 < S; s0 += kMergeSlices * kMergeUnroll) {
    float mv[kMergeUnroll], av[kMergeUnroll], lv[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {  // clamped, unconditional loads
      const int s = s0 + kMergeSlices * u;
      const size_t c = size_t(s < S ? s : 0) * stride;  // partial 0 always exists (S >= 1)
      mv[u] = p[c + kD];
      av[u] = p[c + d];
      lv[u] = p[c + kD + 1];
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float f = s0 + kMergeSlices * u < S ? __builtin_amdgcn_exp2f(mv[u] - M) : 0.f;
      a = __builtin_fmaf(f, av[u], a);
      ls = __builtin_fmaf(f, lv[u], ls);
    }
  }
  accs[k][d] = a;
  if (d == 0) lss[k] = ls;
  __syncthreads();
  if (k == 0) {
    const float num = (accs[0][d] + accs[1][d]) + (accs[2][d] + accs[3][d]);
    const float den = (lss[0] + lss[1]) + (lss[2] + lss[3]);
    o[size_t(h) * kD + d] = num / den;
  }
}

typedef void (*attn_fn)(const uint32_t*, const uint8_t*, float*, int, int, int, float);
typedef void (*comb_fn)(const float*, float*, int);

template <int BITS>
attn_fn attn_for(int gq) {
  switch (gq) {
    case 1: return &kv_attn_kernel<BITS, 1>;
    case 2: return &kv_attn_kernel<BITS, 2>;
    case 4: return &kv_attn_kernel<BITS, 4>;
    case 8: return &kv_attn_kernel<BITS, 8>;
    default: return nullptr;
  }
}
comb_fn comb_for(int gq) {
  switch (gq) {
    case 1: return &kv_combine_kernel<1>;
    case 2: return &kv_combine_kernel<2>;
    case 4: return &kv_combine_kernel<4>;
    case 8: return &kv_combine_kernel<8>;
    default: return nullptr;
  }
}

constexpr int32_t kMaxT = 1 << 24;

int64_t record_bytes(int bits) { return bits == 8 ? Rec<8>::kBytes : Rec<4>::kBytes; }

bool shape_ok(int32_t bits, int32_t T, int32_t Hq, int32_t Hkv) {
  if (bits != 8 && bits != 4) return false;
  if (T < 1 || T > kMaxT || Hkv < 1 || Hq < Hkv || Hq % Hkv) return false;
  const int gq = Hq / Hkv;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8) return false;
  return int64_t(Hq) <= 4096;
}

// Waves of the attention kernel that fit on the device at once (cached per
// instantiation; without a device, the gfx950 figure for 4 query heads per
// KV head: three workgroups per CU).
int resident_waves(int bits, int gq, int cus, bool have_device) {
  static std::atomic<int> cache[2][4];
  const int bi = bits == 8 ? 0 : 1, gi = gq == 1 ? 0 : gq == 2 ? 1 : gq == 4 ? 2 : 3;
  int occ = cache[bi][gi].load(std::memory_order_relaxed);
  if (occ <= 0) {
    if (!have_device) return cus * 3 * kWaves;
    const attn_fn fa = bits == 8 ? attn_for<8>(gq) : attn_for<4>(gq);
    occ = w4a16_host::occupancy_of(reinterpret_cast<const void*>(fa), 64 * kWaves);
    cache[bi][gi].store(occ, std::memory_order_relaxed);
  }
  return cus * occ * kWaves;
}

// Blocks per workgroup: as few as keep every workgroup resident in one round
// (each wave then walks its blocks with no wave waiting for a free slot),
// four blocks or more per workgroup (one per wave), a multiple of four.
int blocks_per_wg(int nb, int Hkv, int resident) {
  int64_t bw = (int64_t(nb) * Hkv + resident - 1) / resident;
  if (bw < 1) bw = 1;
  return int(4 * bw);
}

// The most partials a launch can produce for (T, Hq): every workgroup has at
// least four blocks unless the head has fewer.
int64_t max_partials(int32_t T, int32_t Hq) {
  const int64_t nb = (int64_t(T) + kBlockTokens - 1) / kBlockTokens;
  return int64_t(Hq) * ((nb + 3) / 4);
}

w4a16_status kv_enqueue(int32_t bits, const void* q, const void* kv, float* o, int32_t T, int32_t Hq, int32_t Hkv,
                        void* workspace, size_t workspace_bytes, void* stream, hipEvent_t start, hipEvent_t stop) {
  if (!q || !kv || !o || !workspace) return W4A16_ERR_NULL;
  if (!shape_ok(bits, T, Hq, Hkv)) return W4A16_ERR_SHAPE;
  const uintptr_t qa = reinterpret_cast<uintptr_t>(q), ka = reinterpret_cast<uintptr_t>(kv);
  const uintptr_t oa = reinterpret_cast<uintptr_t>(o), wa = reinterpret_cast<uintptr_t>(workspace);
  if (qa % 16 || ka % 256 || oa % 16 || wa % 16) return W4A16_ERR_ALIGN;
  const int nb = (T + kBlockTokens - 1) / kBlockTokens;
  const size_t cache = size_t(Hkv) * size_t(nb) * size_t(record_bytes(bits));
  const size_t need = size_t(max_partials(T, Hq)) * kPartFloats * sizeof(float);
  if (workspace_bytes < need) return W4A16_ERR_SIZE;
  const size_t obytes = size_t(Hq) * kD * sizeof(float);
  using w4a16_host::ranges_overlap;
  if (ranges_overlap(oa, obytes, qa, size_t(Hq) * kD * 2) || ranges_overlap(oa, obytes, ka, cache) ||
      ranges_overlap(oa, obytes, wa, need) || ranges_overlap(wa, need, qa, size_t(Hq) * kD * 2) ||
      ranges_overlap(wa, need, ka, cache))
    return W4A16_ERR_OVERLAP;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  const int gq = Hq / Hkv;
  const int bpw = blocks_per_wg(nb, Hkv, resident_waves(bits, gq, w4a16_host::cu_count(dev), true));
  const int S = (nb + bpw - 1) / bpw;
  const attn_fn fa = bits == 8 ? attn_for<8>(gq) : attn_for<4>(gq);
  const comb_fn fc = comb_for(gq);
  // log2(e) / sqrt(128): scores go to the exp2 domain
  const float scale_log2 = 1.4426950408889634f * 0.08838834764831845f;
  const uint32_t* qp = static_cast<const uint32_t*>(q);
  const uint8_t* kp = static_cast<const uint8_t*>(kv);
  float* pp = static_cast<float*>(workspace);
  int t_arg = T, nb_arg = nb, bpw_arg = bpw, s_arg = S;
  float sc_arg = scale_log2;
  void* a1[] = {&qp, &kp, &pp, &t_arg, &nb_arg, &bpw_arg, &sc_arg};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // the events (if any) bracket the split attention pass, the dominant kernel
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fa), dim3(S, Hkv), dim3(64 * kWaves), a1, 0, st, start,
                         stop, 0) != hipSuccess)
    return W4A16_ERR_HIP;
  const float* cp = pp;
  void* a2[] = {&cp, &o, &s_arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fc), dim3(Hq), dim3(kMergeThreads), a2, 0, st, nullptr, nullptr, 0) !=
      hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}

}  // namespace

extern "C" size_t w4a16_kv_packed_bytes(int32_t bits, int32_t T, int32_t Hkv) {
  if ((bits != 8 && bits != 4) || T < 1 || T > kMaxT || Hkv < 1 || Hkv > 4096) return 0;
  const int64_t nb = (int64_t(T) + kBlockTokens - 1) / kBlockTokens;
  return size_t(int64_t(Hkv) * nb * record_bytes(bits));
}

extern "C" size_t w4a16_kv_workspace_bytes(int32_t T, int32_t Hq) {
  if (T < 1 || T > kMaxT || Hq < 1 || Hq > 4096) return 0;
  return size_t(max_partials(T, Hq)) * kPartFloats * sizeof(float);
}

extern "C" w4a16_status w4a16_kv_attention(int32_t bits, const void* q, const void* kv, float* o, int32_t T,
                                           int32_t Hq, int32_t Hkv, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  return kv_enqueue(bits, q, kv, o, T, Hq, Hkv, workspace, workspace_bytes, stream, nullptr, nullptr);
}

extern "C" w4a16_status w4a16_kv_attention_timed(int32_t bits, const void* q, const void* kv, float* o, int32_t T,
                                                 int32_t Hq, int32_t Hkv, void* workspace, size_t workspace_bytes,
                                                 void* stream, void* start_event, void* stop_event) {
  if (!start_event || !stop_event) return W4A16_ERR_NULL;
  return kv_enqueue(bits, q, kv, o, T, Hq, Hkv, workspace, workspace_bytes, stream,
                    static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
}

extern "C" w4a16_status w4a16_kv_launch_shape(int32_t bits, int32_t T, int32_t Hq, int32_t Hkv, int32_t out[3]) {
  if (!out) return W4A16_ERR_NULL;
  if (!shape_ok(bits, T, Hq, Hkv)) return W4A16_ERR_SHAPE;
  int dev = 0, ndev = 0;
  const bool have_device = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0 && hipGetDevice(&dev) == hipSuccess;
  const int cus = have_device ? w4a16_host::cu_count(dev) : 256;
  const int nb = (T + kBlockTokens - 1) / kBlockTokens;
  const int bpw = blocks_per_wg(nb, Hkv, resident_waves(bits, Hq / Hkv, cus, have_device));
  out[0] = Hq / Hkv;
  out[1] = bpw;
  out[2] = (nb + bpw - 1) / bpw;
  return W4A16_OK;
}
