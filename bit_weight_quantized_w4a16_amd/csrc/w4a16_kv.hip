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
//   (INT8) or eight (INT4) waves takes a contiguous range of a head's blocks;
//   its waves take the blocks round-robin. All GQ query heads that share the KV head are served
//   by the same pass over the block, so the cache is read once for all of them.
// * The two products of a block are small dense contractions over four query
//   heads (GQ = 4 per KV head in the 8B model), so they run on the matrix
//   cores (v_mfma_f32_4x4x4_16b_f16, the heads as the four rows), with the
//   codes turned into binary16 subnormal operands by masking: exact, no
//   per-value conversions.
// * Phase 1, one lane per token: the key codes of its token (chunks laid out
//   so that each load instruction reads 1 KiB contiguously) against the
//   query rows held in LDS give its scores for four heads per MFMA, group by
//   group of 32 dims; the group scale and offset fold them. An online softmax
//   across the wave keeps the running maximum per query head, and each lane
//   writes its token's binary16 weights p * s_v to LDS.
// * Phase 2, one lane per head dimension (two halves of 64 dims): the value
//   codes of four tokens of its dim against the weights of those tokens give
//   the weighted values of four heads per MFMA.
// * The waves' partial results are merged through LDS in a fixed order
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
// Waves per workgroup: four for INT8 caches, eight for INT4 (measured: the
// INT4 kernel is faster in larger workgroups with fewer partials per head, the
// INT8 one in smaller).
constexpr int waves_of(int bits) { return bits == 8 ? 4 : 8; }
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

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float half_lo(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xFFFFu))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16))); }

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Four binary16 numbers from two words (halves in order lo(a), hi(a), lo(b), hi(b)).
__device__ __forceinline__ h4 halves(uint32_t a, uint32_t b) { return __builtin_bit_cast(h4, u32x2{a, b}); }
__device__ __forceinline__ h4 lds_h4(const _Float16* p) { return *reinterpret_cast<const h4*>(p); }

// v_mfma_f32_4x4x4_16b_f16: sixteen independent 4x4x4 products per wave. For
// block b = lane / 4 the lane 4b + i holds row i of A (four k), the lane
// 4b + j column j of B, and the result D_b[i][j] lands in register i of lane
// 4b + j. Binary16 subnormal inputs are exact.
__device__ __forceinline__ f4 mfma4(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0); }

// The split attention pass. Both dot products run on the matrix cores with
// four query heads as the MFMA's four rows:
// * scores: A = four heads' query dims (from LDS, lane & 3 = head), B = this
//   lane's token's key dims as binary16 subnormal pairs (lane = token); the
//   result gives lane t the scores of its token for the four heads;
// * values: A = the binary16 weights of four tokens (from LDS, lane & 3 =
//   head), B = the value codes of four tokens for one dim (lane = dim); the
//   result gives lane d the weighted values of dim 64h + d for the four heads.
template <int BITS, int GQ>
__global__ void __launch_bounds__(64 * waves_of(BITS))
kv_attn_kernel(const uint32_t* __restrict__ q_pairs, const uint8_t* __restrict__ kv, float* __restrict__ part, int T,
               int nb, int bpw, float scale_log2, int S) {
  using R = Rec<BITS>;
  constexpr int kWaves = waves_of(BITS);
  constexpr int HG = (GQ + 3) / 4;       // groups of four query heads: the rows of one MFMA
  constexpr int kKPar = BITS == 8 ? 8 : 16;  // parameter bytes per token
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.y;           // KV head
  const int split = blockIdx.x;
  // S (splits per KV head, the grid's x extent) is an argument: explicit
  // arguments arrive preloaded in scalar registers, gridDim.x would be a load
  const int b0 = split * bpw;
  const int b1 = min(b0 + bpw, nb);

  // binary16 token weights p * s_v * 2^E per (wave, head, value group, token)
  __shared__ __attribute__((aligned(16))) _Float16 wh[kWaves][4 * HG][4][kBlockTokens];
  // this wave's copy of the query rows (heads past GQ are zero)
  __shared__ __attribute__((aligned(16))) _Float16 qh[kWaves][4 * HG][kD];
  __shared__ float comb[kWaves][GQ][kPartFloats];

  // The query: 4 * HG rows of 256 bytes, 16 chunks of 16 bytes each; lane i
  // of load c takes chunk 64c + i (head i / 16, group (i / 4) % 4). The loads
  // go out before the first block's loads; the per-group sums and the LDS
  // copy are formed after them, so the two latencies overlap.
  u32x4 qv[HG];
#pragma unroll
  for (int c = 0; c < HG; ++c) {
    const int i = 64 * c + lane;
    qv[c] = reinterpret_cast<const u32x4*>(q_pairs + size_t(g) * GQ * (kD / 2))[i < GQ * 16 ? i : 0];
  }
  float qsum[4 * HG][4];  // per head and group: the offset / min terms of the score
#pragma unroll
  for (int j = 0; j < 4 * HG; ++j)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) qsum[j][grp] = 0.f;
  // heads past GQ have zero weights, so the value products ignore them
  if constexpr (GQ < 4) {
#pragma unroll
    for (int j = GQ; j < 4; ++j)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) wh[wave][j][grp][lane] = _Float16(0.f);
  }

  // Running state per query head j: the maximum m (uniform, exp2 domain) and,
  // in real units, l (the weight sum of this lane's tokens), acc (the weighted
  // values of dims lane and 64 + lane) and off[grp] (the offset / min term of
  // this lane's tokens for value group grp).
  float m[GQ], l[GQ], acc[4 * HG][2], off[GQ][4];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    m[j] = -__builtin_inff();
    l[j] = 0.f;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) off[j][grp] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < 4 * HG; ++j) acc[j][0] = acc[j][1] = 0.f;
  const int qrow = lane & 3;         // the head row this lane feeds to the MFMA's A operand
  const int vgrp_hi = lane >> 5;     // value group of this lane's dims, minus 2h

  for (int b = b0 + wave; b < b1; b += kWaves) {
    const uint8_t* rec = kv + (size_t(g) * nb + b) * R::kBytes;
    // every key load of the block first
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
    if (b == b0 + wave) {  // this wave's first block: its loads are out; the query sums and LDS copy
      float qs[HG];
#pragma unroll
      for (int c = 0; c < HG; ++c) {
        asm volatile("" : "+v"(qv[c]));  // keeps this work here, after the block's loads
        float t = dot2(qv[c].x, kOnes, 0.f);
        t = dot2(qv[c].y, kOnes, t);
        t = dot2(qv[c].z, kOnes, t);
        t = dot2(qv[c].w, kOnes, t);
        t += dpp<0xB1>(t);         // quad_perm [1,0,3,2]
        qs[c] = t + dpp<0x4E>(t);  // quad_perm [2,3,0,1]: the group's sum in each lane of its quad
        const int i = 64 * c + lane;  // chunk i: head i / 16, dims 8 (i % 16) .. + 7
        *reinterpret_cast<u32x4*>(&qh[wave][i / 16][8 * (i % 16)]) = i < GQ * 16 ? qv[c] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int gi = 0; gi < GQ * 4; ++gi)
        qsum[gi / 4][gi % 4] =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qs[gi / 16]), 4 * (gi % 16)));
      wave_lds_sync();  // the MFMAs read rows other lanes wrote
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

    // phase 1: scores of this lane's token for every head, group by group (the
    // key scale and offset apply per group of 32 dims)
    float sc[4 * HG];
#pragma unroll
    for (int j = 0; j < 4 * HG; ++j) sc[j] = 0.f;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      f4 dl[HG], dh[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) dl[hg] = dh[hg] = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BITS == 8) {
#pragma unroll
        for (int s4 = 0; s4 < 8; ++s4) {  // dims 32 grp + 4 s4 .. + 3: word s4 % 4 of chunk 2 grp + s4 / 4
          const uint32_t w = elem(kc[2 * grp + s4 / 4], s4 % 4);  // bytes: dims (0, 2, 1, 3), each q + 128
          const h4 kb = halves(w & 0x00FF00FFu, (w >> 8) & 0x00FF00FFu);
#pragma unroll
          for (int hg = 0; hg < HG; ++hg)
            dl[hg] = mfma4(lds_h4(&qh[wave][4 * hg + qrow][32 * grp + 4 * s4]), kb, dl[hg]);
        }
        const float s = (grp & 1) ? half_hi(elem(kp, grp >> 1)) : half_lo(elem(kp, grp >> 1));
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[4 * hg + i] = __builtin_fmaf(s * 0x1p24f, dl[hg][i], sc[4 * hg + i]);
            sc[4 * hg + i] = __builtin_fmaf(-128.f * s, qsum[4 * hg + i][grp], sc[4 * hg + i]);
          }
      } else {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {  // dims 32 grp + 8 wd + 0..3 (low nibbles), + 4..7 (high nibbles)
          const uint32_t w = elem(kc[grp], wd), w8 = w >> 8;
          const h4 klo = halves(w & 0x000F000Fu, w8 & 0x000F000Fu);  // q * 2^-24
          const h4 khi = halves(w & 0x00F000F0u, w8 & 0x00F000F0u);  // q * 2^-20
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            dl[hg] = mfma4(lds_h4(&qh[wave][4 * hg + qrow][32 * grp + 8 * wd]), klo, dl[hg]);
            dh[hg] = mfma4(lds_h4(&qh[wave][4 * hg + qrow][32 * grp + 8 * wd + 4]), khi, dh[hg]);
          }
        }
        const uint32_t par = elem(kp, grp);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[4 * hg + i] =
                __builtin_fmaf(half_lo(par) * 0x1p20f, __builtin_fmaf(dl[hg][i], 16.f, dh[hg][i]), sc[4 * hg + i]);
            sc[4 * hg + i] = __builtin_fmaf(half_hi(par), qsum[4 * hg + i][grp], sc[4 * hg + i]);
          }
      }
    }

    // online softmax per head, and the binary16 weights
    const bool valid = b * kBlockTokens + lane < T;
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
      const float scj = valid ? sc[j] * scale_log2 : -__builtin_inff();
      const float m_new = uniform(fmaxf(m[j], wave_max(scj)));  // finite: every block has a valid token
      const float corr = __builtin_amdgcn_exp2f(m[j] - m_new);
      const float p = __builtin_amdgcn_exp2f(scj - m_new);
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
        wh[wave][j][grp][lane] = h;
      }
    }
    // the value codes are loaded only now: their registers are live in
    // phase 2 only, which keeps the kernel at more waves per SIMD
#pragma unroll
    for (int c = 0; c < R::kVLoads; ++c)
      vc[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + R::kVCodes + c * 1024) + lane);
    wave_lds_sync();  // phase 2 reads the weights other lanes wrote

    // phase 2: lane d accumulates dims d and 64 + d; A = the weights of four
    // tokens for head row lane & 3 and the value group of the lane's block
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int vg = 2 * hh + vgrp_hi;
      f4 dl[HG], dh[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) dl[hg] = dh[hg] = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BITS == 8) {
#pragma unroll
        for (int s4 = 0; s4 < 16; ++s4) {  // tokens 4 s4 .. + 3: word s4 % 4 of load 4 hh + s4 / 4
          const uint32_t w = elem(vc[4 * hh + s4 / 4], s4 % 4);  // bytes: tokens (0, 2, 1, 3), each q + 128
          const h4 vb = halves(w & 0x00FF00FFu, (w >> 8) & 0x00FF00FFu);
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) dl[hg] = mfma4(lds_h4(&wh[wave][4 * hg + qrow][vg][4 * s4]), vb, dl[hg]);
        }
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
#pragma unroll
          for (int i = 0; i < 4; ++i)  // codes were q + 128 times 2^-24, weights times 2^E
            acc[4 * hg + i][hh] = __builtin_fmaf(dl[hg][i], __builtin_ldexpf(1.f, 24 - E), acc[4 * hg + i][hh]);
      } else {
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {  // tokens 8 s8 .. + 7: word s8 % 4 of load 2 hh + s8 / 4
          const uint32_t w = elem(vc[2 * hh + s8 / 4], s8 % 4), w8 = w >> 8;
          const h4 vlo = halves(w & 0x000F000Fu, w8 & 0x000F000Fu);  // tokens 0..3, q * 2^-24
          const h4 vhi = halves(w & 0x00F000F0u, w8 & 0x00F000F0u);  // tokens 4..7, q * 2^-20
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            dl[hg] = mfma4(lds_h4(&wh[wave][4 * hg + qrow][vg][8 * s8]), vlo, dl[hg]);
            dh[hg] = mfma4(lds_h4(&wh[wave][4 * hg + qrow][vg][8 * s8 + 4]), vhi, dh[hg]);
          }
        }
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
#pragma unroll
          for (int i = 0; i < 4; ++i) {  // low nibbles in units of 2^-24, high of 2^-20, weights times 2^E
            acc[4 * hg + i][hh] = __builtin_fmaf(dl[hg][i], __builtin_ldexpf(1.f, 24 - E), acc[4 * hg + i][hh]);
            acc[4 * hg + i][hh] = __builtin_fmaf(dh[hg][i], __builtin_ldexpf(1.f, 20 - E), acc[4 * hg + i][hh]);
          }
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
    comb[wave][j][lane] = acc[j][0] + (vgrp_hi == 0 ? o4[0] : o4[1]);
    comb[wave][j][64 + lane] = acc[j][1] + (vgrp_hi == 0 ? o4[2] : o4[3]);
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
// KV head, kMergeChunk partials at a time (one chunk for the 8B shapes).
// Per chunk: thread t < n loads the maximum and weight sum of partial t; a
// block reduction gives the chunk's maximum and, in LDS, each partial's
// factor exp2(m_s - M); each thread, one dim of one of 4 fixed slices of the
// partials (slice k takes s = k, k+4, ...), has issued its weighted-value
// loads at the start of the chunk and sums them with those factors. The
// slices are added in order 0..3: a fixed summation order, so the result is
// bitwise repeatable.
constexpr int kMergeThreads = 512, kMergeSlices = kMergeThreads / kD, kMergeUnroll = 24;
constexpr int kMergeChunk = kMergeSlices * kMergeUnroll;  // partials per chunk
constexpr int kMergeWaves = kMergeThreads / 64;
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
  __shared__ float fs[kMergeChunk];
  __shared__ float red[kMergeWaves];
  __shared__ float accs[kMergeSlices][kD];

  float M = -__builtin_inff(), a = 0.f, den = 0.f;
  for (int c0 = 0; c0 < S; c0 += kMergeChunk) {
    const int n = min(kMergeChunk, S - c0);
    float av[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {  // clamped, unconditional loads
      const int s = k + kMergeSlices * u;
      av[u] = p[size_t(c0 + (s < n ? s : 0)) * stride + d];
    }
    const size_t ct = size_t(c0 + (tid < n ? tid : 0)) * stride;
    const float mv = tid < n ? p[ct + kD] : -__builtin_inff();
    const float lv = tid < n ? p[ct + kD + 1] : 0.f;
    // the chunk's maximum over the block
    float cm = wave_max(mv);
    if (lane == 0) red[wave] = cm;
    __syncthreads();
    cm = red[0];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) cm = fmaxf(cm, red[w]);
    const float M_new = fmaxf(M, cm);  // finite: every chunk has a partial
    const float r = __builtin_amdgcn_exp2f(M - M_new);  // 0 on the first chunk
    const float f = tid < n ? __builtin_amdgcn_exp2f(mv - M_new) : 0.f;
    if (tid < kMergeChunk) fs[tid] = f;
    // the chunk's weight sum over the block, in wave order
    const float ws = wave_sum(f * lv);
    __syncthreads();  // every wave has read red[] and written fs[]
    if (lane == 0) red[wave] = ws;
    __syncthreads();
    float cden = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) cden += red[w];
    den = __builtin_fmaf(den, r, cden);
    a *= r;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u)  // fs[] is 0 past n, and av[] there is partial 0's, finite
      a = __builtin_fmaf(fs[k + kMergeSlices * u], av[u], a);
    M = M_new;
    __syncthreads();  // fs[] and red[] are rewritten by the next chunk
  }
  accs[k][d] = a;
  __syncthreads();
  if (k == 0) o[size_t(h) * kD + d] = ((accs[0][d] + accs[1][d]) + (accs[2][d] + accs[3][d])) / den;
}

typedef void (*attn_fn)(const uint32_t*, const uint8_t*, float*, int, int, int, float, int);
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
    if (!have_device) return cus * 3 * 4;
    const attn_fn fa = bits == 8 ? attn_for<8>(gq) : attn_for<4>(gq);
    occ = w4a16_host::occupancy_of(reinterpret_cast<const void*>(fa), 64 * waves_of(bits));
    cache[bi][gi].store(occ, std::memory_order_relaxed);
  }
  return cus * occ * waves_of(bits);
}

// Blocks per workgroup: as few as keep every workgroup resident in one round
// (each wave then walks its blocks with no wave waiting for a free slot), a
// multiple of the workgroup's wave count (at least one block per wave).
int blocks_per_wg(int nb, int Hkv, int resident, int waves) {
  int64_t bw = (int64_t(nb) * Hkv + resident - 1) / resident;
  if (bw < 1) bw = 1;
  return int(waves * bw);
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
  const int bpw = blocks_per_wg(nb, Hkv, resident_waves(bits, gq, w4a16_host::cu_count(dev), true), waves_of(bits));
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
  void* a1[] = {&qp, &kp, &pp, &t_arg, &nb_arg, &bpw_arg, &sc_arg, &s_arg};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // the events (if any) bracket the split attention pass, the dominant kernel
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fa), dim3(S, Hkv), dim3(64 * waves_of(bits)), a1, 0, st,
                         start, stop, 0) != hipSuccess)
    return W4A16_ERR_HIP;
  const float* cp = pp;
  void* a2[] = {&cp, &o, &s_arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fc), dim3(Hq), dim3(kMergeThreads), a2, 0, st, nullptr, nullptr, 0) !=
      hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}

}  // namespace

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

namespace {

// The partials of w4a16_kv_attention_static: a file-scope array that every
// device holds its own copy of, for as long as the process lives. Its name
// in host code is a host-side stand-in, never a device address: host code
// uses only the per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[W4A16_KV_STATIC_WORKSPACE_BYTES / sizeof(float)];

// Device address of `scratch` on device `dev`, looked up on the first call
// on that device (which must be current) and kept; nullptr on failure.
float* scratch_on(int dev) {
  static std::atomic<float*> cache[w4a16_host::kMaxDevices];
  if (dev < 0 || dev >= w4a16_host::kMaxDevices) return nullptr;
  float* ptr = cache[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  cache[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" w4a16_status w4a16_kv_attention_static(int32_t bits, const void* q, const void* kv, float* o, int32_t T,
                                                  int32_t Hq, int32_t Hkv, void* stream) {
  if (!q || !kv || !o) return W4A16_ERR_NULL;
  if (!shape_ok(bits, T, Hq, Hkv)) return W4A16_ERR_SHAPE;
  if (w4a16_kv_workspace_bytes(T, Hq) > W4A16_KV_STATIC_WORKSPACE_BYTES) return W4A16_ERR_SIZE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  float* ptr = scratch_on(dev);
  if (!ptr) return W4A16_ERR_HIP;
  // every partial the merge reads is written by the split pass of the same
  // call, so nothing has to be cleared first
  return kv_enqueue(bits, q, kv, o, T, Hq, Hkv, ptr, W4A16_KV_STATIC_WORKSPACE_BYTES, stream, nullptr, nullptr);
}

extern "C" w4a16_status w4a16_kv_launch_shape(int32_t bits, int32_t T, int32_t Hq, int32_t Hkv, int32_t out[3]) {
  if (!out) return W4A16_ERR_NULL;
  if (!shape_ok(bits, T, Hq, Hkv)) return W4A16_ERR_SHAPE;
  int dev = 0, ndev = 0;
  const bool have_device = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0 && hipGetDevice(&dev) == hipSuccess;
  const int cus = have_device ? w4a16_host::cu_count(dev) : 256;
  const int nb = (T + kBlockTokens - 1) / kBlockTokens;
  const int bpw = blocks_per_wg(nb, Hkv, resident_waves(bits, Hq / Hkv, cus, have_device), waves_of(bits));
  out[0] = Hq / Hkv;
  out[1] = bpw;
  out[2] = (nb + bpw - 1) / bpw;
  return W4A16_OK;
}
