// The single-GEMV kernel skeleton, shared by every weight code, and the
// host-side choice of its launch shape. Internal header of libw4a16.
//
// The skeleton streams 4-row tiles of a weight matrix: a lane owns GPL groups
// of 32 k along K and keeps that slice of every activation row in registers,
// the W waves of a workgroup cover W*64*GPL groups per pass over K, each
// tile's loads are issued before the previous tile is computed, lane partials
// are summed across the wave without LDS and across waves through LDS in a
// fixed order. What differs between weight codes is only how one tile is
// loaded and how its codes become dot products; a codec policy supplies
// those two steps:
//
//   template <int GPL> struct Loads;   // one lane's loads of one tile
//   template <int GPL> static void fetch(const WeightPtrs&, int N, int G, int t,
//                                        const int (&g0)[GPL], int lane, Loads<GPL>&);
//   template <int M, int GPL, class XA> static void compute(const Loads<GPL>&, const XA&,
//                                                           float (&acc)[kTileRows][M]);
//   static constexpr int kTileVgprs;    // VGPRs of one group slot's loads
//   static constexpr int kCodec;        // the codec id its blobs' headers carry
//
// compute() returns the lane's partial sums; the skeleton adds them over the
// wave (tile_sums).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16_device.h"

namespace w4a16_dev {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Launch modes of one GEMV.
//   kDirect: one wave covers all of K for its tile and stores the results;
//   kBlock:  the waves of a workgroup split K; per-wave partials of a block
//            of tiles are combined through LDS;
//   kMulti:  K also takes several passes of the workgroup (x re-fetched per
//            pass, partials carried in LDS).
constexpr int kDirect = 0, kBlock = 1, kMulti = 2;

// The next tile's loads are issued before the current tile is computed (two
// load buffers) in every shape except a one-wave workgroup with more than
// four activation rows, where the second buffer would spill (M = 8: 217
// VGPRs and 48 bytes of scratch per lane; 210-232 VGPRs without spills in the
// wider shapes, still two waves per SIMD).
__host__ __device__ constexpr bool double_buffered(int M, int MODE) { return M <= 4 || MODE != kDirect; }

// Regions of one packed blob, in the units the loads use.
struct WeightPtrs {
  const u32x4* codes;  // code chunks
  const u32x4* aux;    // extra per-tile entries (the 5-bit code's fifth-bit plane), else null
  const void* side;    // per-tile scale (and min) entries
};

// Lane-clamped group slot: the lane reads group g0 + base + gl. A lane past G
// reads group G-1 instead (its activations are zero, so it adds exactly 0), a
// slot entirely past G is pulled back to G-1. Every load stays unconditional.
struct Slot {
  int base, gl;
};
__device__ __forceinline__ Slot slot_of(int G, int g0, int lane) {
  const int last = G - 1 - g0;  // wave-uniform; < 0 when the whole slot is past G
  return Slot{last < 0 ? G - 1 - g0 : 0, lane < last ? lane : (last > 0 ? last : 0)};
}
__device__ __forceinline__ int clamp_row(int t, int r, int N) {
  return t * kTileRows + r < N ? t * kTileRows + r : N - 1;
}

// binary16 number h of a 4-row entry of 8 bytes (row r in bytes 2r..2r+1)
__device__ __forceinline__ float half_of(const u32x2& v, int r) {
  const uint32_t w = r < 2 ? v.x : v.y;
  const uint16_t b = uint16_t((r & 1) ? (w >> 16) : (w & 0xFFFFu));
  return float(__builtin_bit_cast(_Float16, b));
}

// ---------------------------------------------------------------------------
// Codec policies
// ---------------------------------------------------------------------------

// 4-bit group-affine code (w_hat = s*q + m): the tile loads and dot products
// of the device header, unchanged.
struct CodecQ4 {
  static constexpr int kCodec = W4A16_CODEC_Q4;
  static constexpr int kTileVgprs = 20;
  template <int GPL>
  using Loads = TileLoads<GPL>;
  template <int GPL>
  __device__ __forceinline__ static void fetch(const WeightPtrs& w, int N, int G, int t, const int (&g0)[GPL],
                                               int lane, Loads<GPL>& L) {
    fetch_tile<GPL>(w.codes, static_cast<const u32x4*>(w.side), N, G, t, g0, lane, L);
  }
  template <int M, int GPL, class XA>
  __device__ __forceinline__ static void compute(const Loads<GPL>& L, const XA& xa, float (&acc)[kTileRows][M]) {
    compute_tile<M, GPL>(L, xa, acc);
  }
};

// The four nibble pairs of one 32-bit code word against one 16-byte chunk of
// x (as in compute_tile): lo gathers q * 2^-24 terms, hi gathers q * 2^-20.
// `five` adds a fifth code bit below each nibble's plane (0 for 4-bit codes):
// bits 4/20 of fa and 8/24 of fa for the first two pairs, of fb for the last
// two, already shifted into place by the caller. `first`: the chunk starts
// lo and hi (from 0) instead of adding to them.
template <int M, bool FIVE>
__device__ __forceinline__ void nibble_dots(uint32_t w, uint32_t fa, uint32_t fb, const u32x4 (&xq)[M],
                                            float (&lo)[M], float (&hi)[M], bool first) {
  const uint32_t w8 = w >> 8;
  uint32_t pa = w & 0x000F000Fu, pb = w & 0x00F000F0u, pc = w8 & 0x000F000Fu, pd = w8 & 0x00F000F0u;
  if constexpr (FIVE) {
    pa |= fa & 0x00100010u;
    pb |= fa & 0x01000100u;
    pc |= fb & 0x00100010u;
    pd |= fb & 0x01000100u;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (first) {
      lo[m] = dot2_from_zero(pa, elem(xq[m], 0));
      hi[m] = dot2_from_zero(pb, elem(xq[m], 1));
    } else {
      lo[m] = dot2(pa, elem(xq[m], 0), lo[m]);
      hi[m] = dot2(pb, elem(xq[m], 1), hi[m]);
    }
    lo[m] = dot2(pc, elem(xq[m], 2), lo[m]);
    hi[m] = dot2(pd, elem(xq[m], 3), hi[m]);
  }
}

// Symmetric 4-bit code (w_hat = s*(q - 8)): the 4-bit code chunks, and one
// 8-byte entry of four binary16 scales per (tile, group).
struct CodecQ4Sym {
  static constexpr int kCodec = W4A16_CODEC_Q4_SYM;
  static constexpr int kTileVgprs = 18;
  template <int GPL>
  struct Loads {
    u32x2 sc[GPL];
    u32x4 code[kTileRows][GPL];
  };
  template <int GPL>
  __device__ __forceinline__ static void fetch(const WeightPtrs& w, int N, int G, int t, const int (&g0)[GPL],
                                               int lane, Loads<GPL>& L) {
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const Slot s = slot_of(G, g0[j], lane);
      const u32x2* sp = static_cast<const u32x2*>(w.side) + (size_t(t) * G + g0[j] + s.base);
      L.sc[j] = __builtin_nontemporal_load(sp + s.gl);
#pragma unroll
      for (int r = 0; r < kTileRows; ++r)
        L.code[r][j] = __builtin_nontemporal_load(w.codes + (size_t(clamp_row(t, r, N)) * G + g0[j] + s.base) + s.gl);
    }
  }
  template <int M, int GPL, class XA>
  __device__ __forceinline__ static void compute(const Loads<GPL>& L, const XA& xa, float (&acc)[kTileRows][M]) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      float lo[kTileRows][M], hi[kTileRows][M];
#pragma unroll
      for (int r = 0; r < kTileRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) lo[r][m] = hi[r][m] = 0.f;
      tile_walk<M>(
          xa, j,
          [&](int r, int d, const u32x4(&xq)[M]) __attribute__((always_inline)) {
            nibble_dots<M, false>(elem(L.code[r][j], d), 0u, 0u, xq, lo[r], hi[r], d == 0);
          },
          [&](int r) __attribute__((always_inline)) {
            const float s = half_of(L.sc[j], r);
            const float sc = s * 0x1p20f;
            const float mn = -8.f * s;  // exact
#pragma unroll
            for (int m = 0; m < M; ++m) {
              acc[r][m] = __builtin_fmaf(sc, __builtin_fmaf(lo[r][m], 16.f, hi[r][m]), acc[r][m]);
              acc[r][m] = __builtin_fmaf(mn, xa.sum(m, j), acc[r][m]);
            }
          });
    }
  }
};

// 5-bit group-affine code (w_hat = s*q + m, q = nibble + 16 * fifth bit): the
// low nibbles in 4-bit code chunks, one 16-byte entry of four 32-bit
// fifth-bit words per (tile, group), and the 4-bit code's scale/min entries.
// Bit 4j + d of a row's fifth-bit word belongs to k = 8d + 2(j mod 4) + j/4
// of the group, so for chunk word d the word shifted left by 4 - d has the
// bits of its first two nibble pairs at 4/20 and 8/24, and shifted right by
// 4 + d those of the last two.
struct CodecQ5 {
  static constexpr int kCodec = W4A16_CODEC_Q5;
  static constexpr int kTileVgprs = 24;
  template <int GPL>
  struct Loads {
    u32x4 sm[GPL];
    u32x4 hb[GPL];
    u32x4 code[kTileRows][GPL];
  };
  template <int GPL>
  __device__ __forceinline__ static void fetch(const WeightPtrs& w, int N, int G, int t, const int (&g0)[GPL],
                                               int lane, Loads<GPL>& L) {
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const Slot s = slot_of(G, g0[j], lane);
      const size_t e = size_t(t) * G + g0[j] + s.base;
      L.sm[j] = __builtin_nontemporal_load(static_cast<const u32x4*>(w.side) + e + s.gl);
      L.hb[j] = __builtin_nontemporal_load(w.aux + e + s.gl);
#pragma unroll
      for (int r = 0; r < kTileRows; ++r)
        L.code[r][j] = __builtin_nontemporal_load(w.codes + (size_t(clamp_row(t, r, N)) * G + g0[j] + s.base) + s.gl);
    }
  }
  template <int M, int GPL, class XA>
  __device__ __forceinline__ static void compute(const Loads<GPL>& L, const XA& xa, float (&acc)[kTileRows][M]) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      float lo[kTileRows][M], hi[kTileRows][M];
#pragma unroll
      for (int r = 0; r < kTileRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) lo[r][m] = hi[r][m] = 0.f;
      tile_walk<M>(
          xa, j,
          [&](int r, int d, const u32x4(&xq)[M]) __attribute__((always_inline)) {
            const uint32_t h = elem(L.hb[j], r);
            nibble_dots<M, true>(elem(L.code[r][j], d), h << (4 - d), h >> (4 + d), xq, lo[r], hi[r], d == 0);
          },
          [&](int r) __attribute__((always_inline)) {
            const f16x2 hm = __builtin_bit_cast(f16x2, elem(L.sm[j], r));
            const float sc = float(hm[0]) * 0x1p20f;
            const float mn = float(hm[1]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
              acc[r][m] = __builtin_fmaf(sc, __builtin_fmaf(lo[r][m], 16.f, hi[r][m]), acc[r][m]);
              acc[r][m] = __builtin_fmaf(mn, xa.sum(m, j), acc[r][m]);
            }
          });
    }
  }
};

// Symmetric 8-bit code (w_hat = s*q, q signed): offset-binary bytes u = q + 128,
// each row's group halves in two runs of 16-byte chunks (all low halves, then
// all high halves, so each load instruction reads 1 KiB contiguously), and
// the symmetric 4-bit code's 8-byte scale entries. In a code word the bytes
// hold k = 4e + (0, 2, 1, 3): AND 0x00FF00FF gives the pair (k, k+1) as
// binary16 subnormals u * 2^-24, the word shifted right by 8 the pair
// (k+2, k+3). The offset is removed with the group's activation sum:
// s * sum u*x - 128 s * sum x.
struct CodecQ8Sym {
  static constexpr int kCodec = W4A16_CODEC_Q8_SYM;
  static constexpr int kTileVgprs = 34;
  template <int GPL>
  struct Loads {
    u32x2 sc[GPL];
    u32x4 code[kTileRows][GPL][2];
  };
  template <int GPL>
  __device__ __forceinline__ static void fetch(const WeightPtrs& w, int N, int G, int t, const int (&g0)[GPL],
                                               int lane, Loads<GPL>& L) {
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const Slot s = slot_of(G, g0[j], lane);
      const u32x2* sp = static_cast<const u32x2*>(w.side) + (size_t(t) * G + g0[j] + s.base);
      L.sc[j] = __builtin_nontemporal_load(sp + s.gl);
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) {
        const u32x4* row = w.codes + size_t(clamp_row(t, r, N)) * (2 * size_t(G)) + g0[j] + s.base;
        L.code[r][j][0] = __builtin_nontemporal_load(row + s.gl);
        L.code[r][j][1] = __builtin_nontemporal_load(row + G + s.gl);
      }
    }
  }
  template <int M, int GPL, class XA>
  __device__ __forceinline__ static void compute(const Loads<GPL>& L, const XA& xa, float (&acc)[kTileRows][M]) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      float lo[kTileRows][M], hi[kTileRows][M];
#pragma unroll
      for (int r = 0; r < kTileRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) lo[r][m] = hi[r][m] = 0.f;
      tile_walk<M>(
          xa, j,
          [&](int r, int d, const u32x4(&xq)[M]) __attribute__((always_inline)) {
            // x chunk d: k = 8d .. 8d+7 = half d/2, code words 2(d%2), 2(d%2)+1
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t w = elem(L.code[r][j][d / 2], 2 * (d % 2) + i);
              const uint32_t p0 = w & 0x00FF00FFu, p1 = (w >> 8) & 0x00FF00FFu;
#pragma unroll
              for (int m = 0; m < M; ++m) {
                if (d == 0 && i == 0) {  // each (row, group) chain starts from 0
                  lo[r][m] = dot2_from_zero(p0, elem(xq[m], 0));
                  hi[r][m] = dot2_from_zero(p1, elem(xq[m], 1));
                } else {
                  lo[r][m] = dot2(p0, elem(xq[m], 2 * i), lo[r][m]);
                  hi[r][m] = dot2(p1, elem(xq[m], 2 * i + 1), hi[r][m]);
                }
              }
            }
          },
          [&](int r) __attribute__((always_inline)) {
            const float s = half_of(L.sc[j], r);
            const float sc = s * 0x1p24f;
            const float mn = -128.f * s;  // exact
#pragma unroll
            for (int m = 0; m < M; ++m) {
              acc[r][m] = __builtin_fmaf(sc, lo[r][m] + hi[r][m], acc[r][m]);
              acc[r][m] = __builtin_fmaf(mn, xa.sum(m, j), acc[r][m]);
            }
          });
    }
  }
};

// Palettised 4-bit code (w_hat = lut[n][q], a 16-entry binary16 palette per
// row): code chunks holding the group's canonical bytes (byte i of word d =
// k = 8d + 2i in the low nibble, k + 1 in the high nibble), and per tile a
// 128-byte entry with the palettes entry by entry (entry c of row r at byte
// 8c + 2r). A code byte b indexes a pair of weights, so each wave expands the
// tile's four palettes into a table of 256 binary16 pairs per row,
// (lut[r][b & 15], lut[r][b >> 4]), in its own 4 KiB of LDS: lane l builds
// the four consecutive entries 4l .. 4l + 3 of every row (low nibbles
// 4(l & 3) .. +3, high nibble l >> 2) from 40 bytes of the palette tile. Each
// code byte then costs one address operation and one LDS read, and the pair
// it returns lines up with the activation pair (x_k, x_k+1) of the same word,
// so it goes straight into v_dot2.
struct CodecPal4 {
  static constexpr int kCodec = W4A16_CODEC_PAL4;
  static constexpr int kTileVgprs = 26;
  static constexpr int kLdsBytesPerWave = kTileRows * 256 * 4;
  template <int GPL>
  struct Loads {
    u32x4 lo[2];  // palette entries 4(l & 3) .. 4(l & 3) + 3 of the four rows
    u32x2 hi;     // palette entry l >> 2 of the four rows
    u32x4 code[kTileRows][GPL];
  };
  template <int GPL>
  __device__ __forceinline__ static void fetch(const WeightPtrs& w, int N, int G, int t, const int (&g0)[GPL],
                                               int lane, Loads<GPL>& L) {
    const uint8_t* pt = static_cast<const uint8_t*>(w.side) + size_t(t) * 128;
    const u32x4* lp = reinterpret_cast<const u32x4*>(pt + 32 * (lane & 3));
    L.lo[0] = lp[0];
    L.lo[1] = lp[1];
    L.hi = *reinterpret_cast<const u32x2*>(pt + 8 * (lane >> 2));
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const Slot s = slot_of(G, g0[j], lane);
#pragma unroll
      for (int r = 0; r < kTileRows; ++r)
        L.code[r][j] = __builtin_nontemporal_load(w.codes + (size_t(clamp_row(t, r, N)) * G + g0[j] + s.base) + s.gl);
    }
  }
  // this wave's table: 256 words per row
  __device__ __forceinline__ static uint32_t* table() {
    extern __shared__ __align__(16) uint32_t pal4_tables[];
    return pal4_tables + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * (kLdsBytesPerWave / 4);
  }
  template <int M, int GPL, class XA>
  __device__ __forceinline__ static void compute(const Loads<GPL>& L, const XA& xa, float (&acc)[kTileRows][M]) {
    uint32_t* tab = table();
    const int lane = threadIdx.x & 63;
    {
      // entry 4l + i of row r: (binary16 of low nibble 4(l & 3) + i, of high
      // nibble l >> 2); rows 0 and 1 share a word of each palette entry, as do
      // rows 2 and 3
      constexpr uint32_t kLow = 0x05040100u, kHigh = 0x07060302u;
      const uint32_t hw[2] = {L.hi.x, L.hi.y};
      const uint32_t lw[2][4] = {{L.lo[0].x, L.lo[0].z, L.lo[1].x, L.lo[1].z},
                                 {L.lo[0].y, L.lo[0].w, L.lo[1].y, L.lo[1].w}};
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) {
        const uint32_t sel = (r & 1) ? kHigh : kLow;
        u32x4 e;
        e.x = __builtin_amdgcn_perm(hw[r >> 1], lw[r >> 1][0], sel);
        e.y = __builtin_amdgcn_perm(hw[r >> 1], lw[r >> 1][1], sel);
        e.z = __builtin_amdgcn_perm(hw[r >> 1], lw[r >> 1][2], sel);
        e.w = __builtin_amdgcn_perm(hw[r >> 1], lw[r >> 1][3], sel);
        *reinterpret_cast<u32x4*>(tab + r * 256 + 4 * lane) = e;
      }
    }
    wave_lds_sync();  // the lookups read entries other lanes wrote
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int r = 0; r < kTileRows; ++r) {
          const uint32_t w = elem(L.code[r][j], d);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t pair = tab[r * 256 + ((w >> (8 * i)) & 0xFFu)];  // (w_k, w_k+1), k = 8d + 2i
#pragma unroll
            for (int m = 0; m < M; ++m)
              acc[r][m] = (j == 0 && d == 0 && i == 0) ? dot2_from_zero(pair, elem(xa.x(m, j, d), i))
                                                       : dot2(pair, elem(xa.x(m, j, d), i), acc[r][m]);
          }
        }
      }
    }
    wave_lds_sync();  // the next tile's table overwrites this one
  }
};

// Waves per workgroup an instantiation may use: its VGPR estimate (x slice,
// tile loads in flight, accumulators) must fit the 512-entry register file
// shared by the waves on one SIMD.
template <class C>
__host__ __device__ constexpr int max_waves_of(int M, int GPL) {
  return (16 * M * GPL + (double_buffered(M, kBlock) ? 2 : 1) * C::kTileVgprs * GPL + 6 * M + 30) <= 128 ? 16 : 8;
}

// ---------------------------------------------------------------------------
// The kernel body
// ---------------------------------------------------------------------------

// nwaves is the workgroup's wave count, passed by the host: the device-side
// workgroup size (blockDim.x) is a vector load from the dispatch packet, and
// every wave would wait for it, a full memory latency, before it could issue
// its activation loads. For the same reason the launch's workgroup count
// comes in the high 16 bits of tpb_grid (tiles per workgroup in the low 16):
// gridDim.x is a load from the kernel argument segment's implicit part,
// while every explicit argument arrives preloaded in scalar registers (the
// library is built with kernel-argument preloading; at most 64 bytes of
// explicit arguments preload, and these kernels use 56 or 64).
//
// The packed blob's header sits just before its code region (wp.codes). Its
// first 16 bytes (one scalar load at the start) are compared where results
// are stored: a blob whose header does not name this codec, N and K (a stale
// layout, another matrix, another codec) makes every workgroup skip its y
// stores, and workgroup 0 counts the launch in *mismatch, a word of the
// kernel's own module. The weight loads never wait for the check, the header
// words live in scalar registers (vector registers set the occupancy here),
// and the kernel arguments are those of a kernel without the check.
template <class C, int M, int GPL, int MODE>
__device__ __forceinline__ void gemv_body(const u32x4* __restrict__ x, const WeightPtrs& wp, float* __restrict__ y,
                                          int N, int G, int T, int nchunks, int tpb_grid, int nwaves,
                                          unsigned* __restrict__ mismatch) {
  const int lane = threadIdx.x & 63;
  // wave-uniform values kept in scalar registers, so every load address is a
  // scalar base plus the one per-lane offset `lane`
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk_groups = nwaves * 64 * GPL;  // groups covered by one pass over K
  const int tpb = tpb_grid & 0xFFFF, grid = tpb_grid >> 16;
  const int nblocks = (T + tpb - 1) / tpb;
  if (int(blockIdx.x) >= nblocks) return;
  // Every kernel argument is in registers before the header's scalar load
  // goes out: scalar loads complete out of order, so the wait for an
  // argument loaded after it would wait for the header as well.
  asm volatile("" ::"s"(x), "s"(wp.codes), "s"(wp.aux), "s"(wp.side), "s"(y), "s"(N), "s"(G), "s"(T), "s"(nchunks),
               "s"(tpb_grid), "s"(nwaves));
  const BlobHead head = read_head(reinterpret_cast<const uint8_t*>(wp.codes) - W4A16_BLOB_HEADER_BYTES);
  auto head_ok = [&]() { return head_matches(head, C::kCodec, N, G * kGroup); };
  // after the last store: one count per launch whose header did not match
  auto count_mismatch = [&]() {
    if (blockIdx.x == 0 && threadIdx.x == 0 && !head_ok())
      __hip_atomic_fetch_add(mismatch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  auto bases = [&](int c, int (&g0)[GPL]) {
#pragma unroll
    for (int j = 0; j < GPL; ++j) g0[j] = c * chunk_groups + (wave * GPL + j) * 64;
  };

  u32x4 xv[M][GPL][4];
  float xs[M][GPL];
  auto fetch_x = [&](int c) {
    int g0[GPL];
    bases(c, g0);
    load_x<M, GPL>(x, G, g0, lane, xv, xs);
  };

  // per-wave partials of one block of tiles: [tile][row][m][wave]
  __shared__ float part[MODE == kDirect ? 1 : kTilesPerBlock][kTileRows][M][MODE == kDirect ? 1 : kMaxWaves];

  // combine the waves' partials of block b (all passes done) and store
  auto reduce_block = [&](int b) {
    __syncthreads();
    const int ntiles = min(tpb, T - b * tpb);
    for (int i = threadIdx.x; i < ntiles * kTileRows * M; i += 64 * nwaves) {
      const int ti = i / (kTileRows * M);
      const int r = (i / M) % kTileRows;
      const int m = i % M;
      const int n = (b * tpb + ti) * kTileRows + r;
      if (n < N && head_ok()) {
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += part[ti][r][m][w];
        y[size_t(m) * N + n] = s;
      }
    }
    __syncthreads();
  };

  using Loads = typename C::template Loads<GPL>;

  if constexpr (MODE == kMulti) {
    // passes over K outermost within a block: x of pass c is fetched once at
    // the top of the pass and stays in registers for the block's tiles. With
    // one group per lane and the 256-register budget of at most eight waves
    // (M >= 3), the next tile's loads are issued before the current tile is
    // computed, as in the single-pass loop below; the 128-register budget of
    // wider workgroups has no room for the second buffer.
    constexpr bool kPrefetch = GPL == 1 && max_waves_of<C>(M, GPL) <= 8;
    for (int b = blockIdx.x; b < nblocks; b += grid) {
      const int ntiles = min(tpb, T - b * tpb);
      for (int c = 0; c < nchunks; ++c) {
        int g0[GPL];
        bases(c, g0);
        auto fetch_tb = [&](int tb, Loads& L) { C::template fetch<GPL>(wp, N, G, b * tpb + tb, g0, lane, L); };
        auto work = [&](const Loads& L, int tb) {
          float acc[kTileRows][M], v[M];
          C::template compute<M, GPL>(L, RegX<M, GPL>{xv, xs}, acc);
          tile_sums<M>(acc, v);
          if ((lane & 15) == 0) {  // the first lane of each 16-lane row: output row lane / 16
            const int r = lane >> 4;
#pragma unroll
            for (int m = 0; m < M; ++m) part[tb][r][m][wave] = (c == 0 ? 0.f : part[tb][r][m][wave]) + v[m];
          }
        };
        Loads la, lb;
        fetch_tb(0, la);
        fetch_x(c);  // after the pass's first tile loads, so both latencies overlap
        int tb = 0;
        if constexpr (!kPrefetch) {
          work(la, 0);
          for (tb = 1; tb < ntiles; ++tb) {
            fetch_tb(tb, la);
            work(la, tb);
          }
          continue;
        }
        while (tb + 2 < ntiles) {
          fetch_tb(tb + 1, lb);
          __builtin_amdgcn_sched_barrier(0);
          work(la, tb);
          fetch_tb(tb + 2, la);
          __builtin_amdgcn_sched_barrier(0);
          work(lb, tb + 1);
          tb += 2;
        }
        if (ntiles - tb == 2) {
          fetch_tb(tb + 1, lb);
          __builtin_amdgcn_sched_barrier(0);
          work(la, tb);
          work(lb, tb + 1);
        } else {
          work(la, tb);
        }
      }
      reduce_block(b);
    }
    count_mismatch();
    return;
  } else {
    // Items e = 0 .. n_items-1 of this workgroup: tile tb = e % tpb of its
    // (e / tpb)-th block. The item count is known up front and the loop's
    // only exit is its condition, so every fetch inside the loop is
    // unconditional (a fetch that might not happen would make the compiler
    // merge buffer contents with register moves that wait for the loads in
    // flight); tiles past T (in the matrix's last block only) fetch a clamped
    // tile and are skipped. A scheduling barrier after each fetch keeps the
    // next tile's loads ahead of the current tile's compute.
    const int my_blocks = (nblocks - int(blockIdx.x) + grid - 1) / grid;
    const int n_items = my_blocks * tpb;
    int g0[GPL];
    bases(0, g0);
    auto tile_of = [&](int e) { return (int(blockIdx.x) + (e / tpb) * grid) * tpb + e % tpb; };
    auto fetch = [&](int e, Loads& L) {
      const int t = tile_of(e);
      C::template fetch<GPL>(wp, N, G, t < T ? t : T - 1, g0, lane, L);
    };
    auto finish = [&](const Loads& L, int e) {
      const int t = tile_of(e);
      if (t < T) {
        float acc[kTileRows][M], v[M];
        C::template compute<M, GPL>(L, RegX<M, GPL>{xv, xs}, acc);
        tile_sums<M>(acc, v);
        if constexpr (MODE == kDirect) {
          if (head_ok()) store_tile<M>(v, y, N, t, lane);
        } else if ((lane & 15) == 0) {  // the first lane of each 16-lane row: output row lane / 16
          const int tb = e % tpb;
          const int r = lane >> 4;
#pragma unroll
          for (int m = 0; m < M; ++m) part[tb][r][m][wave] = v[m];
        }
      }
      if constexpr (MODE == kBlock) {
        if (e % tpb == tpb - 1) reduce_block(int(blockIdx.x) + (e / tpb) * grid);
      }
    };

    Loads la, lb;
    fetch(0, la);
    fetch_x(0);  // after the first tile's loads, so both latencies overlap
    int e = 0;
    if constexpr (double_buffered(M, MODE)) {
      while (e + 2 < n_items) {
        fetch(e + 1, lb);
        __builtin_amdgcn_sched_barrier(0);
        finish(la, e);
        fetch(e + 2, la);
        __builtin_amdgcn_sched_barrier(0);
        finish(lb, e + 1);
        e += 2;
      }
      if (n_items - e == 2) {
        fetch(e + 1, lb);
        __builtin_amdgcn_sched_barrier(0);
        finish(la, e);
        finish(lb, e + 1);
      } else {
        finish(la, e);
      }
    } else {
      finish(la, 0);
      for (e = 1; e < n_items; ++e) {
        fetch(e, la);
        finish(la, e);
      }
    }
    count_mismatch();
  }
}

}  // namespace w4a16_dev

// ---------------------------------------------------------------------------
// Host side: launch-shape choice
// ---------------------------------------------------------------------------

namespace w4a16_host {

constexpr int kGplOptions[] = {1, 2, 4};
constexpr int kNumGpl = 3;

// the x slice of one lane stays within 32 VGPRs (one group per lane always allowed)
constexpr bool gpl_allowed(int M, int gpl) { return 16 * M * gpl <= 32 || gpl == 1; }

inline int mode_of(int waves, int nchunks) {
  return nchunks > 1 ? w4a16_dev::kMulti : waves > 1 ? w4a16_dev::kBlock : w4a16_dev::kDirect;
}

struct LaunchShape {
  int gi;       // index into kGplOptions
  int waves;    // waves per workgroup
  int nchunks;  // passes over K
};

template <class C>
LaunchShape shape_for_gpl(int M, int G, int gi) {
  const int gpl = kGplOptions[gi];
  const int wmax = w4a16_dev::max_waves_of<C>(M, gpl);
  const int nchunks = (G + wmax * 64 * gpl - 1) / (wmax * 64 * gpl);
  const int waves = (G + nchunks * 64 * gpl - 1) / (nchunks * 64 * gpl);
  return LaunchShape{gi, waves, nchunks};
}

// Fewest passes over K; then avoid leaving more than a quarter of the lanes
// idle; then, at M = 1, one group per lane (a tile's K split over more waves:
// each wave loads less of x and more waves share the streaming; measured
// faster on every decode-step shape); then the fewest waves per workgroup;
// then the fewest idle lanes.
template <class C>
LaunchShape choose_shape(int M, int G) {
  LaunchShape best{-1, 0, 0};
  long best_key[5] = {0, 0, 0, 0, 0};
  for (int gi = kNumGpl - 1; gi >= 0; --gi) {
    if (!gpl_allowed(M, kGplOptions[gi])) continue;
    const LaunchShape s = shape_for_gpl<C>(M, G, gi);
    const long slots = long(s.nchunks) * s.waves * 64 * kGplOptions[gi];
    const long idle = slots - G;
    const long key[5] = {s.nchunks, 4 * idle > slots ? 1 : 0, M == 1 ? kGplOptions[gi] : 0, s.waves, idle};
    bool better = best.gi < 0;
    for (int i = 0; i < 5 && !better; ++i) {
      if (key[i] < best_key[i]) better = true;
      if (key[i] > best_key[i]) break;
    }
    if (better) {
      best = s;
      for (int i = 0; i < 5; ++i) best_key[i] = key[i];
    }
  }
  return best;
}

// Resident workgroups per CU that a launch uses. From four activation rows
// on, a wave's x slice (M * 64 bytes per lane, 16 KiB at M = 4) is as large
// as several tiles of weights, and each workgroup loads it once per block:
// at most two waves per SIMD are kept resident, so each workgroup walks more
// tiles per x slice (the 8B gate_up at M = 4: 4 workgroups of 7 tiles per
// CU instead of 8 of 4). At M = 8 the register file already allows no more.
inline int resident_workgroups(int M, int waves, int occ) {
  if (M < 4) return occ;
  const int cap = waves >= 8 ? 1 : 8 / waves;
  return occ < cap ? occ : cap;
}

// Tiles per block and grid of a launch: every workgroup resident at once,
// each walking an equal share of the tiles. A workgroup reads its x slices
// once per block, so wide workgroups (long K split over four or more waves, a
// large x) take enough tiles per block for about one workgroup per CU;
// narrower ones fill the resident slots first. That choice stands if it gives
// the busiest CU (workgroup w counted on CU w % cus, the first workgroups
// walking one block more when blocks outnumber them) as few tiles as any
// tiles-per-block count can and, from four activation rows on, fits in one
// round of resident workgroups when some such count does. Otherwise the
// count is changed to a qualifying one: for narrow workgroups the smallest
// above the first choice (7168 tiles over 2048 slots: 4 per block, 28 tiles
// on every CU, not 3 per block and 27 or 30 per CU), for wide ones the
// largest (2560 tiles of 4-wave workgroups: 5 per block on 512 workgroups,
// 10 tiles per CU, not 8 per block on 320 workgroups and 16 tiles on a fifth
// of the CUs).
inline void grid_of(int T, int M, int waves, bool direct, int cus, int occ, int& tpb, int& grid) {
  const int max_grid = cus * occ;
  auto cdiv = [](int a, int b) { return (a + b - 1) / b; };
  const bool wide = waves >= 4;
  tpb = direct ? 1 : wide ? T / cus : T / max_grid;
  tpb = tpb < 1 ? 1 : tpb > w4a16_dev::kTilesPerBlock ? w4a16_dev::kTilesPerBlock : tpb;
  if (!direct) {
    auto busiest_cu = [&](int b) {
      const int blocks = cdiv(T, b), g = blocks < max_grid ? blocks : max_grid;
      return b * (cdiv(g, cus) * (blocks / g) + cdiv(blocks % g, cus));
    };
    // a count qualifies if it reaches the fewest tiles on the busiest CU and,
    // from four activation rows on (a large x slice per wave), also fits in
    // one round of resident workgroups if any such count does: one round
    // loads each workgroup's x slices once
    auto one_round = [&](int b) { return cdiv(T, b) <= max_grid; };
    int best = busiest_cu(tpb);
    for (int b = 1; b <= w4a16_dev::kTilesPerBlock; ++b) best = busiest_cu(b) < best ? busiest_cu(b) : best;
    bool round_ok = false;
    for (int b = 1; b <= w4a16_dev::kTilesPerBlock && M >= 4; ++b) round_ok = round_ok || (busiest_cu(b) == best && one_round(b));
    auto qualifies = [&](int b) { return busiest_cu(b) == best && (!round_ok || one_round(b)); };
    if (!qualifies(tpb)) {
      const int first = tpb;
      tpb = 0;
      for (int b = 1; b <= w4a16_dev::kTilesPerBlock; ++b) {
        if (!qualifies(b)) continue;
        if (wide ? b > tpb : (b > first && tpb == 0)) tpb = b;
      }
      if (tpb == 0) {  // narrow, and every qualifying count lies below the first choice: the largest of them
        for (int b = 1; b <= w4a16_dev::kTilesPerBlock; ++b)
          if (qualifies(b)) tpb = b;
      }
    }
  }
  const int blocks = cdiv(T, tpb);
  grid = blocks < max_grid ? blocks : max_grid;
}

// The kernels' tpb_grid argument: tiles per workgroup in the low 16 bits, the
// launch's workgroup count in the high 16 (0 if either does not fit; the
// caller then refuses the launch).
inline int tpb_grid_arg(int tpb, int grid) {
  return tpb >= 1 && tpb < (1 << 16) && grid >= 1 && grid < (1 << 15) ? tpb | (grid << 16) : 0;
}

}  // namespace w4a16_host
