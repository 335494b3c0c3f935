// Device building blocks shared by the single-GEMV kernel and the chained
// (whole decode step) kernel: the tile loads, the activation slice and the
// per-tile dot products. Internal header of libw4a16.
//
// Notation: G = K/32 groups per row; a tile is 4 consecutive rows; a lane
// owns GPL groups (group bases g0[j] are wave-uniform, the lane adds its
// index); the packed layout is the one documented in include/w4a16.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16.h"

namespace w4a16_dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 32;
constexpr int kTileRows = 4;
constexpr int kMaxWaves = 16;
constexpr int kMaxM = 8;
constexpr int kTilesPerBlock = 8;        // most tiles between two LDS reductions
constexpr uint32_t kOnes = 0x3C003C00u;  // binary16 pair (1.0, 1.0)

// Element i of a 4 x u32 vector. Written as an explicit select rather than
// v[i]: with ROCm 7.2's clang, v[i] on an unrolled index inside the tile loop
// was folded to v[0] (the scale/min load shrank to one dword and every row of
// a tile used row 0's scale), so vector elements are only ever read this way.
__device__ __forceinline__ uint32_t elem(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// a.b + 0 in one VOP3P instruction with the inline constant 0 as its
// accumulator. Written with fdot2(a, b, 0), the compiler picks the
// two-address v_dot2c form and zeroes its destination with a v_mov first: one
// extra VALU operation per partial sum started, 2M per (row, group).
__device__ __forceinline__ float dot2_from_zero(uint32_t a, uint32_t b) {
  float d;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane ends with the same bits.
// Within rows of 16 lanes: DPP butterflies. Across rows: gfx950's
// v_permlane16_swap / v_permlane32_swap, which exchange whole rows between
// two VGPRs inside the VALU (no LDS round trip as with ds_bpermute): after
// swap(v, v) one register holds rows (0,0,2,2) and the other rows (1,1,3,3),
// so their sum is the pairwise row sum in every lane, in the same order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  const unsigned b = __builtin_bit_cast(unsigned, v);
  const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = __builtin_bit_cast(float, unsigned(p[0])) + __builtin_bit_cast(float, unsigned(p[1]));
  const unsigned c = __builtin_bit_cast(unsigned, v);
  const auto q = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __builtin_bit_cast(float, unsigned(q[0])) + __builtin_bit_cast(float, unsigned(q[1]));
}

// A wave reads LDS words that other lanes of the same wave wrote: its LDS
// operations complete in order once lgkmcnt drains, and the empty asm keeps
// the compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  asm volatile("" ::: "memory");
}

// Maximum over the 64 lanes of a wave, by the same exchanges as wave_sum;
// every lane ends with the same value. The exchanges compare order keys: the
// bits of a float, with the magnitude bits flipped when the sign is set,
// order as signed integers the way the floats do (NaN aside), and an integer
// max needs no NaN quieting, so each DPP exchange and its max issue as one
// v_max_i32 with a DPP operand (fmaxf costs a move, a canonicalising max and
// the max per exchange).
__device__ __forceinline__ int order_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float from_order_key(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF)); }
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float wave_max(float v) {
  int k = order_key(v);
  k = max(k, dpp_i<0xB1>(k));   // quad_perm [1,0,3,2]
  k = max(k, dpp_i<0x4E>(k));   // quad_perm [2,3,0,1]
  k = max(k, dpp_i<0x141>(k));  // row_half_mirror
  k = max(k, dpp_i<0x140>(k));  // row_mirror
  const auto p = __builtin_amdgcn_permlane16_swap(unsigned(k), unsigned(k), false, false);
  k = max(int(p[0]), int(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(unsigned(k), unsigned(k), false, false);
  return from_order_key(max(int(q[0]), int(q[1])));
}

// Loads of one 4-row tile for this lane: GPL scale/min entries, 4*GPL chunks.
template <int GPL>
struct TileLoads {
  u32x4 sm[GPL];
  u32x4 code[kTileRows][GPL];
};

// Issue the 16-byte non-temporal loads of tile t (rows 4t..4t+3) for the
// groups g0[j] + lane. Every load is unconditional: a lane past G reads group
// G-1 instead (its activations are zero, so it adds exactly 0) and a row past
// N reads row N-1 (its results are never stored). A conditional load would
// make the compiler merge "zero or loaded" with a register move that waits
// for the load, which serialises the prefetch of the next tile.
template <int GPL>
__device__ __forceinline__ void fetch_tile(const u32x4* __restrict__ codes, const u32x4* __restrict__ sm, int N,
                                           int G, int t, const int (&g0)[GPL], int lane, TileLoads<GPL>& L) {
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int last = G - 1 - g0[j];  // wave-uniform; < 0 when the whole slot is past G
    const int gl = lane < last ? lane : (last > 0 ? last : 0);
    const int base = last < 0 ? G - 1 - g0[j] : 0;  // pulls an all-idle slot back to group G-1
    const u32x4* sp = sm + (size_t(t) * G + g0[j] + base);
    L.sm[j] = __builtin_nontemporal_load(sp + gl);
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const int n = t * kTileRows + r < N ? t * kTileRows + r : N - 1;
      const u32x4* cp = codes + (size_t(n) * G + g0[j] + base);
      L.code[r][j] = __builtin_nontemporal_load(cp + gl);
    }
  }
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3:
// 32-bit data format, the setting for untyped raw access). A load whose
// offset falls outside the range returns zeros without touching memory.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kLoadNT = 2;  // buffer-load cache policy: non-temporal stream

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRawBufferWord3);
}

// The first 16 bytes of a packed blob's header (layout in include/w4a16.h):
// magic, layout version | codec << 16, N, K.
struct BlobHead {
  uint32_t w[4];
};
__host__ __device__ constexpr uint32_t head_version_codec(int codec) {
  return uint32_t(W4A16_LAYOUT_VERSION) | (uint32_t(codec) << 16);
}

// The header read through the constant address space (a blob is never
// written during a launch): one scalar load, which the caller issues at the
// start of the kernel.
__device__ __forceinline__ BlobHead read_head(const void* blob) {
  typedef const __attribute__((address_space(4))) uint32_t* Words;
  const Words p = (Words)(reinterpret_cast<uintptr_t>(blob));
  return BlobHead{{p[0], p[1], p[2], p[3]}};
}

// Does the header name this codec, N and K? Called where a result is stored.
// The empty asm statement marks copies of the header words as changed there,
// so the compiler cannot hoist the comparison, and with it the wait for the
// scalar load, to the entry of the loop around the store: there the wait
// would hold back the next tile's loads by a full memory latency, while at
// the store it is long over. (Scalar loads share their counter with LDS
// traffic, so the first LDS wait after the load would take it anyway.)
__device__ __forceinline__ bool head_matches(const BlobHead& h, int codec, int N, int K) {
  uint32_t m = h.w[0], v = h.w[1], n = h.w[2], k = h.w[3];
  asm volatile("" : "+s"(m), "+s"(v), "+s"(n), "+s"(k));
  return m == W4A16_BLOB_MAGIC && v == head_version_codec(codec) && n == uint32_t(N) && k == uint32_t(K);
}

// fetch_tile with buffer loads and no per-lane address arithmetic: every
// (row, group slot) gets its own descriptor, based at the slot's first group
// and sized to the groups left in the row, and lane l reads at byte offset
// voff = 16 * l (computed once by the caller). Lanes past the end of the row
// fall outside the descriptor and read zeros without touching memory (their
// activations are zero too, so they add exactly 0). `valid` = 0 sizes every
// descriptor to 0 (a team with no tile, or a fetch past the end: no traffic,
// and no branch around the fetch); it must be -1 otherwise, formed by integer
// arithmetic on scalar values (a select of a comparison would be built in a
// vector register). All address arithmetic is scalar: a vector temporary
// here can be placed by the register allocator in a buffer whose previous
// load the compiler cannot prove complete, and it then waits for it. A row
// past N reads row N-1 (its results are never stored).
template <int GPL>
__device__ __forceinline__ void fetch_tile_rows(const u32x4* __restrict__ codes, const u32x4* __restrict__ sm,
                                                int N, int G, int t, const int (&g0)[GPL], int voff, int valid,
                                                TileLoads<GPL>& L) {
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int left = G - g0[j];  // groups of the slot inside the row (may be <= 0)
    const int bytes = (left > 0 ? left * 16 : 0) & valid;
    L.sm[j] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(sm + (size_t(t) * G + g0[j]), bytes), voff, 0,
                                                    kLoadNT);
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const int n = t * kTileRows + r < N ? t * kTileRows + r : N - 1;
      L.code[r][j] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(codes + (size_t(n) * G + g0[j]), bytes),
                                                           voff, 0, kLoadNT);
    }
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads (a __syncthreads would also drain the
// prefetched tile).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
}

// Sum of the 32 binary16 activations of one group held as four 16-byte
// chunks, in a fixed tree: each chunk's 8 values in one v_dot2 chain from 0,
// then (c0 + c1) + (c2 + c3). Every path that needs a group sum forms it this
// way (a wave holding the four chunks in four lanes adds them with two DPP
// steps in the same order), so results do not depend on who formed it.
__device__ __forceinline__ float chunk_sum(const u32x4& q) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = dot2(elem(q, e), kOnes, s);
  return s;
}
__device__ __forceinline__ float group_sum(const u32x4 (&q)[4]) {
  return (chunk_sum(q[0]) + chunk_sum(q[1])) + (chunk_sum(q[2]) + chunk_sum(q[3]));
}

// This lane's slice x[m][32g .. 32g+31] of every activation row for the
// groups g = g0[j] + lane, loaded straight into the registers that keep it,
// plus the per-group sums used by the min term.
template <int M, int GPL>
__device__ __forceinline__ void load_x(const u32x4* __restrict__ x, int G, const int (&g0)[GPL], int lane,
                                       u32x4 (&xv)[M][GPL][4], float (&xs)[M][GPL]) {
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int g = g0[j] + lane;
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[m][j][q] = u32x4{0, 0, 0, 0};
      if (g < G) {
        const u32x4* p = x + (size_t(m) * G + g) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[m][j][q] = p[q];
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int j = 0; j < GPL; ++j) xs[m][j] = group_sum(xv[m][j]);
}

// Activations held in registers (the single-GEMV kernel): chunk d of the
// lane's group j of row m, and that group's sum.
template <int M, int GPL>
struct RegX {
  static constexpr bool kRowOuter = true;  // chunks are free to re-read: walk a tile row by row
  const u32x4 (&xv)[M][GPL][4];
  const float (&xs)[M][GPL];
  __device__ __forceinline__ u32x4 x(int m, int j, int d) const { return xv[m][j][d]; }
  __device__ __forceinline__ float sum(int m, int j) const { return xs[m][j]; }
};

// Visits (row r, chunk d) of group j of a tile: row by row when the
// accessor's chunks are free to re-read (activations in registers: one row's
// partial sums are live at a time), chunk by chunk otherwise (activations in
// LDS: each chunk is read once for the four rows). step(r, d, xq) gets chunk
// d of every activation row; fold(r) runs after row r's last chunk. Each
// (row, activation row) sees the same sequence of operations either way.
template <int M, class XA, class Step, class Fold>
__device__ __forceinline__ void tile_walk(const XA& xa, int j, Step&& step, Fold&& fold) {
  if constexpr (XA::kRowOuter) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4 xq[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xq[m] = xa.x(m, j, d);
        step(r, d, xq);
      }
      fold(r);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 xq[M];
#pragma unroll
      for (int m = 0; m < M; ++m) xq[m] = xa.x(m, j, d);
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) step(r, d, xq);
    }
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) fold(r);
  }
}

// One lane's partial row sums of one tile over its groups (tile_sums adds
// them over the wave): acc[r][m] = sum over the lane's groups g of
//   scale[4t+r][g] * sum_k q*x[m][k] + min[4t+r][g] * sum_k x[m][k].
// sum_k q*x is formed with v_dot2c_f32_f16 on binary16 subnormal pairs: the
// packed word AND 0x000F000F is a pair of halfs whose bit patterns are the
// codes (values q * 2^-24), AND 0x00F000F0 gives q * 2^-20. Both are exact,
// so are their products with x in fp32, and no offset is cancelled later.
// The activations come from an accessor (registers or LDS) chunk by chunk,
// as they are used; the arithmetic per (row, activation row) is the same
// sequence whatever the accessor.
template <int M, int GPL, class XA>
__device__ __forceinline__ void compute_tile(const TileLoads<GPL>& L, const XA& xa, float (&acc)[kTileRows][M]) {
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
          const uint32_t w = elem(L.code[r][j], d);
          const uint32_t w8 = w >> 8;
          const uint32_t pa = w & 0x000F000Fu;   // k = 8d+0, 8d+1  -> q * 2^-24
          const uint32_t pb = w & 0x00F000F0u;   // k = 8d+2, 8d+3  -> q * 2^-20
          const uint32_t pc = w8 & 0x000F000Fu;  // k = 8d+4, 8d+5  -> q * 2^-24
          const uint32_t pd = w8 & 0x00F000F0u;  // k = 8d+6, 8d+7  -> q * 2^-20
#pragma unroll
          for (int m = 0; m < M; ++m) {
            if (d == 0) {  // each (row, group) chain starts from 0
              lo[r][m] = dot2_from_zero(pa, elem(xq[m], 0));
              hi[r][m] = dot2_from_zero(pb, elem(xq[m], 1));
            } else {
              lo[r][m] = dot2(pa, elem(xq[m], 0), lo[r][m]);
              hi[r][m] = dot2(pb, elem(xq[m], 1), hi[r][m]);
            }
            lo[r][m] = dot2(pc, elem(xq[m], 2), lo[r][m]);
            hi[r][m] = dot2(pd, elem(xq[m], 3), hi[r][m]);
          }
        },
        [&](int r) __attribute__((always_inline)) {
          const f16x2 h = __builtin_bit_cast(f16x2, elem(L.sm[j], r));
          const float sc = float(h[0]) * 0x1p20f;
          const float mn = float(h[1]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            acc[r][m] = __builtin_fmaf(sc, __builtin_fmaf(lo[r][m], 16.f, hi[r][m]), acc[r][m]);
            acc[r][m] = __builtin_fmaf(mn, xa.sum(m, j), acc[r][m]);
          }
        });
  }
}

// Wave sums of a tile's kTileRows x M lane partials, by one transposed
// exchange per activation row m: rows 0 and 2, then rows 1 and 3, are paired
// across the wave halves (v_permlane32_swap: lanes 0-31 end with row 0's
// half sums, lanes 32-63 with row 2's), the two results across odd and even
// 16-lane rows (v_permlane16_swap), which leaves output row r in lanes
// 16r .. 16r + 15, and four DPP butterflies finish each 16-lane row. Every
// lane of row group r ends with the same bits in v[m]: the sum over the 64
// lanes of acc[r][m]. 10 VALU operations per m, against 32 for four
// separate wave sums.
template <int M>
__device__ __forceinline__ void tile_sums(const float (&acc)[kTileRows][M], float (&v)[M]) {
  static_assert(kTileRows == 4, "one output row per 16-lane row");
  auto f = [](unsigned u) { return __builtin_bit_cast(float, u); };
  auto u = [](float x) { return __builtin_bit_cast(unsigned, x); };
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const auto p = __builtin_amdgcn_permlane32_swap(u(acc[0][m]), u(acc[2][m]), false, false);
    const float s02 = f(unsigned(p[0])) + f(unsigned(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(u(acc[1][m]), u(acc[3][m]), false, false);
    const float s13 = f(unsigned(q[0])) + f(unsigned(q[1]));
    const auto h = __builtin_amdgcn_permlane16_swap(u(s02), u(s13), false, false);
    float t = f(unsigned(h[0])) + f(unsigned(h[1]));
    t += dpp<0xB1>(t);   // quad_perm [1,0,3,2]
    t += dpp<0x4E>(t);   // quad_perm [2,3,0,1]
    t += dpp<0x141>(t);  // row_half_mirror
    t += dpp<0x140>(t);  // row_mirror
    v[m] = t;
  }
}

// Store one result. COHERENT stores go through to device-coherent memory
// (a relaxed agent-scope atomic store, "sc1"), so a later reader on any XCD
// sees them after the usual ordering point without any L2 write-back.
template <bool COHERENT>
__device__ __forceinline__ void store_y(float* p, float v) {
  if constexpr (COHERENT)
    __hip_atomic_store(reinterpret_cast<unsigned*>(p), __builtin_bit_cast(unsigned, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// The tile_sums result of activation row m that lane `lane` stores: lane
// 16r + m holds output row r's v[m] (M <= 16; lanes with lane % 16 >= M get
// an unspecified value and store nothing). A tree of selects on the bits of
// the index, whose operands pass through empty asm statements: otherwise the
// compiler turns a select between two array elements into an indexed read of
// a stack array, and that scratch load waits for every global load in flight.
template <int M>
__device__ __forceinline__ float pick_sum(const float (&v)[M], int lane) {
  const int i = lane & 15;
  float t[M];
#pragma unroll
  for (int m = 0; m < M; ++m) t[m] = v[m];
#pragma unroll
  for (int k = 1; k < M; k <<= 1)
#pragma unroll
    for (int j = 0; j + k < M; j += 2 * k) {
      float a = t[j + k], b = t[j];
      asm("" : "+v"(a), "+v"(b));
      t[j] = (i & k) ? a : b;
    }
  return t[0];
}

// A wave that covers all of K for its tile writes the tile's 4*M results
// itself from tile_sums: lane 16r + m stores y[m][4t + r].
template <int M, bool COHERENT = false>
__device__ __forceinline__ void store_tile(const float (&v)[M], float* __restrict__ y, int N, int t, int lane) {
  const float s = pick_sum<M>(v, lane);
  const int n = t * kTileRows + (lane >> 4);
  if ((lane & 15) < M && n < N) store_y<COHERENT>(y + size_t(lane & 15) * N + n, s);
}

}  // namespace w4a16_dev
