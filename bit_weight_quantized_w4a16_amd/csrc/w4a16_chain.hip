// gfx950 kernel and C-ABI entry points of the decode-step chain: a list of
// W4A16 GEMVs executed in order by ONE persistent launch.
//
// Why: a decode step is the same list of matrix-vector products every token
// (the tight decode loop of the core-modules page, section 5.2), and its
// scheduler notes (section 5.3) call for fetching the next product's weights
// while other work runs. On an MI355X a kernel boundary costs about 1.5 us of
// launch gap plus the ramp of the next kernel, about as long as streaming
// 10 MB of weights; a 32-layer 8B step has 128 such boundaries.
//
// How: one workgroup per CU, eight waves with two roles.
//
// * Seven compute waves only stream weights and do arithmetic. Product i's
//   4-row tiles are split evenly over the workgroups; inside a workgroup a
//   unit of work is (tile, K segment of 64*GPL groups), handed to the compute
//   waves round-robin. Each wave keeps RING units' loads in registers and
//   issues the loads of unit e+RING-1 before computing unit e, across product
//   boundaries: weights never depend on earlier results, so HBM keeps
//   streaming while the products' ordering points are reached. A unit's
//   result (4 rows x M partial sums) goes to LDS; a compute wave never
//   stores to global memory and never waits for its own stores, which on
//   gfx9 would also wait for every weight load it has in flight.
//
// * One sync wave does everything that has to wait on memory: it stages each
//   product's activations into LDS (coherent loads, since an earlier product
//   of the same launch may have written them on another XCD), publishes them
//   to the compute waves through an LDS counter, sums the segment partials in
//   a fixed order and writes y with coherent stores, and takes part in the
//   device-wide ordering between products.
//
// Ordering between products: after its y stores have completed, a
// workgroup's sync wave adds 1 to its leaf of a two-level counter tree in the
// caller's workspace; the last arrival at a leaf climbs to the top counter,
// the last arrival at the top raises every leaf's flag to i+1. A sync wave
// stages product i+1's x only after its leaf flag reaches i+1. Every wait is
// bounded: a wait that gives up flags the workspace's error word, releases
// the other workgroups and ends the launch (its results are then invalid),
// so a launch whose workgroups cannot all be resident ends instead of
// hanging. The last workgroup out resets the counters for the next call.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "w4a16.h"
#include "w4a16_device.h"
#include "w4a16_host.h"

using namespace w4a16_dev;

namespace {

constexpr uint32_t kChainMagic = 0x48433457u;  // "W4CH"
constexpr uint32_t kChainVersion = 3;
constexpr unsigned kSpinLimit = 1u << 20;      // global polls before an ordering wait gives up (~1 s)
constexpr unsigned kLdsSpinLimit = 1u << 26;   // LDS polls before a wave gives up (several s)
constexpr int kLeaves = 16;                    // leaf counters of the ordering tree
constexpr int kLineWords = 1024;               // 4 KiB between counters (separate memory pages)
constexpr int kWaves = 8;                      // per workgroup
constexpr int kComputeWaves = kWaves - 1;      // wave kWaves-1 is the sync wave
constexpr int kXLdsBytes = 65536;              // LDS staging of one pass of x
constexpr int kYLdsBytes = 65536;              // LDS partial sums of one block of tiles
constexpr int kLoadCoherent = 16;              // buffer-load cache policy: device-coherent (sc1)

// groups per lane (the x slice stays within 32 VGPRs at M = 1 and 2)
constexpr int chain_gpl(int M) { return M == 1 ? 2 : 1; }
// groups of one K segment (one unit of work covers one segment of one tile)
constexpr int chain_seg_groups(int M) { return 64 * chain_gpl(M); }
// segments of x one LDS pass holds, and the LDS row stride of x in groups
constexpr int chain_pass_segs(int M) { return kXLdsBytes / (64 * M) / chain_seg_groups(M); }
constexpr int chain_x_groups(int M) { return chain_pass_segs(M) * chain_seg_groups(M); }
// units whose loads a compute wave keeps in registers (register budget: two
// waves per SIMD, 256 VGPRs each)
constexpr int chain_ring(int M) { return M == 1 ? 4 : M == 2 ? 8 : M <= 4 ? 6 : M == 5 ? 4 : 3; }

struct ChainHeader {
  uint32_t magic, version;
  int32_t count, M, gpl, ring;
  int32_t pad[10];
};
static_assert(sizeof(ChainHeader) == 64, "plan header is 64 bytes");

struct ChainEntry {
  const u32x4* x;
  const u32x4* codes;
  const u32x4* sm;
  float* y;
  int32_t N, G, T;  // rows, groups per row, 4-row tiles
  int32_t S;        // K segments per tile
  int32_t passes;   // LDS passes of x over the segments
  int32_t TB;       // tiles per block (the LDS partials of one block fit kYLdsBytes)
  int32_t pad[2];
};
static_assert(sizeof(ChainEntry) == 64, "plan entry is 64 bytes");

// The plan never changes during a launch: it is read through the constant
// address space, which the compiler always serves with scalar loads. Through
// a global pointer, the y stores and the ordering operations of the kernel
// would make it assume the plan may have changed and read it with vector
// loads, whose completion shares the in-order counter of the weight loads in
// flight and would drain them at every product boundary.
typedef const __attribute__((address_space(4))) ChainEntry* EntryPtr;

// Workspace words: the tree's top counter, the exit counter and the error
// word share the first page; leaf g's counter and flag sit on page 1 + g.
constexpr int kTopWord = 0, kExitWord = 32, kErrorWord = 64;
constexpr int leaf_word(int g) { return kLineWords * (1 + g); }
constexpr int flag_word(int g) { return kLineWords * (1 + g) + 32; }
static_assert(kLineWords * (1 + kLeaves) * 4 == W4A16_CHAIN_WORKSPACE_BYTES, "workspace layout");

__device__ __forceinline__ unsigned ld_coherent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_coherent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Product p as one workgroup sees it, walked stage by stage: a stage is
// (block b of this workgroup's tiles, LDS pass c over K); its units are
// (tile, segment) pairs, tile-major. All fields are wave-uniform.
struct Walk {
  int p, b, c, s;  // product, block, pass, running stage number
  EntryPtr e;
  int t0, ntile, nb;     // this workgroup's tiles of product p, blocks
  int tb0, nt, sg0, ns;  // the stage's first tile and count, first segment and count
};

__device__ __forceinline__ void walk_product(Walk& w, EntryPtr ents, int p, int nwg, int wg) {
  w.p = p;
  w.e = ents + p;
  const int T = w.e->T, TB = w.e->TB;
  const int q = T / nwg, rem = T - q * nwg;
  w.t0 = wg * q + (wg < rem ? wg : rem);
  w.ntile = q + (wg < rem ? 1 : 0);
  w.nb = w.ntile > 0 ? (w.ntile + TB - 1) / TB : 1;  // a workgroup with no tiles still walks one empty stage
  w.b = 0;
  w.c = 0;
}

template <int M>
__device__ __forceinline__ void walk_stage(Walk& w) {
  constexpr int SP = chain_pass_segs(M);
  const int TB = w.e->TB, S = w.e->S;
  w.tb0 = w.t0 + w.b * TB;
  const int left = w.ntile - w.b * TB;
  w.nt = left < TB ? (left > 0 ? left : 0) : TB;
  w.sg0 = w.c * SP;
  w.ns = S - w.sg0 < SP ? S - w.sg0 : SP;
}

// next stage; false past the last product
template <int M>
__device__ __forceinline__ bool walk_next(Walk& w, EntryPtr ents, int count, int nwg, int wg) {
  ++w.s;
  if (++w.c == w.e->passes) {
    w.c = 0;
    if (++w.b == w.nb) {
      if (w.p + 1 >= count) {
        w.p = count;
        return false;
      }
      walk_product(w, ents, w.p + 1, nwg, wg);
    }
  }
  walk_stage<M>(w);
  return true;
}

// A compute wave's position: a stage, and unit ti * ns + si of it, i.e. tile
// tb0 + ti and segment sg0 + si (wave v takes units v, v + 7, ... of every
// stage). Kept as (ti, si) and moved with scalar adds: an integer division
// here would be emulated in vector registers right next to the weight loads.
struct Cursor {
  Walk w;
  int ti, si;
};

// unit index (ti, si) + n within a stage of ns segments per tile
__device__ __forceinline__ void unit_add(int& ti, int& si, int ns, int n) {
  si += n;
  if (ns == 1) {
    ti += si;
    si = 0;
  } else {
    while (si >= ns) {
      si -= ns;
      ++ti;
    }
  }
}

// move past stages where this wave has no unit
template <int M>
__device__ __forceinline__ void cursor_settle(Cursor& u, EntryPtr ents, int count, int nwg, int wg,
                                              int wave) {
  while (u.w.p < count && u.ti >= u.w.nt) {
    if (!walk_next<M>(u.w, ents, count, nwg, wg)) break;
    u.ti = 0;
    u.si = 0;
    unit_add(u.ti, u.si, u.w.ns, wave);
  }
}

// Activations read from LDS as they are used: chunk d of row m's group at
// pass-local index gl[j], and that group's sum (written by the sync wave).
template <int M, int GPL, int XG>
struct LdsX {
  static constexpr bool kRowOuter = false;  // each chunk is an LDS read: walk a tile chunk by chunk
  const u32x4* xl;
  const float* xsl;
  int gl[GPL];
  __device__ __forceinline__ u32x4 x(int m, int j, int d) const { return xl[(m * XG + gl[j]) * 4 + d]; }
  __device__ __forceinline__ float sum(int m, int j) const { return xsl[m * XG + gl[j]]; }
};

// step(k) for k = K .. RING-1 with k a compile-time constant (the ring's
// buffer indices must be constants; a pragma cannot unroll a loop this size
// with an exit in it); false as soon as one step ends the walk
template <int K, int RING, class Step>
__device__ __forceinline__ bool ring_steps(Step& step) {
  if constexpr (K == RING) {
    return true;
  } else {
    if (!step(std::integral_constant<int, K>{})) return false;
    return ring_steps<K + 1, RING>(step);
  }
}

template <int M, int GPL, int RING>
__global__ void __launch_bounds__(64 * kWaves)
chain_kernel(const ChainHeader* __restrict__ hdr, unsigned* __restrict__ ws, int count) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  if (hdr->magic != kChainMagic || hdr->version != kChainVersion || hdr->count != count || hdr->M != M ||
      hdr->gpl != GPL || hdr->ring != RING)
    return;  // every workgroup sees the same header, so all leave together
  const EntryPtr ents = (EntryPtr)(reinterpret_cast<uintptr_t>(hdr + 1));

  constexpr int SG = chain_seg_groups(M);
  constexpr int XG = chain_x_groups(M);
  __shared__ u32x4 xl[kXLdsBytes / 16];  // x of the current pass: [m][XG groups][32 halfs]
  __shared__ float xsl[kXLdsBytes / 64];  // the pass's group sums: [m][XG groups]
  __shared__ float ys[kYLdsBytes / 4];   // partials of the current block: [tile][segment][row][m]
  __shared__ int x_epoch;                // stages whose x is in xl
  __shared__ int units_done;             // units written to ys so far
  __shared__ int s_abort;

  // Poll an LDS counter until it reaches v; false: the launch is being
  // abandoned. Every lane reads the same word; taking lane 0's value keeps the
  // loop's exit (and so everything after it) wave-uniform in the compiler's
  // eyes, which keeps the walk in scalar registers and its plan reads scalar.
  auto lds_wait_ge = [&](const int* p, int v) __attribute__((always_inline)) -> bool {
    unsigned spins = 0;
    while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) < v) {
      if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&s_abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)))
        return false;
      if (++spins > kLdsSpinLimit) {
        __hip_atomic_store(&s_abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  };

  if (wave < kComputeWaves) {
    // ------------------------------------------------------------ compute wave
    const int voff = lane * 16;  // this lane's byte offset in every weight descriptor
    auto fetch = [&](const Cursor& u, TileLoads<GPL>& L) __attribute__((always_inline)) {
      // -1 inside the walk, 0 past its end (every load then out of range)
      const int valid = ~((count - 1 - u.w.p) >> 31);
      const int seg = u.w.sg0 + u.si;
      int g0[GPL];
#pragma unroll
      for (int k = 0; k < GPL; ++k) g0[k] = seg * SG + k * 64;
      const EntryPtr e = u.w.e;
      fetch_tile_rows<GPL>(e->codes, e->sm, e->N, e->G, (u.w.tb0 + u.ti) & valid, g0, voff, valid, L);
    };

    int cur_s = -1;

    // compute unit u from its loads; false when the walk is over
    auto consume = [&](const Cursor& u, const TileLoads<GPL>& L) __attribute__((always_inline)) -> bool {
      if (u.w.p >= count) return false;
      if (u.w.s != cur_s) {
        if (!lds_wait_ge(&x_epoch, u.w.s + 1)) return false;
        cur_s = u.w.s;
      }
      const int ti = u.ti;
      const int seg = u.w.sg0 + u.si;
      LdsX<M, GPL, XG> xa{xl, xsl, {}};
#pragma unroll
      for (int k = 0; k < GPL; ++k) xa.gl[k] = (seg - u.w.sg0) * SG + k * 64 + lane;
      float acc[kTileRows][M], v[M];
      compute_tile<M, GPL>(L, xa, acc);
      tile_sums<M>(acc, v);
      // lane 16r + m writes the partial of row r, activation row m
      if ((lane & 15) < M)
        ys[(ti * u.w.e->S + seg) * kTileRows * M + (lane >> 4) * M + (lane & 15)] = pick_sum<M>(v, lane);
      if (lane == 0) __hip_atomic_fetch_add(&units_done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      return true;
    };

    Cursor F;
    F.w.s = 0;
    walk_product(F.w, ents, 0, nwg, wg);
    walk_stage<M>(F.w);
    F.ti = 0;
    F.si = 0;
    unit_add(F.ti, F.si, F.w.ns, wave);
    cursor_settle<M>(F, ents, count, nwg, wg, wave);
    Cursor C = F;
    auto advance = [&](Cursor& u) __attribute__((always_inline)) {
      unit_add(u.ti, u.si, u.w.ns, kComputeWaves);
      cursor_settle<M>(u, ents, count, nwg, wg, wave);
    };

    // Ring of RING load buffers in a fixed rotation: the loads of the unit
    // RING-1 ahead are issued before each unit is computed, so RING-1 units
    // stay in flight while one is computed. Every fetch is unconditional
    // (past the end it reads nothing), so no buffer is merged behind a branch.
    TileLoads<GPL> L[RING];
#pragma unroll
    for (int k = 0; k < RING - 1; ++k) {
      fetch(F, L[k]);
      advance(F);
    }
    lds_barrier();  // the sync wave has initialised the LDS counters
    auto step = [&](auto kc) __attribute__((always_inline)) -> bool {
      constexpr int k = decltype(kc)::value % RING;
      fetch(F, L[(k + RING - 1) % RING]);
      advance(F);
      __builtin_amdgcn_sched_barrier(0);
      if (!consume(C, L[k])) return false;
      advance(C);
      return true;
    };
    // two rotations per loop trip: the compiler's wait counts at the top of
    // the loop are conservative (one unit in flight instead of RING-1)
    while (ring_steps<0, 2 * RING>(step)) {
    }
  } else {
    // --------------------------------------------------------------- sync wave
    // ordering tree: workgroup b reports to leaf b % leaves
    const int leaves = nwg < kLeaves ? nwg : kLeaves;
    const int leaf = wg % leaves;
    const unsigned leaf_size = unsigned((nwg - leaf + leaves - 1) / leaves);
    if (lane == 0) {
      x_epoch = 0;
      units_done = 0;
      s_abort = 0;
    }
    lds_barrier();

    bool aborted = false;
    int arrived = 0;
    auto give_up = [&]() {
      aborted = true;
      if (lane == 0) {
        add_coherent(ws + kErrorWord, 1u);
        __hip_atomic_store(&s_abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    };
    // wait until products 0..i-1 are complete everywhere; false: give up
    auto wait_for = [&](int i) -> bool {
      int ok = 1;
      if (lane == 0) {
        unsigned spins = 0;
        while (ld_coherent(ws + flag_word(leaf)) < unsigned(i)) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kSpinLimit) {
            ok = 0;
            break;
          }
        }
      }
      return __builtin_amdgcn_readfirstlane(ok) != 0;
    };
    // this workgroup's results of product i are written: report to the tree;
    // the last report of a leaf climbs to the top, the last at the top raises
    // every leaf's flag to i+1
    auto arrive = [&](int i) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's coherent y stores are complete
      if (lane == 0) {
        const unsigned old = add_coherent(ws + leaf_word(leaf), 1u);
        if (old == unsigned(i + 1) * leaf_size - 1u) {
          const unsigned top = add_coherent(ws + kTopWord, 1u);
          if (top == unsigned(i + 1) * unsigned(leaves) - 1u)
            for (int l = 0; l < leaves; ++l) st_coherent(ws + flag_word(l), unsigned(i + 1));
        }
      }
      ++arrived;
    };
    // the stage's pass of activations, global -> LDS, with each group's sum;
    // groups of the pass's last segment past G read as zeros. All loads of a
    // batch are issued before the first is used: staging sits between an
    // ordering point and the compute of the next product. The first product's
    // activations were written before the launch and are read through the
    // caches; every later product's may have been written by an earlier
    // product of this launch on another XCD and are read device-coherently.
    auto stage_x = [&](const Walk& w, auto policy) {
      constexpr int kPolicy = decltype(policy)::value;
      const EntryPtr e = w.e;
      const int G = e->G;
      const int gb = w.sg0 * SG;                               // first group of the pass
      const int ng = G - gb < w.ns * SG ? G - gb : w.ns * SG;  // groups of x in the pass
      const int chunks = ng * 4;                               // 16-byte chunks per activation row
      const int total = M * chunks;
      const __amdgpu_buffer_rsrc_t rx = make_rsrc(e->x, M * G * 64);
      constexpr int kBatch = 16;
      for (int base = 0; base < total; base += 64 * kBatch) {
        u32x4 v[kBatch];
        int mk[kBatch], rk[kBatch];
        int m = (base + lane) / chunks, r = base + lane - m * chunks;  // chunk r of activation row m
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          mk[k] = m;
          rk[k] = r;
          // past the end: an offset beyond the buffer reads zeros and no memory
          const int off = m < M ? ((m * G + gb) * 4 + r) * 16 : M * G * 64;
          v[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, kPolicy);
          r += 64;
          while (r >= chunks) {
            r -= chunks;
            ++m;
          }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          // lanes 4g..4g+3 hold group g's four chunks: its sum in the fixed tree
          float t = chunk_sum(v[k]);
          t += dpp<0xB1>(t);  // (c0 + c1), (c2 + c3)
          t += dpp<0x4E>(t);  // (c0 + c1) + (c2 + c3)
          if (mk[k] < M) {
            xl[mk[k] * XG * 4 + rk[k]] = v[k];
            if ((lane & 3) == 0) xsl[mk[k] * XG + rk[k] / 4] = t;
          }
        }
      }
      const int pad = w.ns * SG - ng;  // groups past G in the last segment
      for (int idx = lane; idx < M * pad * 4; idx += 64) {
        const int m = idx / (pad * 4), r = idx - m * (pad * 4);
        xl[m * XG * 4 + chunks + r] = u32x4{0, 0, 0, 0};
        if ((r & 3) == 0) xsl[m * XG + ng + r / 4] = 0.f;
      }
    };
    // the block's partials, summed over segments in order, to y
    auto flush = [&](const Walk& w) {
      const EntryPtr e = w.e;
      const int S = e->S, N = e->N;
      for (int idx = lane; idx < w.nt * kTileRows * M; idx += 64) {
        const int ti = idx / (kTileRows * M);
        const int rm = idx - ti * (kTileRows * M);
        const int n = (w.tb0 + ti) * kTileRows + rm / M;
        float s = 0.f;
        for (int seg = 0; seg < S; ++seg) s += ys[(ti * S + seg) * kTileRows * M + rm];
        if (n < N) store_y<true>(e->y + size_t(rm % M) * N + n, s);
      }
    };

    Walk w;
    w.s = 0;
    walk_product(w, ents, 0, nwg, wg);
    walk_stage<M>(w);
    int units = 0;
    int staged_p = -1, staged_c = -1;
    while (true) {
      const int p = w.p;
      if (w.b == 0 && w.c == 0 && p > 0) {  // a new product: every earlier one must be complete
        if (!wait_for(p)) {
          give_up();
          break;
        }
      }
      if (w.nt > 0 && (p != staged_p || w.c != staged_c)) {
        if (p == 0)
          stage_x(w, std::integral_constant<int, 0>{});
        else
          stage_x(w, std::integral_constant<int, kLoadCoherent>{});
        staged_p = p;
        staged_c = w.c;
      }
      units += w.nt * w.ns;
      if (lane == 0) __hip_atomic_store(&x_epoch, w.s + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (!lds_wait_ge(&units_done, units)) {
        give_up();
        break;
      }
      const bool block_done = w.c == w.e->passes - 1;
      const bool product_done = block_done && w.b == w.nb - 1;
      if (block_done && w.nt > 0) flush(w);
      if (!walk_next<M>(w, ents, count, nwg, wg)) break;
      if (product_done) arrive(p);
    }

    // Count out. After giving up, first release every waiter (results of this
    // call are then invalid and the error word says so). The last workgroup
    // out resets every counter and flag for the next call. A single product
    // touches no counter and skips this.
    if (lane == 0 && count > 1) {
      if (aborted || arrived < count - 1)
        for (int l = 0; l < leaves; ++l) st_coherent(ws + flag_word(l), unsigned(count));
      const unsigned prev = add_coherent(ws + kExitWord, 1u);
      if (prev == unsigned(nwg) - 1u) {
        st_coherent(ws + kTopWord, 0u);
        for (int l = 0; l < leaves; ++l) {
          st_coherent(ws + leaf_word(l), 0u);
          st_coherent(ws + flag_word(l), 0u);
        }
        st_coherent(ws + kExitWord, 0u);
      }
    }
  }
}

typedef void (*chain_fn)(const ChainHeader*, unsigned*, int);

template <int M>
constexpr chain_fn chain_instance() {
  return &chain_kernel<M, chain_gpl(M), chain_ring(M)>;
}

chain_fn chain_for(int M) {
  switch (M) {
    case 1: return chain_instance<1>();
    case 2: return chain_instance<2>();
    case 3: return chain_instance<3>();
    case 4: return chain_instance<4>();
    case 5: return chain_instance<5>();
    case 6: return chain_instance<6>();
    case 7: return chain_instance<7>();
    case 8: return chain_instance<8>();
    default: return nullptr;
  }
}

std::atomic<int> g_chain_occupancy[kMaxM + 1];

constexpr int32_t kMaxChain = 1 << 20;

}  // namespace

extern "C" size_t w4a16_chain_plan_bytes(int32_t count) {
  if (count < 1 || count > kMaxChain) return 0;
  return sizeof(ChainHeader) + size_t(count) * sizeof(ChainEntry);
}

extern "C" w4a16_status w4a16_chain_plan(const w4a16_chain_entry* entries, int32_t count, int32_t M, void* plan,
                                         size_t plan_bytes) {
  using w4a16_host::ranges_overlap;
  if (!entries || !plan) return W4A16_ERR_NULL;
  if (count < 1 || count > kMaxChain || M < 1 || M > kMaxM) return W4A16_ERR_SHAPE;
  const size_t need = w4a16_chain_plan_bytes(count);
  if (plan_bytes < need) return W4A16_ERR_SIZE;
  for (int32_t i = 0; i < count; ++i) {
    const w4a16_chain_entry& e = entries[i];
    if (!e.x || !e.packed || !e.y) return W4A16_ERR_NULL;
    if (e.N < 1 || e.K < kGroup || e.K % kGroup || e.K > w4a16_max_k(M) || w4a16_packed_bytes(e.N, e.K) == 0)
      return W4A16_ERR_SHAPE;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(e.x), pa = reinterpret_cast<uintptr_t>(e.packed),
                    ya = reinterpret_cast<uintptr_t>(e.y);
    if (xa % 16 || pa % 256 || ya % 4) return W4A16_ERR_ALIGN;
    const size_t yb = size_t(M) * size_t(e.N) * sizeof(float);
    if (ranges_overlap(ya, yb, xa, size_t(M) * size_t(e.K) * 2)) return W4A16_ERR_OVERLAP;
  }
  for (int32_t i = 0; i < count; ++i) {  // no weights inside any product's output
    const uintptr_t ya = reinterpret_cast<uintptr_t>(entries[i].y);
    const size_t yb = size_t(M) * size_t(entries[i].N) * sizeof(float);
    for (int32_t j = 0; j < count; ++j) {
      const uintptr_t pa = reinterpret_cast<uintptr_t>(entries[j].packed);
      if (ranges_overlap(ya, yb, pa, w4a16_packed_bytes(entries[j].N, entries[j].K))) return W4A16_ERR_OVERLAP;
    }
  }

  ChainHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kChainMagic;
  h.version = kChainVersion;
  h.count = count;
  h.M = M;
  h.gpl = chain_gpl(M);
  h.ring = chain_ring(M);
  const int sg = chain_seg_groups(M), sp = chain_pass_segs(M);
  uint8_t* out = static_cast<uint8_t*>(plan);
  std::memcpy(out, &h, sizeof(h));
  for (int32_t i = 0; i < count; ++i) {
    const w4a16_chain_entry& e = entries[i];
    const int G = e.K / kGroup;
    const size_t codes_region = (size_t(e.N) * size_t(e.K) / 2 + 255) / 256 * 256;
    ChainEntry c;
    std::memset(&c, 0, sizeof(c));
    c.x = static_cast<const u32x4*>(e.x);
    c.codes = static_cast<const u32x4*>(e.packed);
    c.sm = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(e.packed) + codes_region);
    c.y = e.y;
    c.N = e.N;
    c.G = G;
    c.T = (e.N + kTileRows - 1) / kTileRows;
    c.S = (G + sg - 1) / sg;
    c.passes = (c.S + sp - 1) / sp;
    // one tile's partials fit: S * 4 * M floats <= kYLdsBytes for every K <= w4a16_max_k
    c.TB = kYLdsBytes / (c.S * kTileRows * M * int(sizeof(float)));
    std::memcpy(out + sizeof(ChainHeader) + size_t(i) * sizeof(ChainEntry), &c, sizeof(c));
  }
  return W4A16_OK;
}

extern "C" w4a16_status w4a16_chain_launch_shape(int32_t M, int32_t out[3]) {
  if (!out) return W4A16_ERR_NULL;
  if (M < 1 || M > kMaxM) return W4A16_ERR_SHAPE;
  out[0] = M;
  out[1] = chain_gpl(M);
  out[2] = chain_ring(M);
  return W4A16_OK;
}

namespace {

w4a16_status chain_enqueue(const void* plan, int32_t count, int32_t M, void* workspace, size_t workspace_bytes,
                           void* stream, hipEvent_t start, hipEvent_t stop) {
  if (!plan || !workspace) return W4A16_ERR_NULL;
  if (count < 1 || count > kMaxChain || M < 1 || M > kMaxM) return W4A16_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(plan) % 16 || reinterpret_cast<uintptr_t>(workspace) % 16) return W4A16_ERR_ALIGN;
  if (workspace_bytes < W4A16_CHAIN_WORKSPACE_BYTES) return W4A16_ERR_SIZE;
  chain_fn fn = chain_for(M);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  int occ = g_chain_occupancy[M].load(std::memory_order_relaxed);
  if (occ <= 0) {
    occ = w4a16_host::occupancy_of(reinterpret_cast<const void*>(fn), 64 * kWaves);
    g_chain_occupancy[M].store(occ, std::memory_order_relaxed);
  }
  // every workgroup must be resident at once: the grid is the occupancy limit
  const int grid = w4a16_host::cu_count(dev) * occ;
  const ChainHeader* hp = static_cast<const ChainHeader*>(plan);
  unsigned* wp = static_cast<unsigned*>(workspace);
  int n_arg = count;
  void* args[] = {&hp, &wp, &n_arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(64 * kWaves), args, 0,
                         static_cast<hipStream_t>(stream), start, stop, 0) != hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}

}  // namespace

extern "C" w4a16_status w4a16_gemv_chain(const void* plan, int32_t count, int32_t M, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return chain_enqueue(plan, count, M, workspace, workspace_bytes, stream, nullptr, nullptr);
}

extern "C" w4a16_status w4a16_gemv_chain_timed(const void* plan, int32_t count, int32_t M, void* workspace,
                                               size_t workspace_bytes, void* stream, void* start_event,
                                               void* stop_event) {
  if (!start_event || !stop_event) return W4A16_ERR_NULL;
  return chain_enqueue(plan, count, M, workspace, workspace_bytes, stream, static_cast<hipEvent_t>(start_event),
                       static_cast<hipEvent_t>(stop_event));
}
