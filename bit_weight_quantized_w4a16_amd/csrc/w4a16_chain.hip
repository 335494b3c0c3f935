// gfx950 kernel and C-ABI entry points of the decode-step chain: a list of
// W4A16 GEMVs executed in order by ONE persistent launch.
//
// Why: a decode step is the same list of matrix-vector products every token
// (the tight decode loop of the core-modules page, section 5.2), and its
// scheduler notes (section 5.3) call for fetching the next product's weights
// while other work runs. On an MI355X a kernel boundary costs several
// microseconds (dispatch ramp, cold first loads, drain), paid 128 times by a
// 32-layer 8B step even when every weight byte is already cached; the weights
// of later products never depend on earlier results, so one launch can keep
// HBM streaming straight through the ordering points between products.
//
// How: one workgroup per CU, twelve waves with two roles.
//
// * Four loader waves stream weights and nothing else. The workgroup's work
//   is a sequence of units (product, 4-row tile, K segment of 64 groups of
//   32 weights); a unit's bytes are 4 rows x 1 KiB of code chunks plus 1 KiB
//   of scale/min entries. A loader keeps five units of 128-bit loads in
//   flight in its registers and copies each unit, once it has landed, into a
//   ring of LDS slots, unit after unit and product after product, as fast as
//   slots free up. Loaders never wait on an ordering point, so up to the ring
//   plus the loaders' registers of the next products' weights (about 220 KiB
//   per CU) stream in while the current product completes.
//
// * Eight compute waves take the units round-robin. Before a product's units
//   they stage its activations into LDS together (each lane one group of 32
//   values and its sum). A unit is computed from its slot and the staged
//   activations; its 4 x M wave sums go to LDS, and the wave that completes
//   the last segment of a tile adds the segment sums in order and stores y.
//   The weights arrive through LDS, so a compute wave's memory counter holds
//   only its own activation loads and y stores: waiting for those never
//   drains weight loads.
//
// Ordering between products: when a product's units are done in a
// workgroup, each compute wave waits for its own y stores to complete and
// counts itself out in LDS; the last one reports to a two-level counter tree
// in the caller's workspace (the last arrival at a leaf climbs to the top
// counter, the last arrival at the top raises every leaf's flag to i+1) and
// waits for its leaf flag, then lets the workgroup's compute waves stage the
// next product's activations. Every wait is bounded: a wait that gives up
// flags the workspace's error word, releases the other workgroups and ends
// the launch (its results are then invalid), so a launch whose workgroups
// cannot all be resident ends instead of hanging. The last workgroup out
// resets the counters for the next call.
//
// Memory model. y is written with device-coherent stores (sc1: through to
// memory, no L2 write-back needed); the tree's atomics and flags are
// device-coherent too, and a wave counts itself out only after its stores are
// acknowledged. An activation buffer that an earlier product of the plan
// writes is read with device-coherent loads (no stale L2 line of another XCD
// can serve it); one that no product of the plan writes is read through the
// caches, where no stale copy can exist (the kernel's start invalidates them).
// The host plan marks which is which.
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
constexpr uint32_t kChainVersion = 5;
constexpr unsigned kSpinLimit = 1u << 20;      // global polls before an ordering wait gives up (~1 s)
constexpr unsigned kLdsSpinLimit = 1u << 24;   // LDS polls before a wave gives up (about a second)
constexpr int kLeaves = 16;                    // leaf counters of the ordering tree
constexpr int kLineWords = 1024;               // 4 KiB between counters (separate memory pages)
constexpr int kLoaderDepth = 5;                // units in flight (in registers) per loader wave
// loader and compute waves per workgroup: eight loaders while the compute
// waves' registers fit four waves per SIMD (128 VGPRs), else four; eight
// compute waves
__host__ __device__ constexpr int chain_loader_waves(int) { return 4; }
__host__ __device__ constexpr int chain_compute_waves(int) { return 8; }
constexpr int kRing = 24;                      // LDS ring slots (a multiple of both wave counts)
constexpr int kSeg = 64;                       // groups per K segment (one per lane)
constexpr int kUnitBytes = (kTileRows + 1) * kSeg * 16;  // 4 code rows + the scale/min entries
constexpr int kXBytes = 32768;                 // LDS activations of one pass over K
constexpr int kPartFloats = 1024;              // LDS segment sums and running sums of a block of tiles
constexpr int kMaxBlockTiles = 32;
constexpr int kLoadCoherent = 16;              // buffer-load cache policy: device-coherent (sc1)
constexpr int32_t kMaxChain = W4A16_CHAIN_MAX_ENTRIES;
static_assert(kRing % 8 == 0 && kRing % 4 == 0,
              "a slot is always filled by the same loader and emptied by the same compute wave");

// K segments of activations one LDS pass holds, and tiles per block (a block's
// segment sums of one pass and its running sums fit kPartFloats)
__host__ __device__ constexpr int chain_pass_segs(int M) { return kXBytes / (M * kSeg * 64); }
__host__ __device__ constexpr int chain_block_tiles(int M) {
  return kPartFloats / (chain_pass_segs(M) * kTileRows * M + kTileRows * M) < kMaxBlockTiles
             ? kPartFloats / (chain_pass_segs(M) * kTileRows * M + kTileRows * M)
             : kMaxBlockTiles;
}

struct ChainHeader {
  uint32_t magic, version;
  int32_t count, M, ring, compute_waves;
  int32_t pad[10];
};
static_assert(sizeof(ChainHeader) == 64, "plan header is 64 bytes");

struct ChainEntry {
  const u32x4* x;
  const u32x4* codes;
  const u32x4* sm;
  float* y;
  int32_t N, G, T;  // rows, groups per row, 4-row tiles
  int32_t S;        // K segments per row
  int32_t passes;   // LDS passes of the activations over the segments
  int32_t xcoh;     // 1: x may have been written by an earlier entry (device-coherent loads)
  int32_t pad[2];
};
static_assert(sizeof(ChainEntry) == 64, "plan entry is 64 bytes");

// The plan never changes during a launch: it is read through the constant
// address space, which the compiler always serves with scalar loads.
typedef const __attribute__((address_space(4))) ChainEntry* EntryPtr;

// Workspace words: the tree's top counter, the exit counter and the error
// word share the first page; leaf g's counter and flag sit on page 1 + g.
constexpr int kTopWord = 0, kExitWord = 32, kErrorWord = W4A16_CHAIN_ERROR_OFFSET / 4;
constexpr int leaf_word(int g) { return kLineWords * (1 + g); }
constexpr int flag_word(int g) { return kLineWords * (1 + g) + 32; }
static_assert(kLineWords * (1 + kLeaves) * 4 == W4A16_CHAIN_WORKSPACE_BYTES, "workspace layout");
static_assert(kErrorWord > kExitWord && kErrorWord < kLineWords, "error word on the first page");

__device__ __forceinline__ unsigned ld_coherent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_coherent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_coherent(unsigned* p, unsigned v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// keeps the compiler from moving memory accesses across this point (no instruction)
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// LDS of one workgroup
struct ChainLds {
  u32x4 ring[kRing * kUnitBytes / 16];   // unit slots: code rows 0..3, then scale/min
  u32x4 xl[kXBytes / 16];                // activations of the pass: [m][chunk][group]
  float xsl[kXBytes / 64];               // their group sums: [m][group]
  float part[kPartFloats];               // [tile][segment of the pass][row][m], then running [tile][row][m]
  int tile_cnt[kMaxBlockTiles];          // segments of the current pass done, per tile of the block
  int ready[kRing];                      // units landed in each slot
  int consumed[kRing];                   // units taken out of each slot
  int done;                              // compute waves past the end of a stage, all stages so far
  int go;                                // stages released
  int staged;                            // compute waves done staging, all stagings so far
  int abort;                             // a wait gave up: every wave leaves
  int bad_blob;                          // some entry's blob header does not match it: nothing is stored
};

// One stage of a workgroup's walk: block b of its tiles of product p, pass c
// over K. All fields are wave-uniform (scalar registers).
struct Stage {
  int p, b, c;
  EntryPtr e;
  int N, G, T, S, passes, xcoh;
  int t0, ntile, nb;  // this workgroup's tiles of p: first, count, blocks
  int tb0, nt;        // the stage's first tile and tile count
  int sg0, ns;        // its first segment and segment count
  int ubase;          // running index (within the workgroup) of its first unit
  unsigned inv;       // ceil(2^32 / workgroups)
};

template <int M>
__device__ __forceinline__ void stage_set(Stage& s) {
  constexpr int TB = chain_block_tiles(M), XS = chain_pass_segs(M);
  s.tb0 = s.t0 + s.b * TB;
  const int left = s.ntile - s.b * TB;
  s.nt = left < TB ? (left > 0 ? left : 0) : TB;
  s.sg0 = s.c * XS;
  s.ns = s.S - s.sg0 < XS ? s.S - s.sg0 : XS;
}

// q = T / nwg, r = T % nwg from the launch-wide reciprocal inv = ceil(2^32 / nwg)
// (scalar multiply-high and one correction step: a division here would be
// emulated in vector registers and pull the walk out of scalar registers)
__device__ __forceinline__ void split_tiles(int T, int nwg, unsigned inv, int& q, int& r) {
  if (nwg == 1) {
    q = T;
    r = 0;
    return;
  }
  q = int(__umulhi(unsigned(T), inv));
  r = T - q * nwg;
  if (r < 0) {
    --q;
    r += nwg;
  }
  if (r >= nwg) {
    ++q;
    r -= nwg;
  }
}

template <int M>
__device__ __forceinline__ void stage_product(Stage& s, EntryPtr ents, int p, int nwg, int wg) {
  constexpr int TB = chain_block_tiles(M);
  s.p = p;
  s.e = ents + p;
  s.N = s.e->N;
  s.G = s.e->G;
  s.T = s.e->T;
  s.S = s.e->S;
  s.passes = s.e->passes;
  s.xcoh = s.e->xcoh;
  int q, rem;
  split_tiles(s.T, nwg, s.inv, q, rem);
  s.t0 = wg * q + (wg < rem ? wg : rem);
  s.ntile = q + (wg < rem ? 1 : 0);
  s.nb = s.ntile > 0 ? (s.ntile + TB - 1) / TB : 1;  // a workgroup with no tiles walks one empty stage
  s.b = 0;
  s.c = 0;
  stage_set<M>(s);
}

// next stage; false past the last product
template <int M>
__device__ __forceinline__ bool stage_next(Stage& s, EntryPtr ents, int count, int nwg, int wg) {
  s.ubase += s.nt * s.ns;
  if (++s.c == s.passes) {
    s.c = 0;
    if (++s.b == s.nb) {
      if (s.p + 1 >= count) return false;
      stage_product<M>(s, ents, s.p + 1, nwg, wg);
      return true;
    }
  }
  stage_set<M>(s);
  return true;
}

// first unit index i >= 0 of a stage with (ubase + i) % n == k, as (tile, segment)
__device__ __forceinline__ int first_unit(int ubase, int k, int n) {
  const int r = (k - ubase) % n;
  return r < 0 ? r + n : r;
}
// (ti, si) + n units, ns segments per tile
__device__ __forceinline__ void unit_step(int& ti, int& si, int ns, int n) {
  si += n;
  while (si >= ns) {
    si -= ns;
    ++ti;
  }
}

// Activations read from LDS as they are used: chunk d of row m's group at
// pass-local index gl, and that group's sum. LDS holds them chunk-major,
// [m][chunk][group], so the 64 lanes of a wave (64 consecutive groups) read
// 1 KiB of consecutive bytes per chunk, free of bank conflicts.
template <int M, int XG>
struct LdsX {
  static constexpr bool kRowOuter = false;  // each chunk is an LDS read: walk a tile chunk by chunk
  const u32x4* xl;
  const float* xsl;
  int gl;
  __device__ __forceinline__ u32x4 x(int m, int, int d) const { return xl[(m * 4 + d) * XG + gl]; }
  __device__ __forceinline__ float sum(int m, int) const { return xsl[m * XG + gl]; }
};

// step(k) for k = K .. N-1 with k a compile-time constant (register-ring
// buffer indices must be constants); false as soon as one step ends the walk
template <int K, int N, class Step>
__device__ __forceinline__ bool ring_steps(Step& step) {
  if constexpr (K == N) {
    return true;
  } else {
    if (!step(std::integral_constant<int, K>{})) return false;
    return ring_steps<K + 1, N>(step);
  }
}

template <int M, int RING, int NCW>
__global__ void __launch_bounds__(64 * (chain_loader_waves(M) + NCW))
chain_kernel(const ChainHeader* __restrict__ hdr, unsigned* __restrict__ ws, int count, int nwg) {
  static_assert(RING == kRing && NCW == chain_compute_waves(M), "one ring; the compute waves of M");
  constexpr int XS = chain_pass_segs(M);
  constexpr int XG = XS * kSeg;  // groups of one LDS pass
  constexpr int TB = chain_block_tiles(M);
  constexpr int NL = chain_loader_waves(M);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // nwg (the launch's workgroup count) is an argument: every explicit
  // argument arrives preloaded in scalar registers, gridDim.x would be a load
  const int wg = blockIdx.x;
  // the header's six words in one go (a chain of || would load and wait for
  // them one at a time)
  const uint32_t h_magic = hdr->magic, h_version = hdr->version;
  const int32_t h_count = hdr->count, h_m = hdr->M, h_ring = hdr->ring, h_cw = hdr->compute_waves;
  if ((h_magic != kChainMagic) | (h_version != kChainVersion) | (h_count != count) | (h_m != M) | (h_ring != RING) |
      (h_cw != NCW)) {
    // every workgroup sees the same header, so all leave together
    if (wg == 0 && threadIdx.x == 0) or_coherent(ws + kErrorWord, W4A16_CHAIN_ERR_PLAN);
    return;
  }
  const EntryPtr ents = (EntryPtr)(reinterpret_cast<uintptr_t>(hdr + 1));
  const unsigned inv = __builtin_amdgcn_readfirstlane(nwg > 1 ? 0xFFFFFFFFu / unsigned(nwg) + 1u : 0u);

  __shared__ ChainLds L;
  constexpr int kThreads = 64 * (chain_loader_waves(M) + NCW);
  for (int i = threadIdx.x; i < kRing; i += kThreads) L.ready[i] = L.consumed[i] = 0;
  for (int i = threadIdx.x; i < kMaxBlockTiles; i += kThreads) L.tile_cnt[i] = 0;
  if (threadIdx.x == 0) L.done = L.go = L.staged = L.abort = L.bad_blob = 0;
  __syncthreads();  // the only workgroup barrier: nothing is in flight yet

  auto lds_aborted = [&]() __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(&L.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
  };

  if (wave < NL) {
    // ------------------------------------------------------------- loader wave
    // A ring of D units in registers: the loads of the unit D-1 ahead go out
    // before the oldest unit is copied into its LDS slot (the copy waits for
    // that unit's loads only, and for its slot to be free). Weight bytes in
    // flight live in these registers; the LDS ring holds landed units only.
    constexpr int D = kLoaderDepth;
    const int voff = lane * 16;
    struct Cur {
      Stage s;
      int i, ti, si;
      int valid;  // -1 inside the walk, 0 past its end (every load then reads nothing)
    };
    auto settle = [&](Cur& c) __attribute__((always_inline)) {
      while (c.valid && c.i >= c.s.nt * c.s.ns) {
        if (!stage_next<M>(c.s, ents, count, nwg, wg)) {
          c.valid = 0;
          break;
        }
        c.i = first_unit(c.s.ubase, wave, NL);
        c.ti = 0;
        c.si = 0;
        unit_step(c.ti, c.si, c.s.ns, c.i);
      }
    };
    auto advance = [&](Cur& c) __attribute__((always_inline)) {
      c.i += NL;
      unit_step(c.ti, c.si, c.s.ns, NL);
      settle(c);
    };
    auto fetch = [&](const Cur& c, TileLoads<1>& T) __attribute__((always_inline)) {
      const int g0[1] = {(c.s.sg0 + c.si) * kSeg};
      fetch_tile_rows<1>(c.s.e->codes, c.s.e->sm, c.s.N, c.s.G, (c.s.tb0 + c.ti) & c.valid, g0, voff, c.valid, T);
    };
    int ok = 1;  // 0 once a wait gave up (every later copy is skipped)
    // copy a landed unit into its slot once the slot's previous unit was
    // taken out, then publish it; nothing past the end of the walk
    auto copy = [&](const Cur& c, const TileLoads<1>& T) __attribute__((always_inline)) {
      const int u = c.s.ubase + c.i;
      const int slot = u % RING, k = u / RING;
      unsigned spins = 0;
      int go = c.valid & ok;
      while (go && __builtin_amdgcn_readfirstlane(__hip_atomic_load(&L.consumed[slot], __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_WORKGROUP)) < k) {
        if (lds_aborted()) {
          ok = go = 0;
        } else if (++spins > kLdsSpinLimit) {  // starved: make every wave of the workgroup leave
          __hip_atomic_store(&L.abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          if (lane == 0) or_coherent(ws + kErrorWord, W4A16_CHAIN_ERR_WAIT);
          ok = go = 0;
        } else {
          __builtin_amdgcn_s_sleep(2);
        }
      }
      if (go) {
        compiler_fence();
        u32x4* dst = L.ring + slot * (kUnitBytes / 16);
#pragma unroll
        for (int r = 0; r < kTileRows; ++r) dst[r * 64 + lane] = T.code[r][0];
        dst[kTileRows * 64 + lane] = T.sm[0];
        compiler_fence();  // LDS operations complete in order: the data before the flag
        if (lane == 0) __hip_atomic_store(&L.ready[slot], k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    };
    Cur F;
    F.s.ubase = 0;
    F.s.inv = inv;
    stage_product<M>(F.s, ents, 0, nwg, wg);
    F.valid = -1;
    F.i = first_unit(0, wave, NL);
    F.ti = 0;
    F.si = 0;
    unit_step(F.ti, F.si, F.s.ns, F.i);
    settle(F);
    Cur C = F;
    TileLoads<1> B[D];
#pragma unroll
    for (int k = 0; k < D - 1; ++k) {
      fetch(F, B[k]);
      advance(F);
    }
    // every step runs (a copy past the end does nothing); the walk's end is
    // tested once per two rotations of the ring, so no buffer is live across
    // an exit in the middle of the rotation
    auto step = [&](auto kc) __attribute__((always_inline)) -> bool {
      constexpr int k = decltype(kc)::value % D;
      fetch(F, B[(k + D - 1) % D]);
      advance(F);
      __builtin_amdgcn_sched_barrier(0);
      copy(C, B[k]);
      advance(C);
      return true;
    };
    do {
      ring_steps<0, 2 * D>(step);
    } while (C.valid && ok);
    return;
  }

  // --------------------------------------------------------------- compute wave
  const int cw = wave - NL;
  // ordering tree: workgroup b reports to leaf b % leaves
  const int leaves = nwg < kLeaves ? nwg : kLeaves;
  const int leaf = wg % leaves;
  const unsigned leaf_size = unsigned((nwg - leaf + leaves - 1) / leaves);
  bool aborted = false;
  auto give_up = [&]() {
    aborted = true;
    if (lane == 0) {
      or_coherent(ws + kErrorWord, W4A16_CHAIN_ERR_WAIT);
      __hip_atomic_store(&L.abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  };
  // Poll an LDS counter until it reaches v; false: the launch is being
  // abandoned. Taking lane 0's value keeps everything after the loop
  // wave-uniform in the compiler's eyes.
  auto lds_wait_ge = [&](const int* p, int v) __attribute__((always_inline)) -> bool {
    unsigned spins = 0;
    while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < v) {
      if (lds_aborted()) return false;
      if (++spins > kLdsSpinLimit) {
        give_up();
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    compiler_fence();
    return true;
  };
  // wait until products 0..i-1 are complete everywhere; false: give up
  auto wait_for = [&](int i) -> bool {
    int ok = 1;
    if (lane == 0) {
      unsigned spins = 0;
      while (ld_coherent(ws + flag_word(leaf)) < unsigned(i)) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          ok = 0;
          break;
        }
      }
    }
    compiler_fence();
    return __builtin_amdgcn_readfirstlane(ok) != 0;
  };
  // this workgroup's results of product i are written: report to the tree;
  // the last report of a leaf climbs to the top, the last at the top raises
  // every leaf's flag to i+1
  auto arrive = [&](int i) {
    if (lane == 0) {
      const unsigned old = add_coherent(ws + leaf_word(leaf), 1u);
      if (old == unsigned(i + 1) * leaf_size - 1u) {
        const unsigned top = add_coherent(ws + kTopWord, 1u);
        if (top == unsigned(i + 1) * unsigned(leaves) - 1u)
          for (int l = 0; l < leaves; ++l) st_coherent(ws + flag_word(l), unsigned(i + 1));
      }
    }
  };

  // this wave's share of the stage's activations, global -> LDS, with each
  // group's sum: lane item c*64 + lane + j*NCW*64 is group (item % XG) of the
  // pass for activation row item / XG (at most one item per lane: M * XS <= 8)
  // `between` runs (on the whole wave) once the loads are issued, before
  // their data is needed
  auto stage_x = [&](const Stage& s, auto&& between) {
    const int gb = s.sg0 * kSeg;
    const int item = cw * 64 + lane;
    const bool mine = item < M * XG;
    const int m = item / XG, lg = item - m * XG;
    const int g = gb + lg;
    u32x4 v[4] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
    {
      if (mine && lg < s.ns * kSeg && g < s.G) {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(s.e->x, M * s.G * 64);
        const int off = (m * s.G + g) * 64;
        if (s.xcoh) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + q * 16, 0, kLoadCoherent);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + q * 16, 0, 0);
        }
      }
    }
    between();
    if (mine) {
#pragma unroll
      for (int q = 0; q < 4; ++q) L.xl[(m * 4 + q) * XG + lg] = v[q];
      L.xsl[m * XG + lg] = group_sum(v);
    }
  };

  // Every entry's blob header, checked once, at the compute waves' first
  // staging, behind that staging's activation loads (lane l of compute wave
  // cw takes entries 64 (cw + r NCW) + l). A mismatch anywhere marks the
  // workgroup's LDS flag before the wave joins the staging count, and every
  // y store of the launch is made after such a count and skipped if the flag
  // is set: a plan naming a wrong blob writes no y at all. The check costs
  // about one memory latency (the entry's blob address, then its header) at
  // the start of the launch and nothing in its loops.
  bool checked = false;
  auto check_blobs = [&]() __attribute__((always_inline)) {
    if (checked) return;
    checked = true;
    typedef const __attribute__((address_space(1))) uint32_t* GlobalWords;
    bool any = false;
    for (int p0 = cw * 64; p0 < count; p0 += NCW * 64) {
      const int p = p0 + lane;
      bool bad = false;
      if (p < count) {
        const GlobalWords h =
            (GlobalWords)(reinterpret_cast<uintptr_t>(ents[p].codes) - uintptr_t(W4A16_BLOB_HEADER_BYTES));
        bad = h[0] != W4A16_BLOB_MAGIC || h[1] != head_version_codec(W4A16_CODEC_Q4) ||
              h[2] != uint32_t(ents[p].N) || h[3] != uint32_t(ents[p].G * kGroup);
      }
      any = any || __ballot(bad) != 0;
    }
    if (any && lane == 0) {
      __hip_atomic_store(&L.bad_blob, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (wg == 0) or_coherent(ws + kErrorWord, W4A16_CHAIN_ERR_BLOB);
    }
  };
  bool blob_ok = false;

  Stage s;
  s.ubase = 0;
  s.inv = inv;
  stage_product<M>(s, ents, 0, nwg, wg);
  int stages = 0, stagings = 0;
  do {
    // activations: once per product when one pass holds all of K, else per stage
    if (s.nt > 0 && (s.passes > 1 || s.b == 0)) {
      stage_x(s, check_blobs);
      compiler_fence();
      ++stagings;
      if (lane == 0) __hip_atomic_fetch_add(&L.staged, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (!lds_wait_ge(&L.staged, stagings * NCW)) break;
      blob_ok = __hip_atomic_load(&L.bad_blob, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
    }
    // this wave's units of the stage
    const int units = s.nt * s.ns;
    int i = first_unit(s.ubase, cw, NCW);
    int ti = 0, si = 0;
    unit_step(ti, si, s.ns, i);
    bool ok = true;
    for (; i < units; i += NCW) {
      const int u = s.ubase + i;
      const int slot = u % RING, k = u / RING;
      if (!lds_wait_ge(&L.ready[slot], k + 1)) {
        ok = false;
        break;
      }
      TileLoads<1> T;
      const u32x4* src = L.ring + slot * (kUnitBytes / 16);
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) T.code[r][0] = src[r * 64 + lane];
      T.sm[0] = src[kTileRows * 64 + lane];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot's bytes are in registers
      compiler_fence();
      if (lane == 0) __hip_atomic_store(&L.consumed[slot], k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      float acc[kTileRows][M], v[M];
      compute_tile<M, 1>(T, LdsX<M, XG>{L.xl, L.xsl, si * kSeg + lane}, acc);
      tile_sums<M>(acc, v);
      // lane 16r + m holds output row r's sum for activation row m
      float* part = L.part + (ti * XS + si) * (kTileRows * M);
      if ((lane & 15) < M) part[(lane >> 4) * M + (lane & 15)] = pick_sum<M>(v, lane);
      compiler_fence();
      int old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(&L.tile_cnt[ti], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      old = __builtin_amdgcn_readfirstlane(old);
      if (old == s.ns - 1) {
        // the tile's last segment of this pass: add the pass's segment sums
        // in order to the running sum of the earlier passes
        compiler_fence();
        float* run = L.part + TB * XS * (kTileRows * M) + ti * (kTileRows * M);
        const float* seg = L.part + ti * XS * (kTileRows * M);
        if ((lane & 15) < M) {
          const int rm = (lane >> 4) * M + (lane & 15);
          float acc_y = s.c == 0 ? 0.f : run[rm];
          for (int sp = 0; sp < s.ns; ++sp) acc_y += seg[sp * (kTileRows * M) + rm];
          const int n = (s.tb0 + ti) * kTileRows + (lane >> 4);
          if (s.c == s.passes - 1) {
            if (n < s.N && blob_ok) store_y<true>(s.e->y + size_t(lane & 15) * s.N + n, acc_y);
          } else {
            run[rm] = acc_y;
          }
        }
        if (lane == 0) L.tile_cnt[ti] = 0;
      }
      unit_step(ti, si, s.ns, NCW);
    }
    if (!ok) break;
    // end of the stage: count out; the last compute wave of the workgroup
    // takes the ordering point when the stage ends a product
    const bool product_end = s.c == s.passes - 1 && s.b == s.nb - 1;
    if (product_end) __builtin_amdgcn_s_waitcnt(0);  // this wave's y stores are complete
    compiler_fence();
    ++stages;
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(&L.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == stages * NCW - 1) {
      if (product_end && s.p + 1 < count) {
        arrive(s.p);
        if (!wait_for(s.p + 1)) {
          give_up();
          break;
        }
      }
      if (lane == 0) __hip_atomic_store(&L.go, stages, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (!lds_wait_ge(&L.go, stages)) break;
  } while (stage_next<M>(s, ents, count, nwg, wg));

  // Count out (one wave per workgroup: the first compute wave, past the last
  // stage, after which this workgroup touches no counter). A wave that gave
  // up first releases every waiter (results of this call are then invalid
  // and the error word says so). The last workgroup out resets every counter
  // and flag for the next call. A single product touches no counter.
  if (aborted && lane == 0 && count > 1)
    for (int l = 0; l < leaves; ++l) st_coherent(ws + flag_word(l), unsigned(count));
  if (cw == 0 && lane == 0 && count > 1) {
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

typedef void (*chain_fn)(const ChainHeader*, unsigned*, int, int);

template <int M>
constexpr chain_fn chain_instance() {
  return &chain_kernel<M, kRing, chain_compute_waves(M)>;
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
  h.ring = kRing;
  h.compute_waves = chain_compute_waves(M);
  const int xs = chain_pass_segs(M);
  uint8_t* out = static_cast<uint8_t*>(plan);
  std::memcpy(out, &h, sizeof(h));
  for (int32_t i = 0; i < count; ++i) {
    const w4a16_chain_entry& e = entries[i];
    const int G = e.K / kGroup;
    const size_t codes_region = (size_t(e.N) * size_t(e.K) / 2 + 255) / 256 * 256;
    const uint8_t* base = static_cast<const uint8_t*>(e.packed);
    ChainEntry c;
    std::memset(&c, 0, sizeof(c));
    c.x = static_cast<const u32x4*>(e.x);
    c.codes = reinterpret_cast<const u32x4*>(base + W4A16_BLOB_HEADER_BYTES);  // the header precedes the codes
    c.sm = reinterpret_cast<const u32x4*>(base + W4A16_BLOB_HEADER_BYTES + codes_region);
    c.y = e.y;
    c.N = e.N;
    c.G = G;
    c.T = (e.N + kTileRows - 1) / kTileRows;
    c.S = (G + kSeg - 1) / kSeg;
    c.passes = (c.S + xs - 1) / xs;
    // an x that an earlier entry writes is read device-coherently
    const uintptr_t xa = reinterpret_cast<uintptr_t>(e.x);
    for (int32_t j = 0; j < i && !c.xcoh; ++j)
      c.xcoh = ranges_overlap(reinterpret_cast<uintptr_t>(entries[j].y), size_t(M) * size_t(entries[j].N) * 4, xa,
                              size_t(M) * size_t(e.K) * 2)
                   ? 1
                   : 0;
    std::memcpy(out + sizeof(ChainHeader) + size_t(i) * sizeof(ChainEntry), &c, sizeof(c));
  }
  return W4A16_OK;
}

extern "C" w4a16_status w4a16_chain_launch_shape(int32_t M, int32_t out[3]) {
  if (!out) return W4A16_ERR_NULL;
  if (M < 1 || M > kMaxM) return W4A16_ERR_SHAPE;
  out[0] = M;
  out[1] = kRing;
  out[2] = chain_compute_waves(M);
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
    occ = w4a16_host::occupancy_of(reinterpret_cast<const void*>(fn), 64 * (chain_loader_waves(M) + chain_compute_waves(M)));
    g_chain_occupancy[M].store(occ, std::memory_order_relaxed);
  }
  // every workgroup must be resident at once: the grid is the occupancy limit
  const int grid = w4a16_host::cu_count(dev) * occ;
  const ChainHeader* hp = static_cast<const ChainHeader*>(plan);
  unsigned* wp = static_cast<unsigned*>(workspace);
  int n_arg = count, g_arg = grid;
  void* args[] = {&hp, &wp, &n_arg, &g_arg};
  const int block = 64 * (chain_loader_waves(M) + chain_compute_waves(M));
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(block), args, 0,
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

extern "C" w4a16_status w4a16_chain_status(const void* workspace, size_t workspace_bytes, void* stream,
                                           uint32_t* bits, int32_t clear) {
  if (!workspace || !bits) return W4A16_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return W4A16_ERR_ALIGN;
  if (workspace_bytes < W4A16_CHAIN_WORKSPACE_BYTES) return W4A16_ERR_SIZE;
  *bits = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return W4A16_ERR_HIP;
  uint32_t word = 0;
  const uint8_t* at = static_cast<const uint8_t*>(workspace) + W4A16_CHAIN_ERROR_OFFSET;
  if (hipMemcpy(&word, at, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return W4A16_ERR_HIP;
  if (word && clear) {
    // the stream is drained, so no chain call of this workspace is running
    if (hipMemsetAsync(const_cast<void*>(workspace), 0, W4A16_CHAIN_WORKSPACE_BYTES, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return W4A16_ERR_HIP;
  }
  *bits = word;
  if (!word) return W4A16_OK;
  return (word & W4A16_CHAIN_ERR_WAIT) ? W4A16_ERR_WAIT : W4A16_ERR_FORMAT;
}
