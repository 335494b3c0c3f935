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
// How: every workgroup walks the whole list. Product i's 4-row tiles are
// spread over all workgroups; a workgroup's waves form teams of `wpr` waves,
// a team covering all of K for its tile (wpr = 1 for K <= 4096 at M = 1).
// Ordering between products is a device-wide counter in the caller's
// workspace: a workgroup adds 1 (release) after writing its part of product
// i, and before touching product i's x it waits (acquire) until the counter
// reaches i * gridDim.x, i.e. every workgroup has finished products 0..i-1.
// The first tile of product i is fetched BEFORE that wait: weights never
// depend on earlier results, so HBM keeps streaming across the ordering
// point. The wait spins a bounded number of times; if it gives up it flags
// the workspace and the workgroup stops computing but still counts in, so a
// starved launch ends instead of hanging. The last workgroup out resets the
// counters for the next call.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "w4a16.h"
#include "w4a16_device.h"
#include "w4a16_host.h"

using namespace w4a16_dev;

namespace {

constexpr uint32_t kChainMagic = 0x48433457u;  // "W4CH"
constexpr uint32_t kChainVersion = 2;
constexpr unsigned kSpinLimit = 1u << 20;      // polls before an ordering wait gives up (~1 s)
constexpr int kLeaves = 16;                    // leaf counters of the ordering tree
constexpr int kLineWords = 1024;               // 4 KiB between counters (separate memory pages)
constexpr int kXLdsBytes = 65536;              // LDS staging of one pass of x

// One workgroup per CU, with as many waves as the register budget of the
// instantiation allows per SIMD (x4 SIMDs).
constexpr int chain_waves(int M) { return 8; }
// groups per lane (the x slice stays within 32 VGPRs)
constexpr int chain_gpl(int M) { return M == 1 ? 2 : 1; }
// groups of x one pass can stage in LDS
constexpr int chain_lds_groups(int M) { return kXLdsBytes / (64 * M); }

struct ChainHeader {
  uint32_t magic, version;
  int32_t count, M, gpl, ww;
  int32_t pad[10];
};
static_assert(sizeof(ChainHeader) == 64, "plan header is 64 bytes");

struct ChainEntry {
  const u32x4* x;
  const u32x4* codes;
  const u32x4* sm;
  float* y;
  int32_t N, G, T, wpr, passes;
  int32_t pad[3];
};
static_assert(sizeof(ChainEntry) == 64, "plan entry is 64 bytes");

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

template <int M, int GPL, int WW>
__global__ void __launch_bounds__(64 * WW)
chain_kernel(const ChainHeader* __restrict__ hdr, unsigned* __restrict__ ws, int count) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwg = gridDim.x;
  if (hdr->magic != kChainMagic || hdr->version != kChainVersion || hdr->count != count || hdr->M != M ||
      hdr->gpl != GPL || hdr->ww != WW)
    return;  // every workgroup sees the same header, so all leave together
  const ChainEntry* __restrict__ ents = reinterpret_cast<const ChainEntry*>(hdr + 1);

  __shared__ u32x4 xl[kXLdsBytes / 16];                      // x of the current pass: [m][group][32 halfs]
  __shared__ float part[kTilesPerBlock][kTileRows][M][WW];  // [tile][row][m][wave]
  __shared__ int s_abort;

  // ordering tree: workgroup b reports to leaf b % leaves
  const int leaves = nwg < kLeaves ? nwg : kLeaves;
  const int leaf = int(blockIdx.x) % leaves;
  const unsigned leaf_size = unsigned((nwg - leaf + leaves - 1) / leaves);

  // product i as seen by this wave (all fields wave-uniform)
  struct Geo {
    const u32x4* x;
    const u32x4* codes;
    const u32x4* sm;
    float* y;
    int N, G, T, wpr, passes, pg, teams, team, wit, tpb, nblocks, rounds;
    bool direct;
  };
  auto geo = [&](int i) {
    const ChainEntry e = ents[i];
    Geo g;
    g.x = e.x;
    g.codes = e.codes;
    g.sm = e.sm;
    g.y = e.y;
    g.N = e.N;
    g.G = e.G;
    g.T = e.T;
    g.wpr = e.wpr;
    g.passes = e.passes;
    g.pg = g.wpr * 64 * GPL;  // groups per pass
    g.teams = WW / g.wpr;
    g.team = wave / g.wpr;
    g.wit = wave % g.wpr;
    g.direct = g.wpr == 1 && g.passes == 1;
    const int units = nwg * g.teams;
    const int tpb = g.direct ? 1 : g.T / units;
    g.tpb = tpb < 1 ? 1 : (tpb > kTilesPerBlock ? kTilesPerBlock : tpb);
    g.nblocks = (g.T + g.tpb - 1) / g.tpb;
    g.rounds = (g.nblocks + units - 1) / units;
    return g;
  };

  // an item is (product i, round k, pass c over K, tile tb of the block);
  // in round k team `team` of this workgroup owns block (k*nwg + wg)*teams + team
  struct Item {
    int i, k, c, tb;
  };
  auto next_item = [&](const Geo& g, Item it) {
    Item n = it;
    if (++n.tb < g.tpb) return n;
    n.tb = 0;
    if (++n.c < g.passes) return n;
    n.c = 0;
    if (++n.k < g.rounds) return n;
    n.k = 0;
    ++n.i;
    return n;
  };
  auto block_of = [&](const Geo& g, int k, int team) { return (k * nwg + int(blockIdx.x)) * g.teams + team; };
  // issue the loads of item `it`; a team with no tile in it (or `enable`
  // false) issues out-of-range buffer loads that cost no memory traffic, so
  // the fetch never sits behind a branch
  auto fetch = [&](const Geo& g, Item it, TileLoads<GPL>& L, bool enable) {
    const int b = block_of(g, it.k, g.team);
    const int t = b * g.tpb + it.tb;
    const bool valid = enable && b < g.nblocks && t < g.T;
    int g0[GPL];
#pragma unroll
    for (int j = 0; j < GPL; ++j) g0[j] = it.c * g.pg + (g.wit * GPL + j) * 64;
    fetch_tile_rsrc<GPL>(g.codes, g.sm, g.N, g.G, valid ? t : 0, g0, lane, valid, L);
  };

  u32x4 xv[M][GPL][4];
  float xs[M][GPL];
  bool aborted = false;
  int arrived = 0;
  int x_i = -1, x_c = -1;  // product and pass whose x is in registers

  // pass c of product g's activations: global -> LDS (coherent loads, since
  // an earlier product of this launch may have written them on another XCD),
  // then this wave's slice LDS -> VGPRs
  auto stage_x = [&](const Geo& g, int c) {
    const int g_first = c * g.pg;
    const int ng = min(g.pg, g.G - g_first);
    lds_barrier();  // every wave is done with the previous pass's LDS copy
    const int words = M * ng * 8;  // 8-byte words
    for (int w = threadIdx.x; w < words; w += blockDim.x) {
      const int m = w / (ng * 8);
      const int r = w - m * ng * 8;  // word within row m's slice
      const unsigned long long* src =
          reinterpret_cast<const unsigned long long*>(g.x + (size_t(m) * g.G + g_first) * 4) + r;
      const unsigned long long v = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      reinterpret_cast<unsigned long long*>(xl)[size_t(m) * g.pg * 8 + r] = v;
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int gl = (g.wit * GPL + j) * 64 + lane;  // group within the pass
#pragma unroll
      for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[m][j][q] = u32x4{0, 0, 0, 0};
        if (gl < ng) {
#pragma unroll
          for (int q = 0; q < 4; ++q) xv[m][j][q] = xl[(size_t(m) * g.pg + gl) * 4 + q];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int j = 0; j < GPL; ++j) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s = dot2(elem(xv[m][j][q], e), kOnes, s);
        }
        xs[m][j] = s;
      }
    }
  };

  // this workgroup's results of product i are written: report to the tree;
  // the last report of a leaf climbs to the top, the last at the top raises
  // every leaf's flag to i+1. Called before the next tile is fetched, so the
  // atomics' returns do not wait behind that prefetch (vmcnt is in order).
  auto arrive = [&](int i) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's coherent y stores are complete
    __builtin_amdgcn_s_barrier();   // ... and every other wave's
    if (threadIdx.x == 0) {
      const unsigned old = add_coherent(ws + leaf_word(leaf), 1u);
      if (old == unsigned(i + 1) * leaf_size - 1u) {
        const unsigned top = add_coherent(ws + kTopWord, 1u);
        if (top == unsigned(i + 1) * unsigned(leaves) - 1u)
          for (int l = 0; l < leaves; ++l) st_coherent(ws + flag_word(l), unsigned(i + 1));
      }
    }
    ++arrived;
  };
  // wait until products 0..i-1 are complete everywhere
  auto wait_for = [&](int i) {
    if (threadIdx.x == 0) {
      unsigned spins = 0;
      int ab = 0;
      while (ld_coherent(ws + flag_word(leaf)) < unsigned(i)) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          ab = 1;
          add_coherent(ws + kErrorWord, 1u);
          break;
        }
      }
      s_abort = ab;
    }
    lds_barrier();
    aborted = s_abort != 0;
  };

  auto finish = [&](const Geo& g, Item it, const TileLoads<GPL>& L) {
    if (it.tb == 0 && (it.i != x_i || it.c != x_c)) {  // this (product, pass) needs its x
      if (it.k == 0 && it.c == 0 && it.i > 0) wait_for(it.i);
      if (!aborted) stage_x(g, it.c);
      x_i = it.i;
      x_c = it.c;
    }
    const int b = block_of(g, it.k, g.team);
    const int t = b * g.tpb + it.tb;
    if (!aborted && b < g.nblocks && t < g.T) {
      float acc[kTileRows][M];
      compute_tile<M, GPL>(L, xv, xs, acc);
      if (g.direct) {
        store_tile<M, true>(acc, g.y, g.N, t, lane);
      } else if (lane == 0) {
#pragma unroll
        for (int r = 0; r < kTileRows; ++r)
#pragma unroll
          for (int m = 0; m < M; ++m)
            part[it.tb][r][m][wave] = (it.c == 0 ? 0.f : part[it.tb][r][m][wave]) + acc[r][m];
      }
    }
    if (!g.direct && it.c == g.passes - 1 && it.tb == g.tpb - 1) {  // block done: combine each team's waves
      lds_barrier();
      if (!aborted) {
        const int per_team = g.tpb * kTileRows * M;
        for (int idx = threadIdx.x; idx < g.teams * per_team; idx += blockDim.x) {
          const int m = idx % M;
          const int r = (idx / M) % kTileRows;
          const int tb = (idx / (M * kTileRows)) % g.tpb;
          const int team = idx / per_team;
          const int bb = block_of(g, it.k, team);
          const int tt = bb * g.tpb + tb;
          const int n = tt * kTileRows + r;
          if (bb < g.nblocks && tt < g.T && n < g.N) {
            float s = 0.f;
            for (int w = 0; w < g.wpr; ++w) s += part[tb][r][m][team * g.wpr + w];
            store_y<true>(g.y + size_t(m) * g.N + n, s);
          }
        }
      }
      lds_barrier();  // partials read before the next block writes them
    }
  };

  // Two load buffers used alternately: the next item's tile is in flight
  // while the current one is computed. Inside a product the next fetch is
  // issued first; at a product's last item the results are written and
  // reported first, then the next product's first tile is fetched, and only
  // then (at that product's first item) does the workgroup wait for the
  // others, with the tile in flight. Every fetch is unconditional: a fetch
  // behind a branch makes the compiler merge buffer contents with register
  // moves that wait for the loads in flight.
  Item ia{0, 0, 0, 0};
  Geo ga = geo(0);
  if constexpr (double_buffered(M)) {
    TileLoads<GPL> la, lb;
    fetch(ga, ia, la, true);
    while (true) {
      const Item ib = next_item(ga, ia);
      const bool more_b = ib.i < count;
      const bool edge_b = ib.i != ia.i;
      const Geo gb = (edge_b && more_b) ? geo(ib.i) : ga;
      if (!edge_b) {
        fetch(gb, ib, lb, true);
        __builtin_amdgcn_sched_barrier(0);
        finish(ga, ia, la);
      } else {
        finish(ga, ia, la);
        arrive(ia.i);
        fetch(gb, ib, lb, more_b);
      }
      if (!more_b || aborted) break;

      const Item ic = next_item(gb, ib);
      const bool more_c = ic.i < count;
      const bool edge_c = ic.i != ib.i;
      const Geo gc = (edge_c && more_c) ? geo(ic.i) : gb;
      if (!edge_c) {
        fetch(gc, ic, la, true);
        __builtin_amdgcn_sched_barrier(0);
        finish(gb, ib, lb);
      } else {
        finish(gb, ib, lb);
        arrive(ib.i);
        fetch(gc, ic, la, more_c);
      }
      if (!more_c || aborted) break;
      ia = ic;
      ga = gc;
    }
  } else {
    // more activation rows: VALU bound, registers go to the x slices
    while (true) {
      TileLoads<GPL> la;
      fetch(ga, ia, la, true);
      const Item ib = next_item(ga, ia);
      finish(ga, ia, la);
      if (ib.i != ia.i) arrive(ia.i);
      if (ib.i >= count || aborted) break;
      if (ib.i != ia.i) ga = geo(ib.i);
      ia = ib;
    }
  }

  // Count out. After an abort, first release every waiter (results of this
  // call are then invalid and the error word says so). The last workgroup
  // out resets every counter and flag for the next call.
  __syncthreads();
  if (threadIdx.x == 0) {
    if (arrived < count)
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

typedef void (*chain_fn)(const ChainHeader*, unsigned*, int);

template <int M>
constexpr chain_fn chain_instance() {
  return &chain_kernel<M, chain_gpl(M), chain_waves(M)>;
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

// waves per team for a product of G groups: the fewest that divide the
// workgroup and cover K in one pass, within the LDS staging limit; otherwise
// the widest such team and several passes
void team_shape(int M, int G, int* wpr_out, int* passes_out) {
  const int ww = chain_waves(M), gpl = chain_gpl(M), cap = chain_lds_groups(M);
  int best = 0;
  for (int w = 1; w <= ww; ++w) {
    if (ww % w || w * 64 * gpl > cap) continue;
    best = w;
    if (w * 64 * gpl >= G) break;
  }
  *wpr_out = best;
  *passes_out = (G + best * 64 * gpl - 1) / (best * 64 * gpl);
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
  const int gpl = chain_gpl(M);
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
  h.gpl = gpl;
  h.ww = chain_waves(M);
  uint8_t* out = static_cast<uint8_t*>(plan);
  std::memcpy(out, &h, sizeof(h));
  for (int32_t i = 0; i < count; ++i) {
    const w4a16_chain_entry& e = entries[i];
    const int G = e.K / kGroup;
    int wpr = 0, passes = 0;
    team_shape(M, G, &wpr, &passes);
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
    c.wpr = wpr;
    c.passes = passes;
    std::memcpy(out + sizeof(ChainHeader) + size_t(i) * sizeof(ChainEntry), &c, sizeof(c));
  }
  return W4A16_OK;
}

extern "C" w4a16_status w4a16_chain_launch_shape(int32_t M, int32_t out[3]) {
  if (!out) return W4A16_ERR_NULL;
  if (M < 1 || M > kMaxM) return W4A16_ERR_SHAPE;
  out[0] = M;
  out[1] = chain_gpl(M);
  out[2] = chain_waves(M);
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
    occ = w4a16_host::occupancy_of(reinterpret_cast<const void*>(fn), 64 * chain_waves(M));
    g_chain_occupancy[M].store(occ, std::memory_order_relaxed);
  }
  if (const int o = w4a16_host::tune("W4A16_TUNE_CHAIN_OCC")) occ = o < occ ? o : occ;  // sweep builds only
  // every workgroup must be resident at once: the grid is the occupancy limit
  const int grid = w4a16_host::cu_count(dev) * occ;
  const ChainHeader* hp = static_cast<const ChainHeader*>(plan);
  unsigned* wp = static_cast<unsigned*>(workspace);
  int n_arg = count;
  void* args[] = {&hp, &wp, &n_arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(64 * chain_waves(M)), args, 0,
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
