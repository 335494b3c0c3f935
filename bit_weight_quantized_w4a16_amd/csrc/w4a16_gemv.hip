// gfx950 (CDNA4) kernel and C-ABI entry point of one W4A16 decode GEMV.
//
// y[m][n] = sum_k (scale[n][k/32] * q[n][k] + min[n][k/32]) * x[m][k]
//
// Decode on the edge is bandwidth bound (Magnitude page, section 3.4; core-
// modules page, section 5.4), and the same holds for a decode-step GEMV on an
// MI355X: 0.625 bytes of weight per multiply-add pair at M = 1. The kernel is
// therefore a streaming kernel, not a contraction: no MFMA (M <= 8 rows of
// activations are far too few for a matrix-core tile to pay), every weight
// byte is loaded once with a 128-bit non-temporal load, and the VALU work per
// weight is about 0.6 bitwise ops + M/2 packed dot products.
//
// Work decomposition
//   * a lane owns GPL groups of 32 k along K (group g = (wave*GPL + j)*64 +
//     lane within one pass over K) and keeps that slice of every activation
//     row in VGPRs, so x is read from memory once per workgroup and pass;
//   * the W waves of a workgroup cover W*64*GPL groups per pass; K longer
//     than that takes several passes, the partial sums carried in LDS;
//   * a workgroup walks 4-row tiles; for each tile a lane issues 4*GPL code
//     loads and GPL scale/min loads, each 16 B and lane-contiguous, so one
//     wave instruction moves 1 KiB. The loads of the next tile are issued
//     before the current tile is computed, and the first tile's loads go out
//     before x is fetched, so the two start-up latencies overlap;
//   * lane partials are summed across the wave with DPP and lane shuffles,
//     across waves through LDS, in a fixed order: results are bitwise
//     repeatable, no atomics are used and y is overwritten.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "w4a16.h"
#include "w4a16_device.h"
#include "w4a16_host.h"

using namespace w4a16_dev;

namespace {

// Waves per workgroup an instantiation may use: its VGPR estimate (x slice,
// tile loads in flight, accumulators) must fit the 512-entry register file
// shared by the waves on one SIMD.
__host__ __device__ constexpr int max_waves(int M, int GPL) {
  return (16 * M * GPL + (double_buffered(M) ? 40 : 20) * GPL + 6 * M + 30) <= 128 ? 16 : 8;
}

// Launch modes of one GEMV.
//   kDirect: one wave covers all of K for its tile and stores the results;
//   kBlock:  the waves of a workgroup split K; per-wave partials of a block
//            of tiles are combined through LDS;
//   kMulti:  K also takes several passes of the workgroup (x re-fetched per
//            pass, partials carried in LDS).
constexpr int kDirect = 0, kBlock = 1, kMulti = 2;

template <int M, int GPL, int MODE>
__global__ void __launch_bounds__(64 * max_waves(M, GPL))
gemv_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ codes, const u32x4* __restrict__ sm,
            float* __restrict__ y, int N, int G, int T, int nchunks, int tpb) {
  const int lane = threadIdx.x & 63;
  // wave-uniform values kept in scalar registers, so every load address is a
  // scalar base plus the one per-lane offset `lane`
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int chunk_groups = nwaves * 64 * GPL;  // groups covered by one pass over K
  const int nblocks = (T + tpb - 1) / tpb;
  if (int(blockIdx.x) >= nblocks) return;

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
    for (int i = threadIdx.x; i < ntiles * kTileRows * M; i += blockDim.x) {
      const int ti = i / (kTileRows * M);
      const int r = (i / M) % kTileRows;
      const int m = i % M;
      const int n = (b * tpb + ti) * kTileRows + r;
      if (n < N) {
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += part[ti][r][m][w];
        y[size_t(m) * N + n] = s;
      }
    }
    __syncthreads();
  };

  if constexpr (MODE == kMulti) {
    // passes over K outermost within a block: x of pass c is fetched once at
    // the top of the pass and stays in registers for the block's tiles
    for (int b = blockIdx.x; b < nblocks; b += gridDim.x) {
      const int ntiles = min(tpb, T - b * tpb);
      for (int c = 0; c < nchunks; ++c) {
        fetch_x(c);
        int g0[GPL];
        bases(c, g0);
        for (int tb = 0; tb < ntiles; ++tb) {
          TileLoads<GPL> la;
          fetch_tile<GPL>(codes, sm, N, G, b * tpb + tb, g0, lane, la);
          float acc[kTileRows][M];
          compute_tile<M, GPL>(la, RegX<M, GPL>{xv, xs}, acc);
          if (lane == 0) {
#pragma unroll
            for (int r = 0; r < kTileRows; ++r)
#pragma unroll
              for (int m = 0; m < M; ++m) part[tb][r][m][wave] = (c == 0 ? 0.f : part[tb][r][m][wave]) + acc[r][m];
          }
        }
      }
      reduce_block(b);
    }
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
    const int my_blocks = (nblocks - int(blockIdx.x) + int(gridDim.x) - 1) / int(gridDim.x);
    const int n_items = my_blocks * tpb;
    int g0[GPL];
    bases(0, g0);
    auto tile_of = [&](int e) { return (int(blockIdx.x) + (e / tpb) * int(gridDim.x)) * tpb + e % tpb; };
    auto fetch = [&](int e, TileLoads<GPL>& L) {
      const int t = tile_of(e);
      fetch_tile<GPL>(codes, sm, N, G, t < T ? t : T - 1, g0, lane, L);
    };
    auto finish = [&](const TileLoads<GPL>& L, int e) {
      const int t = tile_of(e);
      if (t < T) {
        float acc[kTileRows][M];
        compute_tile<M, GPL>(L, RegX<M, GPL>{xv, xs}, acc);
        if constexpr (MODE == kDirect) {
          store_tile<M>(acc, y, N, t, lane);
        } else if (lane == 0) {
          const int tb = e % tpb;
#pragma unroll
          for (int r = 0; r < kTileRows; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) part[tb][r][m][wave] = acc[r][m];
        }
      }
      if constexpr (MODE == kBlock) {
        if (e % tpb == tpb - 1) reduce_block(int(blockIdx.x) + (e / tpb) * int(gridDim.x));
      }
    };

    TileLoads<GPL> la, lb;
    fetch(0, la);
    fetch_x(0);  // after the first tile's loads, so both latencies overlap
    int e = 0;
    if constexpr (double_buffered(M)) {
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
  }
}

// ---------------------------------------------------------------------------
// host side: instantiation table, launch-shape choice, validation
// ---------------------------------------------------------------------------

typedef void (*kernel_fn)(const u32x4*, const u32x4*, const u32x4*, float*, int, int, int, int, int);

constexpr int kGplOptions[] = {1, 2, 4};
constexpr int kNumGpl = 3;
constexpr int32_t kMaxK = 1 << 20;

// the x slice of one lane stays within 32 VGPRs (one group per lane always allowed)
constexpr bool gpl_allowed(int M, int gpl) { return 16 * M * gpl <= 32 || gpl == 1; }

template <int M, int GPL, int MODE>
constexpr kernel_fn instance() {
  if constexpr (gpl_allowed(M, GPL)) return &gemv_kernel<M, GPL, MODE>;
  return nullptr;
}

template <int M, int MODE>
constexpr kernel_fn pick(int gi) {
  return gi == 0 ? instance<M, 1, MODE>() : gi == 1 ? instance<M, 2, MODE>() : instance<M, 4, MODE>();
}

template <int MODE>
kernel_fn kernel_for(int M, int gi) {
  switch (M) {
    case 1: return pick<1, MODE>(gi);
    case 2: return pick<2, MODE>(gi);
    case 3: return pick<3, MODE>(gi);
    case 4: return pick<4, MODE>(gi);
    case 5: return pick<5, MODE>(gi);
    case 6: return pick<6, MODE>(gi);
    case 7: return pick<7, MODE>(gi);
    case 8: return pick<8, MODE>(gi);
    default: return nullptr;
  }
}

int mode_of(int waves, int nchunks) { return nchunks > 1 ? kMulti : waves > 1 ? kBlock : kDirect; }

kernel_fn kernel_for_mode(int mode, int M, int gi) {
  return mode == kMulti ? kernel_for<kMulti>(M, gi) : mode == kBlock ? kernel_for<kBlock>(M, gi)
                                                                      : kernel_for<kDirect>(M, gi);
}

struct LaunchShape {
  int gi;       // index into kGplOptions
  int waves;    // waves per workgroup
  int nchunks;  // passes over K
};

LaunchShape shape_for_gpl(int M, int G, int gi) {
  const int gpl = kGplOptions[gi];
  const int wmax = max_waves(M, gpl);
  const int nchunks = (G + wmax * 64 * gpl - 1) / (wmax * 64 * gpl);
  const int waves = (G + nchunks * 64 * gpl - 1) / (nchunks * 64 * gpl);
  return LaunchShape{gi, waves, nchunks};
}

// Fewest passes over K; then avoid leaving more than a quarter of the lanes
// idle; then, at M = 1, one group per lane (a tile's K split over more waves:
// each wave loads less of x and more waves share the streaming; measured
// faster on every decode-step shape); then the fewest waves per workgroup;
// then the fewest idle lanes.
LaunchShape choose_shape(int M, int G) {
  LaunchShape best{-1, 0, 0};
  long best_key[5] = {0, 0, 0, 0, 0};
  for (int gi = kNumGpl - 1; gi >= 0; --gi) {
    if (!gpl_allowed(M, kGplOptions[gi])) continue;
    const LaunchShape s = shape_for_gpl(M, G, gi);
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

// Resident workgroups per CU of one instantiation at one block size (cached;
// 0 = not yet queried). Every device the library drives is a gfx950, so the
// answer does not depend on the device.
std::atomic<int> g_occupancy[kMaxM + 1][kNumGpl][3][kMaxWaves + 1];

int occupancy(int M, int gi, int mode, int waves, kernel_fn fn) {
  std::atomic<int>& slot = g_occupancy[M][gi][mode][waves];
  int v = slot.load(std::memory_order_relaxed);
  if (v > 0) return v;
  v = w4a16_host::occupancy_of(reinterpret_cast<const void*>(fn), 64 * waves);
  slot.store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

extern "C" int32_t w4a16_max_k(int32_t M) {
  if (M < 1 || M > kMaxM) return 0;
  return kMaxK;
}

extern "C" w4a16_status w4a16_launch_shape(int32_t M, int32_t N, int32_t K, int32_t out[3]) {
  if (!out) return W4A16_ERR_NULL;
  if (M < 1 || M > kMaxM || N < 1 || K < kGroup || K % kGroup || K > w4a16_max_k(M) ||
      w4a16_packed_bytes(N, K) == 0)
    return W4A16_ERR_SHAPE;
  const LaunchShape shape = choose_shape(M, K / kGroup);
  if (shape.gi < 0) return W4A16_ERR_SHAPE;
  out[0] = kGplOptions[shape.gi];
  out[1] = shape.waves;
  out[2] = shape.nchunks;
  return W4A16_OK;
}

namespace {

// Both entry points: validate, choose the launch and enqueue; with events,
// they take the kernel's own start and end times.
w4a16_status gemv_enqueue(const void* x, const void* packed, float* y, int32_t M, int32_t N, int32_t K,
                          void* stream, hipEvent_t start, hipEvent_t stop) {
  using w4a16_host::ranges_overlap;
  using w4a16_host::tune;
  if (!x || !packed || !y) return W4A16_ERR_NULL;
  if (M < 1 || M > kMaxM || N < 1 || K < kGroup || K % kGroup || K > w4a16_max_k(M)) return W4A16_ERR_SHAPE;
  const size_t packed_bytes = w4a16_packed_bytes(N, K);
  if (packed_bytes == 0) return W4A16_ERR_SHAPE;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  const uintptr_t pa = reinterpret_cast<uintptr_t>(packed);
  const uintptr_t ya = reinterpret_cast<uintptr_t>(y);
  if (xa % 16 || pa % 256 || ya % 4) return W4A16_ERR_ALIGN;
  const size_t ybytes = size_t(M) * size_t(N) * sizeof(float);
  if (ranges_overlap(ya, ybytes, xa, size_t(M) * size_t(K) * 2) || ranges_overlap(ya, ybytes, pa, packed_bytes))
    return W4A16_ERR_OVERLAP;

  const int G = K / kGroup;
  LaunchShape shape = choose_shape(M, G);
  if (const int g = tune("W4A16_TUNE_GPL")) {  // sweep builds only
    for (int gi = 0; gi < kNumGpl; ++gi)
      if (kGplOptions[gi] == g && gpl_allowed(M, g)) shape = shape_for_gpl(M, G, gi);
  }
  if (shape.gi < 0) return W4A16_ERR_SHAPE;
  const int mode = mode_of(shape.waves, shape.nchunks);
  kernel_fn fn = kernel_for_mode(mode, M, shape.gi);

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  const int T = (N + kTileRows - 1) / kTileRows;
  const bool direct = mode == kDirect;
  // all workgroups resident at once, each walking an equal share of the tiles
  int occ = occupancy(M, shape.gi, mode, shape.waves, fn);
  if (const int o = tune("W4A16_TUNE_OCC")) occ = o < occ ? o : occ;
  const int max_grid = w4a16_host::cu_count(dev) * occ;
  // tiles per block: a workgroup reads its x slices once per block, so wide
  // workgroups (long K split over four or more waves, a large x) take enough
  // tiles per block for about one workgroup per CU; narrower ones fill the
  // resident slots first
  int tpb = direct ? 1 : shape.waves >= 4 ? T / w4a16_host::cu_count(dev) : T / max_grid;
  tpb = tpb < 1 ? 1 : tpb > kTilesPerBlock ? kTilesPerBlock : tpb;
  if (const int v = tune("W4A16_TUNE_TPB")) tpb = v > kTilesPerBlock ? kTilesPerBlock : v;
  const int units = (T + tpb - 1) / tpb;
  const int grid = units < max_grid ? units : max_grid;

  const size_t codes_region = (size_t(N) * size_t(K) / 2 + 255) / 256 * 256;
  const u32x4* xp = static_cast<const u32x4*>(x);
  const u32x4* cp = static_cast<const u32x4*>(packed);
  const u32x4* sp = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(packed) + codes_region);
  int n_arg = N, g_arg = G, t_arg = T, c_arg = shape.nchunks, b_arg = tpb;
  void* args[] = {&xp, &cp, &sp, &y, &n_arg, &g_arg, &t_arg, &c_arg, &b_arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(64 * shape.waves), args, 0,
                         static_cast<hipStream_t>(stream), start, stop, 0) != hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}

}  // namespace

extern "C" w4a16_status w4a16_gemv(const void* x, const void* packed, float* y, int32_t M, int32_t N,
                                   int32_t K, void* stream) {
  return gemv_enqueue(x, packed, y, M, N, K, stream, nullptr, nullptr);
}

extern "C" w4a16_status w4a16_gemv_timed(const void* x, const void* packed, float* y, int32_t M, int32_t N,
                                         int32_t K, void* stream, void* start_event, void* stop_event) {
  if (!start_event || !stop_event) return W4A16_ERR_NULL;
  return gemv_enqueue(x, packed, y, M, N, K, stream, static_cast<hipEvent_t>(start_event),
                      static_cast<hipEvent_t>(stop_event));
}
