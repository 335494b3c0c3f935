// gfx950 (CDNA4) kernels and C-ABI entry point of the W4A16 decode GEMV.
//
// y[m][n] = sum_k (scale[n][k/32] * q[n][k] + min[n][k/32]) * x[m][k]
//
// Decode on the edge is bandwidth bound (Magnitude page, section 3.4; core-
// modules page, section 5.4), and the same holds for a decode-step GEMV on an
// MI355X: 0.625 bytes of weight per multiply-add pair at M = 1. The kernel is
// therefore a streaming kernel, not a contraction: no MFMA (M <= 8 rows of
// activations are far too few for a matrix-core tile to pay), every weight
// byte is loaded once with a 128-bit non-temporal load, and the VALU work per
// weight is kept to about 0.6 bitwise ops + M/2 packed dot products.
//
// Work decomposition
//   * a lane owns GPL groups of 32 k along K (group g = (wave*GPL + j)*64 +
//     lane) and keeps that slice of every activation row in VGPRs for the
//     whole kernel, so x is read from memory once per workgroup;
//   * the W waves of a workgroup together cover all G = K/32 groups;
//   * a workgroup walks 4-row tiles t = blockIdx.x, blockIdx.x + gridDim.x, ...
//     For each tile a lane issues 4*GPL code loads and GPL scale/min loads
//     (each 16 B, lane-contiguous, so one wave instruction moves 1 KiB);
//   * per group a lane computes sum_k q*x with v_dot2c_f32_f16 on binary16
//     *subnormal* pairs: AND-ing a packed word with 0x000F000F gives two halfs
//     whose bit patterns are the codes, i.e. the values q * 2^-24, and with
//     0x00F000F0 the values q * 2^-20. Both are exact, the products with x are
//     exact in fp32, and no offset has to be cancelled later, so an all-zero
//     weight row gives exactly zero. The group result is folded in fp32 as
//     scale * 2^20 * (16*lo + hi) + min * sum_{k in g} x[k];
//   * lane partials are summed across the wave with DPP and lane shuffles,
//     across waves through LDS, in a fixed order: results are bitwise
//     repeatable, no atomics are used and y is overwritten.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "w4a16.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 32;
constexpr int kTileRows = 4;
constexpr int kMaxWaves = 16;
constexpr int kMaxM = 8;
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Waves per workgroup an instantiation may use: its VGPR estimate must fit
// the 512-entry register file shared by the waves on one SIMD.
__host__ __device__ constexpr int max_waves(int M, int GPL) {
  return (16 * M * GPL + 20 * GPL + 6 * M + 30) <= 128 ? 16 : 8;
}

// Tiles of 4 rows handled between two workgroup barriers when partial sums
// go through LDS.
constexpr int kTilesPerBlock = 8;

template <int M, int GPL>
__global__ void __launch_bounds__(64 * max_waves(M, GPL))
gemv_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ codes,
            const u32x4* __restrict__ sm, float* __restrict__ y, int N, int G, int T, int nchunks) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int chunk_groups = nwaves * 64 * GPL;  // groups covered by one pass over K
  const bool direct = (nwaves == 1 && nchunks == 1);
  const int nblocks = direct ? T : (T + kTilesPerBlock - 1) / kTilesPerBlock;
  const int tpb = direct ? 1 : kTilesPerBlock;

  uint32_t xr[M][GPL][16];
  float xs[M][GPL];
  int grp[GPL];
  bool ok[GPL];

  // this lane's slice of chunk c of every activation row, plus its group sums
  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      grp[j] = c * chunk_groups + (wave * GPL + j) * 64 + lane;
      ok[j] = grp[j] < G;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int j = 0; j < GPL; ++j) {
        u32x4 v[4] = {};
        if (ok[j]) {
          const u32x4* p = x + (size_t(m) * G + grp[j]) * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = p[q];
        }
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xr[m][j][4 * q + e] = elem(v[q], e);
            s = dot2(elem(v[q], e), kOnes, s);
          }
        }
        xs[m][j] = s;
      }
    }
  };

  // partial row sums of one tile over this lane's groups of the current chunk
  auto tile = [&](int t, float (&acc)[kTileRows][M]) {
    u32x4 s4[GPL];
    u32x4 c4[kTileRows][GPL];
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      s4[j] = u32x4{0, 0, 0, 0};
      if (ok[j]) s4[j] = __builtin_nontemporal_load(sm + size_t(t) * G + grp[j]);
    }
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const int n = t * kTileRows + r;
#pragma unroll
      for (int j = 0; j < GPL; ++j) {
        c4[r][j] = u32x4{0, 0, 0, 0};
        if (ok[j] && n < N) c4[r][j] = __builtin_nontemporal_load(codes + size_t(n) * G + grp[j]);
      }
    }
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
#pragma unroll
      for (int j = 0; j < GPL; ++j) {
        float lo[M], hi[M];
#pragma unroll
        for (int m = 0; m < M; ++m) lo[m] = hi[m] = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t w = elem(c4[r][j], d);
          const uint32_t w8 = w >> 8;
          const uint32_t pa = w & 0x000F000Fu;   // k = 8d+0, 8d+1  -> q * 2^-24
          const uint32_t pb = w & 0x00F000F0u;   // k = 8d+2, 8d+3  -> q * 2^-20
          const uint32_t pc = w8 & 0x000F000Fu;  // k = 8d+4, 8d+5  -> q * 2^-24
          const uint32_t pd = w8 & 0x00F000F0u;  // k = 8d+6, 8d+7  -> q * 2^-20
#pragma unroll
          for (int m = 0; m < M; ++m) {
            lo[m] = dot2(pa, xr[m][j][4 * d + 0], lo[m]);
            hi[m] = dot2(pb, xr[m][j][4 * d + 1], hi[m]);
            lo[m] = dot2(pc, xr[m][j][4 * d + 2], lo[m]);
            hi[m] = dot2(pd, xr[m][j][4 * d + 3], hi[m]);
          }
        }
        const f16x2 h = __builtin_bit_cast(f16x2, elem(s4[j], r));
        const float sc = float(h[0]) * 0x1p20f;
        const float mn = float(h[1]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          acc[r][m] = __builtin_fmaf(sc, __builtin_fmaf(lo[m], 16.f, hi[m]), acc[r][m]);
          acc[r][m] = __builtin_fmaf(mn, xs[m][j], acc[r][m]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = wave_sum(acc[r][m]);
    }
  };

  // per-wave partials of one block of tiles: [tile][row][m][wave]
  __shared__ float part[kTilesPerBlock][kTileRows][M][kMaxWaves];

  if (nchunks == 1) load_x(0);
  for (int b = blockIdx.x; b < nblocks; b += gridDim.x) {
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) load_x(c);
      for (int tb = 0; tb < tpb; ++tb) {
        const int t = b * tpb + tb;
        if (t >= T) break;
        float acc[kTileRows][M];
        tile(t, acc);
        if (direct) {
          float v = 0.f;
#pragma unroll
          for (int i = 0; i < kTileRows * M; ++i)
            if (lane == i) v = acc[i / M][i % M];
          if (lane < kTileRows * M) {
            const int n = t * kTileRows + lane / M;
            if (n < N) y[size_t(lane % M) * N + n] = v;
          }
        } else if (lane == 0) {
#pragma unroll
          for (int r = 0; r < kTileRows; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m)
              part[tb][r][m][wave] = (c == 0 ? 0.f : part[tb][r][m][wave]) + acc[r][m];
        }
      }
    }
    if (!direct) {
      __syncthreads();
      for (int i = threadIdx.x; i < tpb * kTileRows * M; i += blockDim.x) {
        const int tb = i / (kTileRows * M);
        const int r = (i / M) % kTileRows;
        const int m = i % M;
        const int n = (b * tpb + tb) * kTileRows + r;
        if (n < N) {
          float s = 0.f;
          for (int w = 0; w < nwaves; ++w) s += part[tb][r][m][w];
          y[size_t(m) * N + n] = s;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// host side: instantiation table, launch-shape choice, validation
// ---------------------------------------------------------------------------

typedef void (*kernel_fn)(const u32x4*, const u32x4*, const u32x4*, float*, int, int, int, int);

constexpr int kGplOptions[] = {1, 2, 4};
constexpr int kNumGpl = 3;
constexpr int32_t kMaxK = 1 << 20;

// the x slice of one lane stays within 64 VGPRs (one group per lane always allowed)
constexpr bool gpl_allowed(int M, int gpl) { return 16 * M * gpl <= 64 || gpl == 1; }

template <int M, int GPL>
constexpr kernel_fn instance() {
  if constexpr (gpl_allowed(M, GPL)) return &gemv_kernel<M, GPL>;
  return nullptr;
}

template <int M>
constexpr kernel_fn pick(int gi) {
  return gi == 0 ? instance<M, 1>() : gi == 1 ? instance<M, 2>() : instance<M, 4>();
}

kernel_fn kernel_for(int M, int gi) {
  switch (M) {
    case 1: return pick<1>(gi);
    case 2: return pick<2>(gi);
    case 3: return pick<3>(gi);
    case 4: return pick<4>(gi);
    case 5: return pick<5>(gi);
    case 6: return pick<6>(gi);
    case 7: return pick<7>(gi);
    case 8: return pick<8>(gi);
    default: return nullptr;
  }
}

struct LaunchShape {
  int gi;       // index into kGplOptions
  int waves;    // waves per workgroup
  int nchunks;  // passes over K
};

// Fewest passes over K; then avoid leaving more than a quarter of the lanes
// idle; then the fewest waves per workgroup; then the fewest idle lanes.
LaunchShape choose_shape(int M, int G) {
  LaunchShape best{-1, 0, 0};
  long best_key[4] = {0, 0, 0, 0};
  for (int gi = kNumGpl - 1; gi >= 0; --gi) {
    const int gpl = kGplOptions[gi];
    if (!gpl_allowed(M, gpl)) continue;
    const int wmax = max_waves(M, gpl);
    const int nchunks = (G + wmax * 64 * gpl - 1) / (wmax * 64 * gpl);
    const int waves = (G + nchunks * 64 * gpl - 1) / (nchunks * 64 * gpl);
    const long slots = long(nchunks) * waves * 64 * gpl;
    const long idle = slots - G;
    const long key[4] = {nchunks, 4 * idle > slots ? 1 : 0, waves, idle};
    bool better = best.gi < 0;
    for (int i = 0; i < 4 && !better; ++i) {
      if (key[i] < best_key[i]) better = true;
      if (key[i] > best_key[i]) break;
    }
    if (better) {
      best = LaunchShape{gi, waves, nchunks};
      for (int i = 0; i < 4; ++i) best_key[i] = key[i];
    }
  }
  return best;
}

// per-device cache of the compute-unit count (0 = not yet queried)
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int c = g_cu_count[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
  g_cu_count[dev].store(c, std::memory_order_relaxed);
  return c;
}

bool ranges_overlap(uintptr_t a, size_t na, uintptr_t b, size_t nb) { return a < b + nb && b < a + na; }

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

extern "C" w4a16_status w4a16_gemv(const void* x, const void* packed, float* y, int32_t M, int32_t N,
                                   int32_t K, void* stream) {
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
  const LaunchShape shape = choose_shape(M, G);
  if (shape.gi < 0) return W4A16_ERR_SHAPE;
  kernel_fn fn = kernel_for(M, shape.gi);

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  const int T = (N + kTileRows - 1) / kTileRows;
  const bool direct = shape.waves == 1 && shape.nchunks == 1;
  const int units = direct ? T : (T + kTilesPerBlock - 1) / kTilesPerBlock;
  const int cus = cu_count(dev);
  // several workgroups per CU, each walking an equal share of the work units
  const int waves_per_cu_target = 16;
  const int max_grid = cus * ((waves_per_cu_target + shape.waves - 1) / shape.waves);
  const int per = (units + max_grid - 1) / max_grid;
  const int grid = (units + per - 1) / per;

  const size_t codes_region = (size_t(N) * size_t(K) / 2 + 255) / 256 * 256;
  const u32x4* xp = static_cast<const u32x4*>(x);
  const u32x4* cp = static_cast<const u32x4*>(packed);
  const u32x4* sp = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(packed) + codes_region);
  int n_arg = N, g_arg = G, t_arg = T, c_arg = shape.nchunks;
  void* args[] = {&xp, &cp, &sp, &y, &n_arg, &g_arg, &t_arg, &c_arg};
  if (hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(64 * shape.waves), args, 0,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}
