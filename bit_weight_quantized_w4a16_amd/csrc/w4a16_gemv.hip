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
#include "w4a16_skeleton.h"

using namespace w4a16_dev;

namespace {

using w4a16_host::LaunchShape;
using w4a16_host::gpl_allowed;
using w4a16_host::kGplOptions;
using w4a16_host::kNumGpl;

// Launches of this module whose blob header did not match their call, one
// word per device (each device holds its own copy; host code reaches it only
// through the address hipGetSymbolAddress returns for that device).
__device__ unsigned blob_mismatch_count;

// The 4-bit group-affine GEMV: the shared skeleton with the device header's
// tile loads and dot products.
template <int M, int GPL, int MODE>
__global__ void __launch_bounds__(64 * max_waves_of<CodecQ4>(M, GPL))
gemv_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ codes, const u32x4* __restrict__ sm,
            float* __restrict__ y, int N, int G, int T, int nchunks, int tpb_grid, int nwaves) {
  gemv_body<CodecQ4, M, GPL, MODE>(x, WeightPtrs{codes, nullptr, sm}, y, N, G, T, nchunks, tpb_grid, nwaves,
                                   &blob_mismatch_count);
}

// ---------------------------------------------------------------------------
// host side: instantiation table, launch-shape choice, validation
// ---------------------------------------------------------------------------

typedef void (*kernel_fn)(const u32x4*, const u32x4*, const u32x4*, float*, int, int, int, int, int, int);

constexpr int32_t kMaxK = 1 << 20;

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

kernel_fn kernel_for_mode(int mode, int M, int gi) {
  return mode == kMulti ? kernel_for<kMulti>(M, gi) : mode == kBlock ? kernel_for<kBlock>(M, gi)
                                                                      : kernel_for<kDirect>(M, gi);
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
  const LaunchShape shape = w4a16_host::choose_shape<CodecQ4>(M, K / kGroup);
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
  const LaunchShape shape = w4a16_host::choose_shape<CodecQ4>(M, G);
  if (shape.gi < 0) return W4A16_ERR_SHAPE;
  const int mode = w4a16_host::mode_of(shape.waves, shape.nchunks);
  kernel_fn fn = kernel_for_mode(mode, M, shape.gi);

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  const int T = (N + kTileRows - 1) / kTileRows;
  const bool direct = mode == kDirect;
  // all workgroups resident at once, each walking an equal share of the tiles
  const int occ = w4a16_host::resident_workgroups(M, shape.waves, occupancy(M, shape.gi, mode, shape.waves, fn));
  int tpb = 0, grid = 0;
  w4a16_host::grid_of(T, M, shape.waves, direct, w4a16_host::cu_count(dev), occ, tpb, grid);
  // regions after the header: codes, then the scale/min tiles
  const size_t codes_region = (size_t(N) * size_t(K) / 2 + 255) / 256 * 256;
  const uint8_t* base = static_cast<const uint8_t*>(packed);
  const u32x4* xp = static_cast<const u32x4*>(x);
  const u32x4* cp = reinterpret_cast<const u32x4*>(base + W4A16_BLOB_HEADER_BYTES);
  const u32x4* sp = reinterpret_cast<const u32x4*>(base + W4A16_BLOB_HEADER_BYTES + codes_region);
  int n_arg = N, g_arg = G, t_arg = T, c_arg = shape.nchunks, b_arg = w4a16_host::tpb_grid_arg(tpb, grid),
      w_arg = shape.waves;
  if (b_arg == 0) return W4A16_ERR_HIP;
  void* args[] = {&xp, &cp, &sp, &y, &n_arg, &g_arg, &t_arg, &c_arg, &b_arg, &w_arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(64 * shape.waves), args, 0,
                         static_cast<hipStream_t>(stream), start, stop, 0) != hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}

}  // namespace

namespace w4a16_host {

unsigned* q4_mismatch_word(int dev) {
  static std::atomic<unsigned*> cache[kMaxDevices];
  return device_word(reinterpret_cast<const void*>(&blob_mismatch_count), cache, dev);
}

}  // namespace w4a16_host

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
