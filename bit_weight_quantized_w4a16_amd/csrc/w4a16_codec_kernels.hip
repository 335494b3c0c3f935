// gfx950 kernels of the weight-code variants: the single-GEMV skeleton with
// one codec policy. This file is compiled once per codec, with
// W4A16_CODEC_ID = 1 (symmetric 4-bit), 2 (5-bit affine), 3 (symmetric 8-bit)
// or 4 (palettised 4-bit); the codec formats are defined in include/w4a16.h.
//
// The variants are the quantisation types the Magnitude page compares when
// converting a model (section 4.2: a symmetric 4-bit type, the 4-bit and
// 5-bit K-quant types) and the 8-bit weights of the core-modules page
// (sections 5.1 and 5.2). Each is streamed exactly like the 4-bit code:
// 128-bit non-temporal loads, codes turned into binary16 subnormal pairs by
// masking, v_dot2 products, a per-group fold with the scale and the group's
// activation sum.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "w4a16.h"
#include "w4a16_codec_internal.h"
#include "w4a16_device.h"
#include "w4a16_host.h"
#include "w4a16_skeleton.h"

#ifndef W4A16_CODEC_ID
#error "compile with -DW4A16_CODEC_ID=1, 2, 3 or 4"
#endif

using namespace w4a16_dev;

namespace {

#if W4A16_CODEC_ID == 1
using Codec = CodecQ4Sym;
#elif W4A16_CODEC_ID == 2
using Codec = CodecQ5;
#elif W4A16_CODEC_ID == 3
using Codec = CodecQ8Sym;
#elif W4A16_CODEC_ID == 4
using Codec = CodecPal4;
#else
#error "unknown W4A16_CODEC_ID"
#endif

// Launches of this module whose blob header did not match their call, one
// word per device (reached from the host through hipGetSymbolAddress).
__device__ unsigned blob_mismatch_count;

// CODEC is the codec's id (it names the kernel in profiles:
// codec_kernel<codec, M, groups per lane, mode>).
template <int CODEC, int M, int GPL, int MODE>
__global__ void __launch_bounds__(64 * max_waves_of<Codec>(M, GPL))
codec_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ codes, const u32x4* __restrict__ aux,
             const void* __restrict__ side, float* __restrict__ y, int N, int G, int T, int nchunks, int tpb_grid,
             int nwaves) {
  gemv_body<Codec, M, GPL, MODE>(x, WeightPtrs{codes, aux, side}, y, N, G, T, nchunks, tpb_grid, nwaves,
                                 &blob_mismatch_count);
}

typedef void (*kernel_fn)(const u32x4*, const u32x4*, const u32x4*, const void*, float*, int, int, int, int, int,
                          int);

template <int M, int GPL, int MODE>
constexpr kernel_fn instance() {
  if constexpr (w4a16_host::gpl_allowed(M, GPL)) return &codec_kernel<W4A16_CODEC_ID, M, GPL, MODE>;
  return nullptr;
}

template <int M, int MODE>
constexpr kernel_fn pick(int gi) {
  // one or two groups per lane (four never fits the x-slice budget)
  return gi == 0 ? instance<M, 1, MODE>() : gi == 1 ? instance<M, 2, MODE>() : nullptr;
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

// LDS a codec asks for per wave beyond the skeleton's own (the palette
// tables of the palettised code), given at launch as dynamic LDS
template <class C, class = void>
struct lds_per_wave {
  static constexpr int value = 0;
};
template <class C>
struct lds_per_wave<C, decltype(void(C::kLdsBytesPerWave))> {
  static constexpr int value = C::kLdsBytesPerWave;
};
constexpr size_t dynamic_lds(int waves) { return size_t(lds_per_wave<Codec>::value) * waves; }

// resident workgroups per CU, cached per instantiation and block size
std::atomic<int> g_occupancy[kMaxM + 1][w4a16_host::kNumGpl][3][kMaxWaves + 1];

int occupancy(int M, int gi, int mode, int waves, kernel_fn fn) {
  std::atomic<int>& slot = g_occupancy[M][gi][mode][waves];
  int v = slot.load(std::memory_order_relaxed);
  if (v > 0) return v;
  v = w4a16_host::occupancy_of(reinterpret_cast<const void*>(fn), 64 * waves, dynamic_lds(waves));
  slot.store(v, std::memory_order_relaxed);
  return v;
}

w4a16_status shape(int M, int K, int32_t out[3]) {
  const w4a16_host::LaunchShape s = w4a16_host::choose_shape<Codec>(M, K / kGroup);
  if (s.gi < 0 || !kernel_for_mode(w4a16_host::mode_of(s.waves, s.nchunks), M, s.gi)) return W4A16_ERR_SHAPE;
  out[0] = w4a16_host::kGplOptions[s.gi];
  out[1] = s.waves;
  out[2] = s.nchunks;
  return W4A16_OK;
}

w4a16_status enqueue(const w4a16_codecs::Launch& l, const w4a16_codecs::Regions& reg) {
  const int G = l.K / kGroup;
  const w4a16_host::LaunchShape s = w4a16_host::choose_shape<Codec>(l.M, G);
  if (s.gi < 0) return W4A16_ERR_SHAPE;
  const int mode = w4a16_host::mode_of(s.waves, s.nchunks);
  const kernel_fn fn = kernel_for_mode(mode, l.M, s.gi);
  if (!fn) return W4A16_ERR_SHAPE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  const int T = (l.N + kTileRows - 1) / kTileRows;
  int tpb = 0, grid = 0;
  w4a16_host::grid_of(T, l.M, s.waves, mode == kDirect, w4a16_host::cu_count(dev),
                      w4a16_host::resident_workgroups(l.M, s.waves, occupancy(l.M, s.gi, mode, s.waves, fn)), tpb,
                      grid);
  const uint8_t* base = static_cast<const uint8_t*>(l.packed);
  const u32x4* xp = static_cast<const u32x4*>(l.x);
  const u32x4* cp = reinterpret_cast<const u32x4*>(base + reg.codes_at);
  const u32x4* ap = reg.aux ? reinterpret_cast<const u32x4*>(base + reg.aux) : nullptr;
  const void* sp = base + reg.side;
  float* y = l.y;
  int n_arg = l.N, g_arg = G, t_arg = T, c_arg = s.nchunks, b_arg = w4a16_host::tpb_grid_arg(tpb, grid),
      w_arg = s.waves;
  if (b_arg == 0) return W4A16_ERR_HIP;
  void* args[] = {&xp, &cp, &ap, &sp, &y, &n_arg, &g_arg, &t_arg, &c_arg, &b_arg, &w_arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(64 * s.waves), args,
                         dynamic_lds(s.waves), l.stream, l.start, l.stop, 0) != hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}

unsigned* mismatch_word(int dev) {
  static std::atomic<unsigned*> cache[w4a16_host::kMaxDevices];
  return w4a16_host::device_word(reinterpret_cast<const void*>(&blob_mismatch_count), cache, dev);
}

}  // namespace

namespace w4a16_codecs {
#if W4A16_CODEC_ID == 1
w4a16_status enqueue_q4_sym(const Launch& l, const Regions& r) { return enqueue(l, r); }
w4a16_status shape_q4_sym(int M, int K, int32_t out[3]) { return shape(M, K, out); }
unsigned* mismatch_word_q4_sym(int dev) { return mismatch_word(dev); }
#elif W4A16_CODEC_ID == 2
w4a16_status enqueue_q5(const Launch& l, const Regions& r) { return enqueue(l, r); }
w4a16_status shape_q5(int M, int K, int32_t out[3]) { return shape(M, K, out); }
unsigned* mismatch_word_q5(int dev) { return mismatch_word(dev); }
#elif W4A16_CODEC_ID == 3
w4a16_status enqueue_q8_sym(const Launch& l, const Regions& r) { return enqueue(l, r); }
w4a16_status shape_q8_sym(int M, int K, int32_t out[3]) { return shape(M, K, out); }
unsigned* mismatch_word_q8_sym(int dev) { return mismatch_word(dev); }
#else
w4a16_status enqueue_pal4(const Launch& l, const Regions& r) { return enqueue(l, r); }
w4a16_status shape_pal4(int M, int K, int32_t out[3]) { return shape(M, K, out); }
unsigned* mismatch_word_pal4(int dev) { return mismatch_word(dev); }
#endif
}  // namespace w4a16_codecs
