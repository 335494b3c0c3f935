// C-ABI entry points of the weight-code variants: argument checks, then the
// per-codec launcher (w4a16_codec_kernels.hip). Codec 0 is the 4-bit
// group-affine code of w4a16_gemv and goes there unchanged.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16.h"
#include "w4a16_codec_internal.h"
#include "w4a16_host.h"

namespace {

constexpr int kMaxM = 8;

w4a16_status codec_enqueue(int32_t codec, const void* x, const void* packed, float* y, int32_t M, int32_t N,
                           int32_t K, void* stream, hipEvent_t start, hipEvent_t stop) {
  if (codec < W4A16_CODEC_Q4 || codec > W4A16_CODEC_PAL4) return W4A16_ERR_FORMAT;
  if (codec == W4A16_CODEC_Q4) {
    if (start || stop) return w4a16_gemv_timed(x, packed, y, M, N, K, stream, start, stop);
    return w4a16_gemv(x, packed, y, M, N, K, stream);
  }
  if (!x || !packed || !y) return W4A16_ERR_NULL;
  w4a16_codecs::Regions reg;
  if (M < 1 || M > kMaxM || K > w4a16_max_k(M) || !w4a16_codecs::regions(codec, N, K, reg)) return W4A16_ERR_SHAPE;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  const uintptr_t pa = reinterpret_cast<uintptr_t>(packed);
  const uintptr_t ya = reinterpret_cast<uintptr_t>(y);
  if (xa % 16 || pa % 256 || ya % 4) return W4A16_ERR_ALIGN;
  const size_t ybytes = size_t(M) * size_t(N) * sizeof(float);
  if (w4a16_host::ranges_overlap(ya, ybytes, xa, size_t(M) * size_t(K) * 2) ||
      w4a16_host::ranges_overlap(ya, ybytes, pa, reg.total))
    return W4A16_ERR_OVERLAP;
  const w4a16_codecs::Launch l{x, packed, y, M, N, K, static_cast<hipStream_t>(stream), start, stop};
  switch (codec) {
    case W4A16_CODEC_Q4_SYM: return w4a16_codecs::enqueue_q4_sym(l, reg);
    case W4A16_CODEC_Q5: return w4a16_codecs::enqueue_q5(l, reg);
    case W4A16_CODEC_Q8_SYM: return w4a16_codecs::enqueue_q8_sym(l, reg);
    default: return w4a16_codecs::enqueue_pal4(l, reg);
  }
}

}  // namespace

extern "C" w4a16_status w4a16_codec_gemv(int32_t codec, const void* x, const void* packed, float* y, int32_t M,
                                         int32_t N, int32_t K, void* stream) {
  return codec_enqueue(codec, x, packed, y, M, N, K, stream, nullptr, nullptr);
}

extern "C" w4a16_status w4a16_codec_gemv_timed(int32_t codec, const void* x, const void* packed, float* y,
                                               int32_t M, int32_t N, int32_t K, void* stream, void* start_event,
                                               void* stop_event) {
  if (!start_event || !stop_event) return W4A16_ERR_NULL;
  return codec_enqueue(codec, x, packed, y, M, N, K, stream, static_cast<hipEvent_t>(start_event),
                       static_cast<hipEvent_t>(stop_event));
}

extern "C" w4a16_status w4a16_codec_launch_shape(int32_t codec, int32_t M, int32_t N, int32_t K, int32_t out[3]) {
  if (!out) return W4A16_ERR_NULL;
  if (codec < W4A16_CODEC_Q4 || codec > W4A16_CODEC_PAL4) return W4A16_ERR_FORMAT;
  if (codec == W4A16_CODEC_Q4) return w4a16_launch_shape(M, N, K, out);
  w4a16_codecs::Regions reg;
  if (M < 1 || M > kMaxM || K > w4a16_max_k(M) || !w4a16_codecs::regions(codec, N, K, reg)) return W4A16_ERR_SHAPE;
  switch (codec) {
    case W4A16_CODEC_Q4_SYM: return w4a16_codecs::shape_q4_sym(M, K, out);
    case W4A16_CODEC_Q5: return w4a16_codecs::shape_q5(M, K, out);
    case W4A16_CODEC_Q8_SYM: return w4a16_codecs::shape_q8_sym(M, K, out);
    default: return w4a16_codecs::shape_pal4(M, K, out);
  }
}

extern "C" w4a16_status w4a16_blob_mismatches(uint32_t* count) {
  if (!count) return W4A16_ERR_NULL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  unsigned* words[] = {w4a16_host::q4_mismatch_word(dev), w4a16_codecs::mismatch_word_q4_sym(dev),
                       w4a16_codecs::mismatch_word_q5(dev), w4a16_codecs::mismatch_word_q8_sym(dev),
                       w4a16_codecs::mismatch_word_pal4(dev)};
  if (hipDeviceSynchronize() != hipSuccess) return W4A16_ERR_HIP;
  uint32_t total = 0;
  for (unsigned* w : words) {
    unsigned v = 0;
    if (!w || hipMemcpy(&v, w, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess || hipMemset(w, 0, sizeof(v)) != hipSuccess)
      return W4A16_ERR_HIP;
    total += v;
  }
  if (hipDeviceSynchronize() != hipSuccess) return W4A16_ERR_HIP;
  *count = total;
  return W4A16_OK;
}
