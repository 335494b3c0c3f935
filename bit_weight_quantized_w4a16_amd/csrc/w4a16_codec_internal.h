// Per-codec launchers of the weight-code variants, one per translation unit
// (w4a16_codec_kernels.hip compiled once per codec). Internal header of
// libw4a16.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "w4a16.h"

namespace w4a16_codecs {

// Region layout of one packed blob of a codec (byte offsets; see include/w4a16.h).
struct Regions {
  size_t codes_at;  // offset of the code region (just past the blob header)
  size_t codes;     // bytes of the code region before its 256-byte padding
  size_t aux;       // offset of the fifth-bit tiles (5-bit code), else 0
  size_t side;      // offset of the scale (and min) tiles
  size_t total;     // w4a16_codec_packed_bytes
};
// false if the codec is unknown or (N, K) is out of range
bool regions(int codec, int32_t N, int32_t K, Regions& r);

// Validated arguments of one launch.
struct Launch {
  const void* x;
  const void* packed;
  float* y;
  int M, N, K;
  hipStream_t stream;
  hipEvent_t start, stop;
};

// Enqueue one GEMV of codec 1, 2, 3 or 4, or report its launch shape
// (groups per lane, waves, passes) through `shape`.
w4a16_status enqueue_q4_sym(const Launch& l, const Regions& r);
w4a16_status enqueue_q5(const Launch& l, const Regions& r);
w4a16_status enqueue_q8_sym(const Launch& l, const Regions& r);
w4a16_status enqueue_pal4(const Launch& l, const Regions& r);
w4a16_status shape_q4_sym(int M, int K, int32_t shape[3]);
w4a16_status shape_q5(int M, int K, int32_t shape[3]);
w4a16_status shape_q8_sym(int M, int K, int32_t shape[3]);
w4a16_status shape_pal4(int M, int K, int32_t shape[3]);
// Each codec module's count of launches whose blob header did not match
// their call, on device dev (current); nullptr if it cannot be located.
unsigned* mismatch_word_q4_sym(int dev);
unsigned* mismatch_word_q5(int dev);
unsigned* mismatch_word_q8_sym(int dev);
unsigned* mismatch_word_pal4(int dev);

}  // namespace w4a16_codecs
