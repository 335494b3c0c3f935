// Host-side repacker: canonical nibbles + per-group binary16 scale/min ->
// the packed blob the gfx950 kernel streams (layout in include/w4a16.h).
//
// The packer of the core-modules page (section 5.1) quantises and lays a model
// out once, offline; doing the re-layout here keeps every run-time load a
// full 16-byte, lane-contiguous chunk and lets the kernel unpack a nibble pair
// with a single AND.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "w4a16.h"
#include "w4a16_codec_internal.h"

namespace {

constexpr int64_t kGroup = 32;
constexpr int64_t kTileRows = 4;
constexpr int64_t kRegionAlign = 256;

// Bytes b0..b3 (little-endian word v) hold k = 8d + 0..7 as (lo = even k,
// hi = odd k) nibble pairs. Return the word with the four even k in the low
// half-word and the four odd k in the high half-word, in increasing k.
inline uint32_t split_even_odd(uint32_t v) {
  uint32_t e = v & 0x0F0F0F0Fu;          // even k, one per byte
  uint32_t o = (v >> 4) & 0x0F0F0F0Fu;   // odd k, one per byte
  e = (e | (e >> 4)) & 0x00FF00FFu;      // squeeze nibbles pairwise
  e = (e | (e >> 8)) & 0x0000FFFFu;
  o = (o | (o >> 4)) & 0x00FF00FFu;
  o = (o | (o >> 8)) & 0x0000FFFFu;
  return e | (o << 16);
}

constexpr int64_t kHead = W4A16_BLOB_HEADER_BYTES;

int64_t codes_region_bytes(int64_t N, int64_t K) {
  int64_t c = N * K / 2;
  return (c + kRegionAlign - 1) / kRegionAlign * kRegionAlign;
}

// The blob header (layout in include/w4a16.h): the fields the kernels
// compare, the blob's size, zeros to 256 bytes.
void write_header(uint8_t* o, int32_t codec, int32_t N, int32_t K, uint64_t total) {
  std::memset(o, 0, size_t(kHead));
  const uint32_t magic = W4A16_BLOB_MAGIC;
  const uint16_t version = W4A16_LAYOUT_VERSION, cid = uint16_t(codec);
  std::memcpy(o, &magic, 4);
  std::memcpy(o + 4, &version, 2);
  std::memcpy(o + 6, &cid, 2);
  std::memcpy(o + 8, &N, 4);
  std::memcpy(o + 12, &K, 4);
  std::memcpy(o + 16, &total, 8);
}

template <class F>
void parallel_rows(int64_t rows, int64_t work_per_row, F&& body) {
  int64_t total = rows * work_per_row;
  unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  int64_t nthreads = std::min<int64_t>(hw, std::max<int64_t>(1, total >> 22));
  nthreads = std::min<int64_t>(nthreads, rows);
  if (nthreads <= 1) {
    body(0, rows);
    return;
  }
  std::vector<std::thread> pool;
  int64_t per = (rows + nthreads - 1) / nthreads;
  for (int64_t t = 0; t < nthreads; ++t) {
    int64_t r0 = t * per, r1 = std::min(rows, r0 + per);
    if (r0 >= r1) break;
    pool.emplace_back([&body, r0, r1] { body(r0, r1); });
  }
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" size_t w4a16_packed_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < kGroup || K % kGroup) return 0;
  int64_t G = K / kGroup;
  if (int64_t(N) * G > INT32_MAX) return 0;
  int64_t T = (int64_t(N) + kTileRows - 1) / kTileRows;
  return size_t(kHead + codes_region_bytes(N, K) + T * G * 16);
}

extern "C" w4a16_status w4a16_pack(const uint8_t* codes, const uint16_t* scale, const uint16_t* min,
                                   int32_t N, int32_t K, void* out, size_t out_bytes) {
  if (!codes || !scale || !min || !out) return W4A16_ERR_NULL;
  size_t need = w4a16_packed_bytes(N, K);
  if (need == 0) return W4A16_ERR_SHAPE;
  if (out_bytes < need) return W4A16_ERR_SIZE;

  const int64_t G = K / kGroup;
  const int64_t row_bytes = int64_t(K) / 2;
  const int64_t S = codes_region_bytes(N, K);
  const int64_t T = (int64_t(N) + kTileRows - 1) / kTileRows;
  write_header(static_cast<uint8_t*>(out), W4A16_CODEC_Q4, N, K, need);
  uint8_t* o = static_cast<uint8_t*>(out) + kHead;

  // codes: same byte footprint as the canonical array, words re-ordered in place
  parallel_rows(N, row_bytes, [&](int64_t r0, int64_t r1) {
    for (int64_t n = r0; n < r1; ++n) {
      const uint8_t* src = codes + n * row_bytes;
      uint8_t* dst = o + n * row_bytes;
      for (int64_t b = 0; b < row_bytes; b += 4) {
        uint32_t v;
        std::memcpy(&v, src + b, 4);
        v = split_even_odd(v);
        std::memcpy(dst + b, &v, 4);
      }
    }
  });
  std::memset(o + int64_t(N) * row_bytes, 0, size_t(S - int64_t(N) * row_bytes));

  // scale/min tiles of 4 rows x 1 group
  uint8_t* sm = o + S;
  parallel_rows(T, G * 16, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t) {
      for (int64_t g = 0; g < G; ++g) {
        uint16_t e[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int64_t r = 0; r < kTileRows; ++r) {
          int64_t n = t * kTileRows + r;
          if (n < N) {
            e[2 * r] = scale[n * G + g];
            e[2 * r + 1] = min[n * G + g];
          }
        }
        std::memcpy(sm + (t * G + g) * 16, e, 16);
      }
    }
  });
  return W4A16_OK;
}

// ---------------------------------------------------------------------------
// Weight-code variants (formats in include/w4a16.h)
// ---------------------------------------------------------------------------

namespace w4a16_codecs {

bool regions(int codec, int32_t N, int32_t K, Regions& r) {
  if (codec < W4A16_CODEC_Q4 || codec > W4A16_CODEC_PAL4) return false;
  if (N < 1 || K < kGroup || K % kGroup) return false;
  const int64_t G = K / kGroup;
  if (int64_t(N) * G > INT32_MAX) return false;
  const int64_t T = (int64_t(N) + kTileRows - 1) / kTileRows;
  const int64_t code_bytes = int64_t(N) * G * (codec == W4A16_CODEC_Q8_SYM ? 32 : 16);
  const int64_t S = kHead + (code_bytes + kRegionAlign - 1) / kRegionAlign * kRegionAlign;
  r.codes_at = size_t(kHead);
  r.codes = size_t(code_bytes);
  r.aux = codec == W4A16_CODEC_Q5 ? size_t(S) : 0;
  r.side = size_t(S + (codec == W4A16_CODEC_Q5 ? T * G * 16 : 0));
  if (codec == W4A16_CODEC_PAL4) {  // one 128-byte palette entry per tile
    r.total = r.side + size_t(T * 128);
    return true;
  }
  const int64_t side_entry = (codec == W4A16_CODEC_Q4_SYM || codec == W4A16_CODEC_Q8_SYM) ? 8 : 16;
  r.total = r.side + size_t(T * G * side_entry);
  return true;
}

}  // namespace w4a16_codecs

namespace {

// Bit b = 4j + d of a row's fifth-bit word of a group holds k = 8d + 2(j mod 4) + j/4.
constexpr int fifth_bit_k(int b) { return 8 * (b % 4) + 2 * ((b / 4) % 4) + (b / 4) / 4; }

// The four binary16 numbers of rows 4t..4t+3 for group g (zero past N).
void tile_halves(const uint16_t* v, int64_t N, int64_t G, int64_t t, int64_t g, uint16_t (&e)[4]) {
  for (int64_t r = 0; r < kTileRows; ++r) {
    const int64_t n = t * kTileRows + r;
    e[r] = n < N ? v[n * G + g] : 0;
  }
}

}  // namespace

extern "C" size_t w4a16_codec_packed_bytes(int32_t codec, int32_t N, int32_t K) {
  w4a16_codecs::Regions r;
  return w4a16_codecs::regions(codec, N, K, r) ? r.total : 0;
}

extern "C" w4a16_status w4a16_codec_pack(int32_t codec, const uint8_t* codes, const uint16_t* scale,
                                         const uint16_t* min, int32_t N, int32_t K, void* out, size_t out_bytes) {
  if (codec < W4A16_CODEC_Q4 || codec > W4A16_CODEC_PAL4) return W4A16_ERR_FORMAT;
  if (codec == W4A16_CODEC_Q4) return w4a16_pack(codes, scale, min, N, K, out, out_bytes);
  const bool affine = codec == W4A16_CODEC_Q5;
  if (!codes || !scale || (affine && !min) || !out) return W4A16_ERR_NULL;
  w4a16_codecs::Regions reg;
  if (!w4a16_codecs::regions(codec, N, K, reg)) return W4A16_ERR_SHAPE;
  if (out_bytes < reg.total) return W4A16_ERR_SIZE;
  const int64_t G = K / kGroup;
  const int64_t T = (int64_t(N) + kTileRows - 1) / kTileRows;
  if (codec == W4A16_CODEC_Q5) {  // every code must fit 5 bits; checked before anything is written
    const int64_t total = int64_t(N) * K;
    for (int64_t i = 0; i < total; ++i)
      if (codes[i] > 31) return W4A16_ERR_FORMAT;
  }
  uint8_t* const blob = static_cast<uint8_t*>(out);
  write_header(blob, codec, N, K, reg.total);
  std::memset(blob + reg.codes_at + reg.codes, 0, reg.total - reg.codes_at - reg.codes);  // padding, tiles past N
  uint8_t* o = blob + reg.codes_at;  // the code region
  if (codec == W4A16_CODEC_PAL4) {
    // codes: the canonical bytes, row after row; palettes: per tile, entry c
    // of row r at byte 8c + 2r (binary16, little-endian)
    std::memcpy(o, codes, size_t(N) * size_t(K / 2));
    uint8_t* lt = blob + reg.side;
    for (int64_t n = 0; n < N; ++n)
      for (int c = 0; c < 16; ++c) {
        const uint16_t e = scale[n * 16 + c];
        uint8_t* dst = lt + (n / kTileRows) * 128 + 8 * c + 2 * (n % kTileRows);
        dst[0] = uint8_t(e & 0xFFu);
        dst[1] = uint8_t(e >> 8);
      }
    return W4A16_OK;
  }

  // code chunks
  parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
    for (int64_t n = r0; n < r1; ++n) {
      if (codec == W4A16_CODEC_Q4_SYM) {  // the 4-bit code's chunk layout
        const uint8_t* src = codes + n * (K / 2);
        uint8_t* dst = o + n * (K / 2);
        for (int64_t b = 0; b < K / 2; b += 4) {
          uint32_t v;
          std::memcpy(&v, src + b, 4);
          v = split_even_odd(v);
          std::memcpy(dst + b, &v, 4);
        }
      } else if (codec == W4A16_CODEC_Q5) {  // low nibbles in the 4-bit layout
        const uint8_t* src = codes + n * int64_t(K);
        uint8_t* dst = o + n * (K / 2);
        for (int64_t k = 0; k < K; k += 8) {
          uint32_t v = 0;
          for (int i = 0; i < 4; ++i)
            v |= uint32_t((src[k + 2 * i] & 0xF) | ((src[k + 2 * i + 1] & 0xF) << 4)) << (8 * i);
          v = split_even_odd(v);
          std::memcpy(dst + k / 2, &v, 4);
        }
      } else {  // 8-bit: offset-binary bytes, low halves then high halves of every group
        const uint8_t* src = codes + n * int64_t(K);
        uint8_t* row = o + n * G * 32;
        static constexpr int kSlotOf[4] = {0, 2, 1, 3};  // byte slot of i = 0..3 in a word
        for (int64_t g = 0; g < G; ++g)
          for (int h = 0; h < 2; ++h) {
            uint8_t* dst = row + (h * G + g) * 16;
            for (int e = 0; e < 4; ++e)
              for (int i = 0; i < 4; ++i)
                dst[4 * e + kSlotOf[i]] = uint8_t(src[32 * g + 16 * h + 4 * e + i] ^ 0x80u);
          }
      }
    }
  });

  // fifth-bit tiles (5-bit code)
  if (codec == W4A16_CODEC_Q5) {
    uint8_t* hb = blob + reg.aux;
    parallel_rows(T, G * 128, [&](int64_t t0, int64_t t1) {
      for (int64_t t = t0; t < t1; ++t)
        for (int64_t g = 0; g < G; ++g) {
          uint32_t e[4] = {0, 0, 0, 0};
          for (int64_t r = 0; r < kTileRows; ++r) {
            const int64_t n = t * kTileRows + r;
            if (n >= N) continue;
            const uint8_t* q = codes + n * int64_t(K) + 32 * g;
            for (int b = 0; b < 32; ++b) e[r] |= uint32_t((q[fifth_bit_k(b)] >> 4) & 1u) << b;
          }
          std::memcpy(hb + (t * G + g) * 16, e, 16);
        }
    });
  }

  // scale (and min) tiles
  uint8_t* side = blob + reg.side;
  parallel_rows(T, G * 16, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t)
      for (int64_t g = 0; g < G; ++g) {
        uint16_t s4[4], m4[4] = {0, 0, 0, 0};
        tile_halves(scale, N, G, t, g, s4);
        if (affine) {
          tile_halves(min, N, G, t, g, m4);
          uint16_t e[8];
          for (int r = 0; r < 4; ++r) {
            e[2 * r] = s4[r];
            e[2 * r + 1] = m4[r];
          }
          std::memcpy(side + (t * G + g) * 16, e, 16);
        } else {
          std::memcpy(side + (t * G + g) * 8, s4, 8);
        }
      }
  });
  return W4A16_OK;
}

// ---------------------------------------------------------------------------
// Quantised KV cache (format in include/w4a16.h)
// ---------------------------------------------------------------------------

// One record holds 64 tokens of one KV head: 17408 bytes at INT8, 10240 at
// INT4. The attention kernels' record structs carry the same sizes; the size
// tests and the KV parity tests fail if the two ever differ.
namespace {
constexpr int64_t kKvTok = 64;
constexpr int64_t kv_record_bytes(int32_t bits) { return bits == 8 ? 17408 : 10240; }
}  // namespace

extern "C" size_t w4a16_kv_packed_bytes(int32_t bits, int32_t T, int32_t Hkv) {
  if ((bits != 8 && bits != 4) || T < 1 || T > (1 << 24) || Hkv < 1 || Hkv > 4096) return 0;
  const int64_t nb = (int64_t(T) + kKvTok - 1) / kKvTok;
  return size_t(int64_t(Hkv) * nb * kv_record_bytes(bits));
}

extern "C" w4a16_status w4a16_kv_pack(int32_t bits, const uint8_t* k_codes, const uint16_t* k_scale,
                                      const uint16_t* k_min, const uint8_t* v_codes, const uint16_t* v_scale,
                                      const uint16_t* v_min, int32_t T, int32_t Hkv, void* out, size_t out_bytes) {
  if (bits != 8 && bits != 4) return W4A16_ERR_FORMAT;
  if (!k_codes || !k_scale || !v_codes || !v_scale || !out || (bits == 4 && (!k_min || !v_min)))
    return W4A16_ERR_NULL;
  const size_t need = w4a16_kv_packed_bytes(bits, T, Hkv);
  if (need == 0) return W4A16_ERR_SHAPE;
  if (out_bytes < need) return W4A16_ERR_SIZE;
  constexpr int64_t kD = 128, kTok = kKvTok;
  const int64_t nb = (int64_t(T) + kTok - 1) / kTok;
  const int64_t R = kv_record_bytes(bits);
  const int64_t cb = bits == 8 ? kD : kD / 2;  // canonical code bytes per (token, head)
  uint8_t* o = static_cast<uint8_t*>(out);
  parallel_rows(int64_t(Hkv) * nb, R, [&](int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r) {
      const int64_t g = r / nb, b = r % nb;
      uint8_t* rec = o + r * R;
      std::memset(rec, 0, size_t(R));
      for (int64_t tt = 0; tt < kTok; ++tt) {
        const int64_t t = b * kTok + tt;
        if (t >= T) break;
        const uint8_t* kc = k_codes + (t * Hkv + g) * cb;
        const uint8_t* vc = v_codes + (t * Hkv + g) * cb;
        const int64_t pi = (t * Hkv + g) * 4;  // parameters of (t, g)
        // byte slot of element i of a 4-element word, and of a 4-bit
        // element i of an 8-element word (low nibble for i < 4): elements
        // (0, 2, 1, 3) in bytes 0..3, so the masks 0x00FF00FF (0x000F000F
        // for nibbles) on the word and on the word >> 8 give elements
        // (0, 1) and (2, 3) as binary16 pairs; the high nibbles hold 4..7
        static constexpr int kSlot[4] = {0, 2, 1, 3};
        if (bits == 8) {
          for (int c = 0; c < 8; ++c)
            for (int e = 0; e < 4; ++e)
              for (int j = 0; j < 4; ++j)
                rec[c * 1024 + tt * 16 + 4 * e + kSlot[j]] = uint8_t(kc[16 * c + 4 * e + j] ^ 0x80u);
          std::memcpy(rec + 8192 + tt * 8, k_scale + pi, 8);
          std::memcpy(rec + 8704 + tt * 8, v_scale + pi, 8);
          // values: load 4h + tq = dims 64h .. 64h + 63 of tokens 16tq .. 16tq + 15; lane l = dim 64h + l,
          // word e = tokens 16tq + 4e .. + 3
          const int64_t tq = tt / 16, e = (tt % 16) / 4;
          for (int d = 0; d < 128; ++d)
            rec[9216 + (4 * (d / 64) + tq) * 1024 + (d % 64) * 16 + 4 * e + kSlot[tt % 4]] = uint8_t(vc[d] ^ 0x80u);
        } else {
          auto nib = [](const uint8_t* canon, int d) { return (canon[d / 2] >> (4 * (d % 2))) & 0xF; };
          // keys: chunk c = group c, word wd = dims 32c + 8wd .. + 7
          for (int c = 0; c < 4; ++c)
            for (int wd = 0; wd < 4; ++wd)
              for (int i = 0; i < 8; ++i)
                rec[c * 1024 + tt * 16 + 4 * wd + kSlot[i % 4]] |= uint8_t(nib(kc, 32 * c + 8 * wd + i) << (4 * (i / 4)));
          uint16_t kp[8], vp[8];
          for (int grp = 0; grp < 4; ++grp) {
            kp[2 * grp] = k_scale[pi + grp];
            kp[2 * grp + 1] = k_min[pi + grp];
            vp[2 * grp] = v_scale[pi + grp];
            vp[2 * grp + 1] = v_min[pi + grp];
          }
          std::memcpy(rec + 4096 + tt * 16, kp, 16);
          std::memcpy(rec + 5120 + tt * 16, vp, 16);
          // values: load 2h + th = dims 64h .. 64h + 63 of tokens 32th .. 32th + 31; lane l = dim 64h + l,
          // word w = tokens 32th + 8w .. + 7
          const int64_t th = tt / 32, w = (tt % 32) / 8, i = tt % 8;
          for (int d = 0; d < 128; ++d)
            rec[6144 + (2 * (d / 64) + th) * 1024 + (d % 64) * 16 + 4 * w + kSlot[i % 4]] |=
                uint8_t(nib(vc, d) << (4 * (i / 4)));
        }
      }
    }
  });
  return W4A16_OK;
}

extern "C" w4a16_status w4a16_blob_check(const void* blob, size_t bytes, int32_t codec, int32_t N, int32_t K) {
  if (!blob) return W4A16_ERR_NULL;
  w4a16_codecs::Regions reg;
  if (!w4a16_codecs::regions(codec, N, K, reg)) return W4A16_ERR_SHAPE;
  if (bytes < size_t(kHead)) return W4A16_ERR_SIZE;
  uint8_t want[kHead];
  write_header(want, codec, N, K, reg.total);
  if (std::memcmp(blob, want, size_t(kHead)) != 0) return W4A16_ERR_FORMAT;
  return bytes < reg.total ? W4A16_ERR_SIZE : W4A16_OK;
}

extern "C" int32_t w4a16_abi_version(void) { return W4A16_LAYOUT_VERSION; }

// The statuses are the refusals a runtime owes its caller under the contract
// table of the core-modules page (section 5.7): an input it does not cover is
// turned away with a reason, never run.
extern "C" const char* w4a16_status_string(int32_t status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_NULL: return "a required pointer is NULL";
    case W4A16_ERR_SHAPE: return "M, N or K outside the supported range";
    case W4A16_ERR_ALIGN: return "a pointer breaks its alignment rule";
    case W4A16_ERR_SIZE: return "output buffer smaller than required";
    case W4A16_ERR_OVERLAP: return "y overlaps x or the packed weights";
    case W4A16_ERR_HIP: return "the HIP runtime reported an error";
    case W4A16_ERR_FORMAT: return "unknown codec, a code outside its codec's range, or a blob header that does not match";
    case W4A16_ERR_WAIT: return "a chain launch's ordering wait gave up; its results are invalid";
    default: return "unknown status";
  }
}
