// Host packers under a sanitizer (AddressSanitizer + UndefinedBehaviorSanitizer,
// or ThreadSanitizer): linked with the library's packer source built the same
// way, this program packs every codec and both KV widths at ragged and large
// shapes. Every input and output buffer is allocated at exactly the size the
// API documents for it, so a read or write one byte past any of them is
// reported; the large shapes make the packers split rows across threads, so
// ThreadSanitizer sees their concurrent writes. It also checks the documented
// results: OK on exact sizes, W4A16_ERR_SIZE with nothing written one byte
// short, the 5-bit range refusal, and w4a16_blob_check on what was written.
// Prints one line per failure and "ok <cases>" at the end; exits nonzero on
// any failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "w4a16.h"

namespace {

int failures = 0;
int cases = 0;

#define EXPECT(cond, ...)                            \
  do {                                               \
    if (!(cond)) {                                   \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);                      \
      std::printf("\n");                             \
      ++failures;                                    \
    }                                                \
  } while (0)

// splitmix64: a seeded stream of bytes for the inputs
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// heap block of exactly n bytes (malloc, so the sanitizer's redzone starts at
// byte n); n = 0 gives NULL
struct Block {
  uint8_t* p = nullptr;
  size_t n = 0;
  explicit Block(size_t bytes) : n(bytes) {
    if (n) p = static_cast<uint8_t*>(std::malloc(n));
  }
  ~Block() { std::free(p); }
  Block(const Block&) = delete;
  Block& operator=(const Block&) = delete;
  void fill(Rng& r, uint8_t mask = 0xFF) {
    for (size_t i = 0; i < n; ++i) p[i] = uint8_t(r.next()) & mask;
  }
  uint16_t* u16() { return reinterpret_cast<uint16_t*>(p); }
};

size_t code_bytes(int codec, int64_t N, int64_t K) {
  return (codec == W4A16_CODEC_Q5 || codec == W4A16_CODEC_Q8_SYM) ? size_t(N * K) : size_t(N * K / 2);
}

void weight_case(int codec, int32_t N, int32_t K, uint64_t seed) {
  ++cases;
  Rng r{seed};
  const bool affine = codec == W4A16_CODEC_Q4 || codec == W4A16_CODEC_Q5;
  const int64_t params = codec == W4A16_CODEC_PAL4 ? int64_t(N) * 16 : int64_t(N) * (K / 32);
  Block codes(code_bytes(codec, N, K)), scale(size_t(params) * 2), mn(affine ? size_t(params) * 2 : 0);
  codes.fill(r, codec == W4A16_CODEC_Q5 ? 0x1F : 0xFF);
  scale.fill(r);
  mn.fill(r);
  const size_t need = w4a16_codec_packed_bytes(codec, N, K);
  EXPECT(need > W4A16_BLOB_HEADER_BYTES, "codec %d N %d K %d: packed bytes %zu", codec, N, K, need);
  if (need <= W4A16_BLOB_HEADER_BYTES) return;

  Block out(need);
  int st = w4a16_codec_pack(codec, codes.p, scale.u16(), mn.u16(), N, K, out.p, out.n);
  EXPECT(st == W4A16_OK, "codec %d N %d K %d: pack status %d", codec, N, K, st);
  st = w4a16_blob_check(out.p, out.n, codec, N, K);
  EXPECT(st == W4A16_OK, "codec %d N %d K %d: blob check %d", codec, N, K, st);
  st = w4a16_blob_check(out.p, out.n - 1, codec, N, K);
  EXPECT(st == W4A16_ERR_SIZE, "codec %d N %d K %d: short blob check %d", codec, N, K, st);

  // the header alone, in a block of exactly its size: only it is read
  Block head(W4A16_BLOB_HEADER_BYTES);
  std::memcpy(head.p, out.p, head.n);
  st = w4a16_blob_check(head.p, need, codec, N, K);
  EXPECT(st == W4A16_OK, "codec %d N %d K %d: header-only check %d", codec, N, K, st);

  // one byte short: refused, nothing written
  Block shorter(need - 1);
  std::memset(shorter.p, 0xA5, shorter.n);
  st = w4a16_codec_pack(codec, codes.p, scale.u16(), mn.u16(), N, K, shorter.p, shorter.n);
  EXPECT(st == W4A16_ERR_SIZE, "codec %d N %d K %d: short pack status %d", codec, N, K, st);
  bool untouched = true;
  for (size_t i = 0; i < shorter.n; ++i) untouched &= shorter.p[i] == 0xA5;
  EXPECT(untouched, "codec %d N %d K %d: short pack wrote", codec, N, K);

  if (codec == W4A16_CODEC_Q4) {
    Block again(need);
    st = w4a16_pack(codes.p, scale.u16(), mn.u16(), N, K, again.p, again.n);
    EXPECT(st == W4A16_OK && std::memcmp(again.p, out.p, need) == 0, "w4a16_pack differs from codec 0 (N %d K %d)",
           N, K);
  }
  if (codec == W4A16_CODEC_Q5) {
    codes.p[codes.n - 1] = 32;  // the last code of the last row leaves the 5-bit range
    Block o2(need);
    std::memset(o2.p, 0xA5, o2.n);
    st = w4a16_codec_pack(codec, codes.p, scale.u16(), mn.u16(), N, K, o2.p, o2.n);
    bool clean = true;
    for (size_t i = 0; i < o2.n; ++i) clean &= o2.p[i] == 0xA5;
    EXPECT(st == W4A16_ERR_FORMAT && clean, "q5 code 32 (N %d K %d): status %d, untouched %d", N, K, st, int(clean));
  }
}

void kv_case(int bits, int32_t T, int32_t Hkv, uint64_t seed) {
  ++cases;
  Rng r{seed};
  const size_t cb = bits == 8 ? 128 : 64;
  const size_t th = size_t(T) * size_t(Hkv);
  Block kc(th * cb), vc(th * cb), ks(th * 8), vs(th * 8), km(bits == 4 ? th * 8 : 0), vm(bits == 4 ? th * 8 : 0);
  for (Block* b : {&kc, &vc, &ks, &vs, &km, &vm}) b->fill(r);
  const size_t need = w4a16_kv_packed_bytes(bits, T, Hkv);
  EXPECT(need > 0, "kv bits %d T %d Hkv %d: packed bytes 0", bits, T, Hkv);
  if (!need) return;
  Block out(need);
  int st = w4a16_kv_pack(bits, kc.p, ks.u16(), km.u16(), vc.p, vs.u16(), vm.u16(), T, Hkv, out.p, out.n);
  EXPECT(st == W4A16_OK, "kv bits %d T %d Hkv %d: status %d", bits, T, Hkv, st);
  Block shorter(need - 1);
  std::memset(shorter.p, 0x5A, shorter.n);
  st = w4a16_kv_pack(bits, kc.p, ks.u16(), km.u16(), vc.p, vs.u16(), vm.u16(), T, Hkv, shorter.p, shorter.n);
  bool untouched = true;
  for (size_t i = 0; i < shorter.n; ++i) untouched &= shorter.p[i] == 0x5A;
  EXPECT(st == W4A16_ERR_SIZE && untouched, "kv bits %d T %d Hkv %d: short status %d", bits, T, Hkv, st);
}

}  // namespace

int main() {
  const int32_t shapes[][2] = {{1, 32}, {3, 96}, {4, 64}, {5, 4128}, {17, 224}, {130, 512}, {257, 32}};
  uint64_t seed = 1;
  for (int codec = 0; codec <= 4; ++codec) {
    for (const auto& s : shapes) weight_case(codec, s[0], s[1], seed++);
    // enough bytes that the packer splits rows across threads
    weight_case(codec, 4100, 4096, seed++);
  }
  const int32_t kv[][2] = {{1, 1}, {63, 2}, {64, 3}, {65, 8}, {200, 1}, {4097, 8}};
  for (int bits : {8, 4})
    for (const auto& s : kv) kv_case(bits, s[0], s[1], seed++);
  if (failures) {
    std::printf("%d failures in %d cases\n", failures, cases);
    return 1;
  }
  std::printf("ok %d cases\n", cases);
  return 0;
}
