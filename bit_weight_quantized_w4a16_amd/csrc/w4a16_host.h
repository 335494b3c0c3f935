// Host-side helpers shared by the entry points of libw4a16. Internal header.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace w4a16_host {

constexpr int kMaxDevices = 64;

// Compute-unit count of a device, cached per device (0 = not yet queried).
inline int cu_count(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

// Resident workgroups per CU of a kernel at a block size and dynamic LDS
// size (never below 1).
inline int occupancy_of(const void* fn, int block_threads, size_t dynamic_lds = 0) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, block_threads, dynamic_lds) != hipSuccess || nb <= 0)
    nb = 1;
  return nb;
}

inline bool ranges_overlap(uintptr_t a, size_t na, uintptr_t b, size_t nb) { return a < b + nb && b < a + na; }

// Device address of a __device__ word of the calling translation unit
// (`symbol` is the address of its host-side stand-in, which is not itself a
// device address) on device `dev`, which must be current:
// every device holds its own copy. Cached per device in `cache`; nullptr if
// it cannot be located.
inline unsigned* device_word(const void* symbol, std::atomic<unsigned*> (&cache)[kMaxDevices], int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  unsigned* p = cache[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* a = nullptr;
  if (hipGetSymbolAddress(&a, symbol) != hipSuccess || !a) return nullptr;
  p = static_cast<unsigned*>(a);
  cache[dev].store(p, std::memory_order_release);
  return p;
}

// The single-GEMV module's count of launches whose blob header did not
// match their call, on device dev (current); nullptr if it cannot be located.
unsigned* q4_mismatch_word(int dev);

}  // namespace w4a16_host
