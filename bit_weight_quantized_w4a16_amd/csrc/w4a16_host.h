// Host-side helpers shared by the entry points of libw4a16. Internal header.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>

namespace w4a16_host {

// Compute-unit count of a device, cached per device (0 = not yet queried).
inline int cu_count(int dev) {
  constexpr int kMaxDevices = 64;
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

#ifdef W4A16_TUNING
// Sweep builds only: integer overrides from the environment (0 = unset).
inline int tune(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}
#else
constexpr int tune(const char*) { return 0; }
#endif

}  // namespace w4a16_host
