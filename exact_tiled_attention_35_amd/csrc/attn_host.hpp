// Host-side argument checks shared by the C ABI entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "attn.h"

namespace eta_host {

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Finite test on the bits, independent of floating-point compile flags.
inline bool finite_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof u);
  return ((u >> 23) & 0xffu) != 0xffu;
}

// ATTN_OK when the current device is a gfx950; the answer is cached per
// device (0 = unknown, 1 = gfx950, 2 = other architecture).
inline int check_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> arch_state[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_NO_DEVICE;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0 || dev >= count) return ATTN_ERR_NO_DEVICE;
  if (dev >= kMaxDevices) return ATTN_ERR_NO_DEVICE;
  int st = arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_NO_DEVICE;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? ATTN_OK : ATTN_ERR_NO_DEVICE;
}

}  // namespace eta_host
