// Device helpers shared by the STA kernels (forward and backward): vector
// types, cross-lane reductions, LDS-DMA, the per-XCD work queues and exact
// small divisions. Internal; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sta_internal.h"

namespace sta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

__device__ inline float swap16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float swap32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS-DMA: each lane moves 16 bytes from its own global address into
// `lds + lane * 16` (the LDS base is wave-uniform).
__device__ inline void dma16(const char* gsrc, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_dst, 16, 0, 0);
}

// Next query unit for a workgroup on XCD `xcd`, or -1 once every queue is
// empty. Queue y holds work[8k + y], k < ceil((total - y) / 8); its head
// claim[y * kClaimStride] counts the items taken (it may run past the end).
// Each successful fetch-add hands out a distinct item, and a workgroup only
// gets -1 after seeing every queue exhausted, so every unit is run exactly
// once whatever the grid size.
__device__ inline int claim_unit(const int32_t* work, int32_t* claim, int total, int xcd) {
  for (int t = 0; t < kQueues; ++t) {
    const int y = (xcd + t) & (kQueues - 1);
    const int n_y = (total - y + kQueues - 1) / kQueues;
    if (n_y <= 0) continue;
    const int k = __hip_atomic_fetch_add(claim + y * kClaimStride, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    if (k < n_y) return work[kQueues * k + y];
  }
  return -1;
}

// floor(n / d) for n >= 0, d >= 1, n * d < 2^32, with m = ceil(2^32 / d) (see Geom).
__device__ inline int div_by(int n, int d, uint32_t m) {
  return d == 1 ? n : int(__umulhi(uint32_t(n), m));
}

// LDS-DMA of one dword per lane: `lds + lane * 4` receives 4 bytes from the
// lane's own global address.
__device__ inline void dma4(const char* gsrc, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_dst, 4, 0, 0);
}

// The lane id through an empty asm when OPAQUE: values derived from it are
// recomputed where they are used instead of being hoisted out of a loop.
template <bool OPAQUE>
__device__ inline int opaque_lane(int lane) {
  if constexpr (OPAQUE) asm volatile("" : "+v"(lane));
  return lane;
}

// Workgroups of `kernel` that fit on the current device at once (CU count
// times occupancy), cached per device in `cache` (kMaxDevices entries,
// zero-initialised). 0 on error.
constexpr int kMaxDevices = 64;
template <typename F>
int resident_workgroups(F kernel, int threads, int* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int* slot = dev < kMaxDevices ? &cache[dev] : nullptr;
  int n = slot != nullptr ? __atomic_load_n(slot, __ATOMIC_RELAXED) : 0;
  if (n > 0) return n;
  int n_cu = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  n = n_cu * (per_cu > 0 ? per_cu : 1);
  if (slot != nullptr) __atomic_store_n(slot, n, __ATOMIC_RELAXED);
  return n;
}

}  // namespace
}  // namespace sta
