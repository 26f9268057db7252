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

// A wait for all vector-memory loads that the compiler sees (the inline-asm
// waits of the kernels are opaque to it). After it the compiler knows that
// every load it issued has returned, so it puts no waits of its own for those
// loads inside the block loops that follow: such a wait would also count the
// LDS-DMA in flight, which the compiler cannot see, and stall on it.
__device__ inline void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0) only

// LDS-DMA: each lane moves 16 (dma16) or 4 (dma4) bytes from its own global
// address into `lds + lane * 16` (or `lane * 4`); the LDS base is
// wave-uniform. The instructions are written as inline asm on purpose: an
// LDS-DMA the compiler can see counts as a store to all of LDS, so the
// compiler makes every later LDS read wait for all outstanding loads
// (vmcnt(0)), exposing the full memory latency in the middle of a block's
// arithmetic. Every kernel here orders these writes itself: a block fetched
// by LDS-DMA is read only after an explicit s_waitcnt vmcnt(0) and a
// workgroup barrier. M0 holds the LDS destination; it is saved and restored
// around the load, and one wait state separates its write from the load.
// (The statements exist in the device pass only: the host pass checks asm
// constraints against the host target.)
#if defined(__HIP_DEVICE_COMPILE__)
#define STA_GLOBAL_LOAD_LDS(OP, gsrc, lds_dst)                                                      \
  do {                                                                                              \
    unsigned saved_m0_;                                                                             \
    const unsigned m0_ = unsigned(reinterpret_cast<unsigned long long>((lds_void*)(lds_dst)));      \
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t" OP " %1, off\n\ts_mov_b32 m0, %0" \
                 : "=&s"(saved_m0_)                                                                  \
                 : "v"(gsrc), "s"(m0_)                                                               \
                 : "memory");                                                                       \
  } while (0)
#else
#define STA_GLOBAL_LOAD_LDS(OP, gsrc, lds_dst) ((void)(gsrc), (void)(lds_dst))
#endif
__device__ inline void dma16(const char* gsrc, char* lds_dst) {
  STA_GLOBAL_LOAD_LDS("global_load_lds_dwordx4", gsrc, lds_dst);
}

// LDS-DMA of 16 bytes per lane from base + soff (wave-uniform) + voff (per
// lane) into lds_dst + 16 lane, through a buffer resource over base (the
// uniform part stays in scalar registers). Written as inline asm for the
// reason given at dma16: the kernel orders these writes itself. M0 holds the
// LDS destination: saved and restored around the load, one wait state between
// its write and the load. The offsets are unsigned byte offsets (the caller's
// tensors are limited to 2^32 bytes per (batch, head) slab). (Device pass only.)
__device__ inline void dma16_buf(const char* base, unsigned voff, unsigned soff, char* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  const i32x4 rsrc = {int(unsigned(b)), int(unsigned(b >> 32) & 0xffffu), 0x7fffffff, 0x00020000};
  const unsigned m0 = unsigned(reinterpret_cast<unsigned long long>((lds_void*)lds_dst));
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(m0), "s"(soff)
      : "memory");
#else
  (void)base, (void)voff, (void)soff, (void)lds_dst;
#endif
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

// LDS-DMA of one dword per lane (see dma16).
__device__ inline void dma4(const char* gsrc, char* lds_dst) {
  STA_GLOBAL_LOAD_LDS("global_load_lds_dword", gsrc, lds_dst);
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
