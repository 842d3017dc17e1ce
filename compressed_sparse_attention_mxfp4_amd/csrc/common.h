// Device-side helpers shared by the CSA2 HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

namespace csa2 {

constexpr int kD = CSA2_D;
constexpr int kDI = CSA2_DI;
constexpr int kPage = CSA2_PAGE;
constexpr int kEntryCodes = CSA2_ENTRY_CODE_BYTES;
constexpr int kEntryScales = CSA2_ENTRY_SCALE_BYTES;
constexpr int kPageBytes = CSA2_PAGE_BYTES;
constexpr int kBlock = CSA2_BLOCK;
constexpr int kSwa = CSA2_SWA;

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// Order-preserving map float -> uint32 (larger float, larger key).  Finite
// floats map to keys >= 0x00800000; key 0 is never produced by a finite
// score and marks an empty candidate slot.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = f2u(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return u2f((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Physical page of logical page lp of sequence b, or -1 when not usable.
__device__ __forceinline__ int64_t phys_page(const int32_t* __restrict__ page_table, int max_pages,
                                             int64_t n_pages, int b, int lp) {
  if (lp < 0 || lp >= max_pages) return -1;
  int32_t p = page_table[(int64_t)b * max_pages + lp];
  return (p >= 0 && p < n_pages) ? (int64_t)p : -1;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Orders this lane's LDS accesses around a hand-off to other lanes of the
// wave: the LDS executes one wave's instructions in order, so keeping the
// compiler from moving memory accesses across this point is enough.
__device__ __forceinline__ void wave_lds_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Events recorded around launches of each kernel (csa2_time_kernel).
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
KernelEvents& kernel_events(int kernel);

}  // namespace csa2

#include <hip/hip_ext.h>

// Launch `kern` on `stream`, bracketed by the events registered for `kid`.
#define CSA2_LAUNCH(kid, kern, grid, block, stream, ...)                                   \
  do {                                                                                      \
    const ::csa2::KernelEvents& ev_ = ::csa2::kernel_events(kid);                          \
    if (ev_.start && ev_.stop)                                                              \
      hipExtLaunchKernelGGL(kern, grid, block, 0, stream, ev_.start, ev_.stop, 0, __VA_ARGS__); \
    else                                                                                    \
      hipLaunchKernelGGL(kern, grid, block, 0, stream, __VA_ARGS__);                        \
  } while (0)
