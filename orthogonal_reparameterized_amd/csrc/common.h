// Shared internals of libpoetx: status plumbing, launch bookkeeping, bf16 helpers,
// workspace carving.  Not part of the public ABI (see include/poetx.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>

#include "../../include/poetx.h"

namespace poetx {

// ------------------------------------------------------------------ status ----
#define POETX_TRY(expr)                  \
  do {                                   \
    int _st = (expr);                    \
    if (_st != POETX_OK) return _st;     \
  } while (0)

// Launch bookkeeping: every kernel launch goes through launch_k, which checks for
// launch errors and, while the calling thread's measurement recorder is on (see
// poetx_prof_enable), attaches a start and a stop event to the dispatch itself
// (hipExtLaunchKernel), so the recorded time is the kernel's own execution with no
// marker packets between kernels.  The recorder is per thread: no state is shared
// between callers.
bool prof_on();
// a pair from this thread's pool when a launch labelled `name` is to be recorded
bool prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop);
void prof_commit(const char *name, hipEvent_t start, hipEvent_t stop);

template <typename... KP, typename... Args>
inline int launch_k(const char *name, hipStream_t s, void (*kern)(KP...), dim3 grid, dim3 block, size_t lds,
                    Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool rec = prof_on() && prof_events(name, &e0, &e1);
  hipExtLaunchKernelGGL(kern, grid, block, (std::uint32_t)lds, s, e0, e1, 0, args...);
  const hipError_t e = hipGetLastError();
  if (rec) prof_commit(name, e0, e1);
  return e == hipSuccess ? POETX_OK : POETX_ERR_HIP;
}

// Raises kernel `fn`'s dynamic-LDS limit to `bytes` on the current device, once per
// device: `done` is that kernel's record, one bit per device id (ids past 63 set the
// attribute on every call).  Two threads may both set it; the call is idempotent.
inline int lds_limit(const void *fn, size_t bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return POETX_ERR_HIP;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return POETX_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
    return POETX_ERR_HIP;
  if (bit) done.fetch_or(bit, std::memory_order_release);
  return POETX_OK;
}

// ------------------------------------------------------------- bf16 bits ----
typedef uint16_t bf16_t;

__host__ __device__ inline float bf16_to_f32(bf16_t h) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)h << 16;
  return v.f;
}

// Round-to-nearest-even (finite inputs; NaN is not produced by the layer's math).
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } v;
  v.f = f;
  uint32_t r = 0x7FFFu + ((v.u >> 16) & 1u);
  return (bf16_t)((v.u + r) >> 16);
}

// Element loaders widening any stored dtype to float.
__device__ inline float ld_f(const float *p) { return *p; }
__device__ inline float ld_f(const bf16_t *p) { return bf16_to_f32(*p); }
__device__ inline float ld_f(const int8_t *p) { return (float)*p; }
__device__ inline void st_f(float *p, float v) { *p = v; }
__device__ inline void st_f(bf16_t *p, float v) { *p = f32_to_bf16(v); }

inline size_t dtype_size(int dt) { return dt == POETX_F32 ? 4 : dt == POETX_BF16 ? 2 : 1; }

// --------------------------------------------------------------- workspace ----
// Bump allocator over the caller's workspace; with base == nullptr it only
// measures (used for the ws == NULL size query).
struct Arena {
  char *base;
  size_t used = 0;
  explicit Arena(void *b) : base((char *)b) {}
  void *take(size_t bytes) {
    size_t off = (used + 255) & ~(size_t)255;
    used = off + ((bytes + 255) & ~(size_t)255);
    return base ? (void *)(base + off) : nullptr;
  }
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace poetx
