// poetx_cnp_noalloc: poetx_cnp with its workspace in a static device array, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops).
#include <atomic>

#include "kernels.h"

namespace poetx {
namespace {

// The workspace of every poetx_cnp_noalloc call on a device.  Host code never uses this
// name as an address (it stands for a host-side shadow): the device address comes from
// hipGetSymbolAddress, once per device, into g_scratch.
static __device__ __align__(256) char scratch[POETX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void *> g_scratch[kMaxDevices];

// This device's address of `scratch`, looked up on its first call (two threads that race
// on a first call look up the same address).
int scratch_ptr(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return POETX_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return POETX_ERR_UNSUPPORTED;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return POETX_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return POETX_OK;
}

}  // namespace
}  // namespace poetx

extern "C" int poetx_cnp_noalloc(int32_t dir, int64_t nblocks, int64_t b, const void *theta, int32_t theta_dtype,
                                 void *g, int32_t g_dtype, const void *dg, int32_t dg_dtype, float *dtheta,
                                 void *stream) {
  using namespace poetx;
  // the requirement first (validates the arguments the query looks at; launches nothing)
  size_t need = 0;
  POETX_TRY(poetx_cnp(dir, nblocks, b, nullptr, theta_dtype, nullptr, g_dtype, nullptr, nullptr, dg_dtype, nullptr,
                      nullptr, &need, nullptr));
  if (need > (size_t)POETX_NOALLOC_SCRATCH_BYTES) return POETX_ERR_WORKSPACE;
  void *ws = nullptr;
  POETX_TRY(scratch_ptr(&ws));
  size_t avail = (size_t)POETX_NOALLOC_SCRATCH_BYTES;
  return poetx_cnp(dir, nblocks, b, theta, theta_dtype, g, g_dtype, nullptr, dg, dg_dtype, dtheta, ws, &avail, stream);
}
