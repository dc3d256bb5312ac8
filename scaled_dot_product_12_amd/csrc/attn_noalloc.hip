// attn_noalloc.hip -- the device-resident scratch array behind attn_bwd_noalloc,
// the backward entry point for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// The backward's one scratch buffer is delta (B*H*M fp32 values: the dQ kernel
// writes delta_i = rowsum(O_i * dO_i), the dK/dV kernel reads it). Here it
// lives in a file-scope __device__ array of a fixed maximum size that every
// GPU the library runs on holds until the process ends. Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and cached; the kernels receive that address like any workspace pointer.
// The host-side name of the array is only a stand-in and is never passed to
// a kernel or a copy. Nothing needs clearing between calls: the dQ kernel
// writes every delta the dK/dV kernel reads, in stream order. Calls that
// overlap on one GPU (different streams) share the array and race.

#include <mutex>

#include "attn_launch.h"

namespace mi355 {

namespace {

static __device__ __align__(256) float scratch[kNoallocMaxRows];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
float* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_delta_scratch(float** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? (float*)p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  if (!g_ptr[dev]) return hipErrorInvalidSymbol;
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mi355
