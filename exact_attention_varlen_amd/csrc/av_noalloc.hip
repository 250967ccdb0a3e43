// av_noalloc.hip — the device scratch of the allocation-free backward entry
// point (attn_varlen_bwd_noalloc): a file-scope device array that holds the
// backward's workspace (the row terms Delta and lse2, and at head_dim 256 the
// partial dK / dV sums), so that callers who cannot allocate device memory
// (code under HIP graph capture, tight serving loops) can still run the
// backward.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends. Host code must not pass the array's name to
// a kernel (in host code it is a host-side stand-in, not a device address): its
// device address is looked up once per device, with that device current, and
// only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "../../include/attn_varlen.h"
#include "av_launch.h"

namespace av {

namespace {

constexpr size_t kScratchBytes = ATTN_VARLEN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace av
