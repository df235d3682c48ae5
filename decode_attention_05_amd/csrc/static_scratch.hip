// static_scratch.hip -- the library-owned workspace of decode_attn_dense_static.
//
// Callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc) take the split partials from this
// file-scope device array instead of a caller-owned workspace. Each device
// holds its own copy, zero-filled when the code object loads, for the life of
// the process. In host code the array's name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, looked up once
// per device and kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "static_scratch.h"

namespace da {

namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace da
