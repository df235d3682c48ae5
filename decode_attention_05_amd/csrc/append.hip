// append.hip -- writes the current token's K and V rows into the capacity cache.
//
// The decode step appends the new token before attending: at row pos for a
// linear cache (fuel-dispatch page "DecodeFlashSpec", field k_len: the live
// length is the cached length plus the new token), or at ring row
// win_base + pos % window for a sliding window (metrale page "AttnV41",
// decode_body: the window ring write with its slot read on the device). The
// position comes from device memory, so the write can sit in a captured graph
// next to the attention call. A position that is negative or lands outside the
// cache writes nothing.
//
// One thread per 16-byte chunk of a (token, kv head, K or V) row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "append.h"

namespace da {

namespace {

__global__ __launch_bounds__(256) void append_kv_kernel(AppendLaunch a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int chunks = a.D / 8;
  const int64_t per_row = chunks;
  const int64_t rows = (int64_t)a.B * a.Hkv;
  if (t >= 2 * rows * per_row) return;
  const int which = (int)(t / (rows * per_row));  // 0: K, 1: V
  const int64_t r = t % (rows * per_row);
  const int64_t bh = r / per_row;
  const int c = (int)(r % per_row);
  const int b = (int)(bh / a.Hkv);
  const int64_t p = a.pos[b];
  if (p < 0) return;
  const int64_t row = a.window > 0 ? a.win_base + p % a.window : p;
  if (row < 0 || row >= a.capacity) return;
  const uint4* src = reinterpret_cast<const uint4*>(which ? a.v_new : a.k_new) + bh * chunks + c;
  uint4* dst = reinterpret_cast<uint4*>(which ? a.v_cache : a.k_cache) +
               (bh * a.capacity + row) * chunks + c;
  *dst = *src;
}

}  // namespace

hipError_t launch_append(const AppendLaunch& L, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)L.B * L.Hkv * (L.D / 8);
  const int64_t blocks = (total + 255) / 256;
  if (total <= 0 || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, L);
  return hipGetLastError();
}

}  // namespace da
