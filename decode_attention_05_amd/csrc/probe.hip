// probe.hip -- the measured streaming-read ceiling (diagnostics, not part of
// the operation): a plain read of a buffer with the attention kernels' load
// style (16-byte non-temporal vector loads), its bytes folded into one word so
// the reads cannot be dropped. One 256-thread workgroup per compute unit, each
// reading one contiguous share with sixteen loads in flight per thread: the
// fastest of the shapes measured on MI355X (4 GiB: 7.22 TB/s, against 7.17 for
// two workgroups per CU with eight loads and 6.24 for one with eight).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "probe.h"

namespace da {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 16;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p,
                                                                    int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  uint32_t acc = 0u;
  constexpr int64_t kStep = (int64_t)kProbeThreads * kProbeLoads;
  int64_t i = begin + threadIdx.x;
  // whole steps: every load in range, all issued before any is used
  for (; i + kStep - threadIdx.x <= end; i += kStep) {
    u32x4 r[kProbeLoads];
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u)
      r[u] = __builtin_nontemporal_load(p + i + (int64_t)kProbeThreads * u);
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u) acc ^= r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3];
  }
  // the rest of the share, one load at a time
  for (; i < end; i += kProbeThreads) {
    const u32x4 r = __builtin_nontemporal_load(p + i);
    acc ^= r[0] ^ r[1] ^ r[2] ^ r[3];
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int cus,
                             hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 != 0 || cus < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)cus), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace da
