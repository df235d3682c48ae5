// probe.h -- launch of the streaming-read ceiling probe (diagnostics).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int cus,
                             hipStream_t stream);

}  // namespace da
