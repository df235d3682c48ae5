// static_scratch.h -- the library-owned workspace of decode_attn_dense_static.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace da {

// Bytes of the per-device static workspace (a plan whose workspace is larger is
// rejected by decode_attn_dense_static).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;

// The current device's static workspace (its device address, looked up once per
// device with that device current). Allocates nothing.
hipError_t static_scratch(void** ptr);

}  // namespace da
