// append.h -- launch descriptor of the KV append / ring write.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

struct AppendLaunch {
  uint16_t* k_cache;        // [B, Hkv, capacity, D] bf16
  uint16_t* v_cache;
  const uint16_t* k_new;    // [B, Hkv, 1, D] bf16
  const uint16_t* v_new;
  const int32_t* pos;       // [B] device positions
  int B, Hkv, D;
  int64_t capacity;
  int window;               // 0: row = pos; > 0: row = win_base + pos % window
  int64_t win_base;
};

hipError_t launch_append(const AppendLaunch& L, hipStream_t stream);

}  // namespace da
