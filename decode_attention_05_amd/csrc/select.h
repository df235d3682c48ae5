// select.h -- launch descriptor of the on-device selection builder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr int kSelectMaxK = 4096;              // most index entries one token can select
constexpr int kSelectMaxCandidates = 131072;   // most index candidates per token (LDS bitmap)

struct SelectLaunch {
  const float* scores;   // [B, score_stride] fp32; candidates 0 .. n_idx - 1 of each row
  int64_t score_stride;
  const int32_t* pos;    // [B] 0-based positions of the tokens
  int32_t* sel;          // [B, topk] output
  int B, n_idx, k_idx, window, topk;
  int64_t win_base;      // KV row of window slot 0
};

hipError_t launch_select(const SelectLaunch& L, hipStream_t stream);

}  // namespace da
