// select.h -- launch descriptor of the on-device selection builder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr int kSelectMaxK = 4096;              // most index entries one token can select
constexpr int kSelectMaxCandidates = 131072;   // most index candidates per token (LDS bitmap)

// Several workgroups per token (decode_attn_build_selection_ws): each filters
// kSelectPartRows candidates, keeping up to kSelectPartCap items for the merge.
constexpr int kSelectPartRows = 4096;
constexpr int kSelectPartCap = 512;
constexpr int kSelectMinSplitRows = 8192;      // fewer candidates: one workgroup per token

struct SelectLaunch {
  const float* scores;   // [B, score_stride] fp32; candidates 0 .. n_idx - 1 of each row
  int64_t score_stride;
  const int32_t* pos;    // [B] 0-based positions of the tokens
  int32_t* sel;          // [B, topk] output
  int B, n_idx, k_idx, window, topk;
  int64_t win_base;      // KV row of window slot 0
  void* ws;              // split builder: per token, 32 part counts then parts x
                         // kSelectPartCap (key, row) items
  int parts;             // split builder: filter workgroups per token
};

// One workgroup per token.
hipError_t launch_select(const SelectLaunch& L, hipStream_t stream);

// Filter workgroups per token, and the workspace bytes of the split builder
// (0: the token count or candidate count takes the one-workgroup builder).
int select_parts(int n_idx);
size_t select_workspace_bytes(int B, int n_idx);

// The split builder: a filter kernel (parts x B workgroups) and a merge kernel
// (one per token). L.ws must hold select_workspace_bytes(B, n_idx) bytes.
hipError_t launch_select_split(const SelectLaunch& L, hipStream_t stream);

}  // namespace da
