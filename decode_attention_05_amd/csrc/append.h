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

// The Sq new rows of each sequence at the end of its live prefix: row t of
// sequence b goes to row clamp(k_lens[b * k_lens_stride], 0, max_len) - Sq + t
// of a contiguous cache, or through a block table into page pools.
struct AppendRowsLaunch {
  uint16_t* k_cache;        // [B, Hkv, capacity, D] bf16, or pools [num_pages, Hkv, page_size, D]
  uint16_t* v_cache;
  const uint16_t* k_new;    // [B, Hkv, Sq, D] bf16
  const uint16_t* v_new;
  const int32_t* k_lens;    // device lengths, counting the new rows
  int k_lens_stride;
  int64_t max_len;          // lengths are clamped to [0, max_len]
  const int32_t* block_table;  // paged: [B, max_pages] page ids, else null
  int page_size, max_pages;
  int64_t num_pages;
  int B, Hkv, Sq, D;
  int64_t capacity;
};

hipError_t launch_append_rows(const AppendRowsLaunch& L, hipStream_t stream);

// Slot-addressed rows: token n's rows go to row slots[n] % page_size of page
// slots[n] / page_size of the pools; a negative slot or one past the pool is
// skipped.
struct SlotWriteLaunch {
  uint16_t* k_pages;        // [num_pages, Hkv, page_size, D] bf16
  uint16_t* v_pages;
  const uint16_t* k_rows;   // [N, Hkv, D] bf16
  const uint16_t* v_rows;
  const int64_t* slots;     // [N] device slot indices
  int N, Hkv, D, page_size;
  int64_t num_pages;
};

hipError_t launch_write_slots(const SlotWriteLaunch& L, hipStream_t stream);

}  // namespace da
