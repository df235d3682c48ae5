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
// One thread per 16-byte chunk of a (token, kv head, K or V) row. The rows of
// a one-call decode pass (several new rows per sequence, at the end of its
// live prefix read on the device, contiguous or paged) use append_rows_kernel.
// write_slots_kernel writes rows to slots named one per token in device memory
// (metrale page "DflashScratch", field slot_mapping_dev: 64-bit paged-cache
// slot indices consumed by a reshape-and-cache write).
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

// One thread per 16-byte chunk of a (sequence, kv head, new row, K or V) row. A
// row before the start of the cache (a length below Sq) or on a page id
// outside the pool is not written.
__global__ __launch_bounds__(256) void append_rows_kernel(AppendRowsLaunch a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int chunks = a.D / 8;
  const int64_t per_side = (int64_t)a.B * a.Hkv * a.Sq * chunks;
  if (t >= 2 * per_side) return;
  const int which = (int)(t / per_side);  // 0: K, 1: V
  int64_t r = t % per_side;
  const int c = (int)(r % chunks);
  r /= chunks;
  const int s = (int)(r % a.Sq);
  const int64_t bh = r / a.Sq;            // b * Hkv + h
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  int64_t len = a.k_lens[(int64_t)b * a.k_lens_stride];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int64_t row = len - a.Sq + s;
  if (row < 0) return;
  int64_t dst_row;
  if (a.block_table) {
    const int64_t page = a.block_table[(int64_t)b * a.max_pages + row / a.page_size];
    if (page < 0 || page >= a.num_pages) return;
    dst_row = (page * a.Hkv + h) * a.page_size + row % a.page_size;
  } else {
    dst_row = bh * a.capacity + row;
  }
  const uint4* src = reinterpret_cast<const uint4*>(which ? a.v_new : a.k_new) + r * chunks + c;
  uint4* dst = reinterpret_cast<uint4*>(which ? a.v_cache : a.k_cache) + dst_row * chunks + c;
  *dst = *src;
}

// One thread per 16-byte chunk of a (token, kv head, K or V) row. Slot s names
// row s % page_size of page s / page_size; a negative slot (a padding token)
// or a slot past the pool writes nothing.
__global__ __launch_bounds__(256) void write_slots_kernel(SlotWriteLaunch a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int chunks = a.D / 8;
  const int64_t per_side = (int64_t)a.N * a.Hkv * chunks;
  if (t >= 2 * per_side) return;
  const int which = (int)(t / per_side);  // 0: K, 1: V
  const int64_t r = t % per_side;          // (token, head, chunk)
  const int c = (int)(r % chunks);
  const int64_t nh = r / chunks;           // n * Hkv + h
  const int64_t n = nh / a.Hkv;
  const int h = (int)(nh % a.Hkv);
  const int64_t slot = a.slots[n];
  if (slot < 0 || slot / a.page_size >= a.num_pages) return;
  const int64_t page = slot / a.page_size, row = slot % a.page_size;
  const uint4* src = reinterpret_cast<const uint4*>(which ? a.v_rows : a.k_rows) + r;
  uint4* dst = reinterpret_cast<uint4*>(which ? a.v_pages : a.k_pages) +
               ((page * a.Hkv + h) * a.page_size + row) * chunks + c;
  *dst = *src;
}

}  // namespace

hipError_t launch_write_slots(const SlotWriteLaunch& L, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)L.N * L.Hkv * (L.D / 8);
  const int64_t blocks = (total + 255) / 256;
  if (total <= 0 || blocks > 0x7fffffff || L.D % 8 != 0 || L.page_size < 1 || L.num_pages < 1)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(write_slots_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, L);
  return hipGetLastError();
}

hipError_t launch_append_rows(const AppendRowsLaunch& L, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)L.B * L.Hkv * L.Sq * (L.D / 8);
  const int64_t blocks = (total + 255) / 256;
  if (total <= 0 || blocks > 0x7fffffff || L.D % 8 != 0) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(append_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, L);
  return hipGetLastError();
}

hipError_t launch_append(const AppendLaunch& L, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)L.B * L.Hkv * (L.D / 8);
  const int64_t blocks = (total + 255) / 256;
  if (total <= 0 || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, L);
  return hipGetLastError();
}

}  // namespace da
