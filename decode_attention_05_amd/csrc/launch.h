// launch.h -- host-side launch descriptors shared by the API layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// Everything one split-K pass needs. Pointers are device pointers.
struct PartialLaunch {
  const uint16_t* q;   // [B, Hq, Sq, D] bf16
  const uint16_t* k;   // [kv_batch, Hkv, capacity, D] bf16
  const uint16_t* v;
  const int32_t* sel;  // sparse only: [B, topk]
  const int32_t* k_len_dev;  // dense, optional: live length(s) read on the device (k_len
                             // then holds their upper bound, the plan's max_k_len)
  int k_lens_stride;         // 0: one length for every sequence; else sequence b's length
                             // is k_len_dev[b * k_lens_stride]
  const int32_t* block_table;  // dense, optional: paged cache [B, max_pages] page ids;
                               // k and v then point at pages [num_pages, Hkv, page_size, D]
  int page_size;             // rows per page, a multiple of the 32-key tile
  int max_pages;             // block-table row length
  int64_t num_pages;
  uint16_t* out;       // [B, Hq, Sq, D] bf16: written directly when S == 1
  float* part_o;       // [B*Hq*Sq, S, D] fp32 unnormalised partial outputs (S > 1); balanced
                       // schedule: [runs, 2, heads_per_wg * Sq, D] with up to
                       // 4 * balanced_wgs runs
  float* part_m;       // [B*Hq*Sq, S] running max, base 2 (S > 1); balanced: [runs, 2,
                       // heads_per_wg * Sq]
  float* part_l;       // [B*Hq*Sq, S] softmax denominators (S > 1); balanced: as part_m
  int balanced_wgs;    // workgroups of the length-balanced schedule (ragged calls)
  int B, Hq, Hkv, G, D;
  int kv_batch;        // sparse: 1 or B; dense: B
  int64_t capacity;
  int64_t k_len;       // dense: attended prefix; sparse: rows usable by sel
  int topk;            // sparse: launch width
  int chunk;           // keys (dense) or selection entries (sparse) per split
  int S;               // number of splits
  int heads_per_wg;    // query heads of one group handled by one workgroup
  int Sq;              // query tokens per sequence: q and out are [B, Hq, Sq, D]; dense
                       // only above 1, heads_per_wg * Sq <= 16
  bool causal;         // Sq > 1: token t sees keys below k_len - Sq + 1 + t
  float qscale;        // softmax_scale * log2(e)
  bool sparse;
};

hipError_t launch_partial(const PartialLaunch& L, hipStream_t stream);
hipError_t launch_combine(const PartialLaunch& L, hipStream_t stream);
// Length-balanced pass over per-sequence device lengths (k_len_dev), and the
// merge of the partials it leaves.
hipError_t launch_balanced(const PartialLaunch& L, hipStream_t stream);
hipError_t launch_balanced_combine(const PartialLaunch& L, hipStream_t stream);

}  // namespace da
