// api.cpp -- the C ABI of the decode-attention library: problem validation, the
// split-K plan, and the entry points (dense with a host, device or per-sequence
// length, paged, the one-call pass, sparse, the selection builder, the KV
// append, the slot-addressed KV write, and diagnostics). Host code only; the
// kernels live in kernels.hip, select.hip, append.hip and probe.hip.
//
// The problem statement follows the fuel-dispatch page "DecodeFlashSpec"
// (shapes of q, k, v; softmax_scale; k_len as the live prefix, counting the
// query tokens of the pass; causal accepted and ignored for one token, applied
// to the last Sq positions of the prefix for several; ALiBi, windows and
// softcap rejected); the sparse call follows
// the metrale page "AttnV41" (decode_fixed_topk: a fixed launch width padded
// with -1). Validation fails closed on host-visible values only, and no call
// synchronises or copies, as the flashinfer page "packed_fused_kda_decode"
// describes for caller-owned, graph-stable buffers.
#include "../../include/decode_attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "append.h"
#include "launch.h"
#include "probe.h"
#include "select.h"
#include "static_scratch.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_ev_before = nullptr;  // optional timing of the partial kernel
thread_local hipEvent_t g_ev_after = nullptr;

decode_attn_status fail(decode_attn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

decode_attn_status ok() {
  g_last_error[0] = '\0';
  return DA_OK;
}

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("DECODE_ATTN_LOG");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

// Compute units per device, queried once per device id.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_cache[kMaxDevices];

decode_attn_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) {
    int c = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return DA_OK;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || c <= 0)
    return fail(DA_ERR_HIP, "querying the compute-unit count failed: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) g_cu_cache[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return DA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// --- split-K heuristic -------------------------------------------------------
//
// The hot path is bound by HBM bandwidth, so the grid must keep every CU
// streaming, in one round of equally sized workgroups. Each CU's read rate is
// close to its own limit when it holds one 4-wave workgroup, so a CU given more
// workgroups than another finishes last (measured: 288 workgroups on 256 CUs run
// 57% slower than 256), and two per CU contend for HBM without reading faster
// (512 workgroups of half the keys run 2-3% slower than 256). A unit (batch, kv
// head, head tile) is split only when there are fewer units than CUs, into
// CUs / units splits (rounded down: a CU left idle costs less than a CU given
// two), and never below kMinChunk keys per split: below that the split merge
// costs more than the streaming it spreads. The selection gather is bound by
// latency instead, so sparse chunks are sized for kResidentPerCu workgroups per
// CU, and never below kMinSparseChunk selection entries.
constexpr int kResidentPerCu = 2;
constexpr int kMinChunk = 1024;
constexpr int kMinSparseChunk = 128;
constexpr int kKeyAlign = 32;  // the kernel's key tile: splits start on tile (and page) edges
constexpr int kMaxSplits = 1 << 16;

// Splits per unit that give every CU at most per_cu workgroups in one round
// (1 when units >= CUs).
int64_t splits_for_occupancy(int64_t units, int cus, int per_cu) {
  if (units >= cus) return 1;
  return std::max<int64_t>(1, (int64_t)per_cu * cus / units);
}

// Query heads per workgroup: the largest divisor of G whose rows (heads times
// tokens) fit the 16 columns of one MFMA tile.
int heads_per_wg(int G, int Sq) {
  for (int gt = 16 / Sq; gt > 1; --gt)
    if (G % gt == 0) return gt;
  return 1;
}

constexpr int kMaxSeqQ = 16;

// Number of splits and keys per split for one dense call of length k_len.
void dense_split(const decode_attn_plan_t& P, int64_t k_len, int* S_out, int* chunk_out,
                 int* bound_out) {
  const auto& p = P.prob;
  const int gt = heads_per_wg(P.group, p.seq_q);
  const int64_t units = (int64_t)p.batch * p.num_kv_heads * (P.group / gt);
  int64_t chunk, S, bound;
  if (p.force_chunk > 0) {
    chunk = p.force_chunk;
    S = ceil_div(k_len, chunk);
    bound = S;
  } else {
    int64_t target = p.force_splits > 0 ? p.force_splits : splits_for_occupancy(units, P.num_cus, 1);
    const int64_t min_chunk = p.force_splits > 0 ? 1 : kMinChunk;
    int64_t s0 = std::min<int64_t>(target, ceil_div(k_len, min_chunk));
    s0 = std::max<int64_t>(1, std::min<int64_t>(s0, kMaxSplits));
    bound = s0;
    chunk = round_up(ceil_div(k_len, s0), p.force_splits > 0 ? 1 : kKeyAlign);
    S = ceil_div(k_len, chunk);
  }
  *S_out = (int)S;
  *chunk_out = (int)chunk;
  if (bound_out) *bound_out = (int)bound;
}

decode_attn_status validate_problem(const decode_attn_problem& p) {
  if (p.has_alibi) return fail(DA_ERR_UNSUPPORTED, "alibi: ALiBi slopes are not supported");
  if (p.window_left != -1)
    return fail(DA_ERR_UNSUPPORTED, "window_left: sliding windows are not supported");
  if (p.window_right != -1)
    return fail(DA_ERR_UNSUPPORTED, "window_right: sliding windows are not supported");
  if (p.has_softcap) return fail(DA_ERR_UNSUPPORTED, "softcap: logit softcap is not supported");
  if (p.seq_q < 1 || p.seq_q > kMaxSeqQ)
    return fail(DA_ERR_UNSUPPORTED, "seq_q: 1 to %d query tokens per sequence are supported, got %d",
                kMaxSeqQ, p.seq_q);
  if (p.seq_q > 1 && p.topk_max > 0)
    return fail(DA_ERR_UNSUPPORTED, "seq_q: the sparse call takes one query token per sequence");
  if (p.head_dim != 64 && p.head_dim != 128)
    return fail(DA_ERR_UNSUPPORTED, "head_dim: only 64 and 128 are supported, got %d", p.head_dim);
  if (p.batch < 1 || p.num_q_heads < 1 || p.num_kv_heads < 1)
    return fail(DA_ERR_INVALID_ARG, "batch, num_q_heads and num_kv_heads must be >= 1");
  if (p.num_q_heads % p.num_kv_heads != 0)
    return fail(DA_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                p.num_q_heads, p.num_kv_heads);
  if (p.capacity < 1) return fail(DA_ERR_INVALID_ARG, "capacity must be >= 1");
  if (p.max_k_len < 1 || p.max_k_len > p.capacity)
    return fail(DA_ERR_INVALID_ARG, "max_k_len must lie in [1, capacity], got %lld",
                (long long)p.max_k_len);
  if (p.topk_max < 0) return fail(DA_ERR_INVALID_ARG, "topk_max must be >= 0");
  if (p.topk_max > 0) {
    if (p.kv_batch != 1 && p.kv_batch != p.batch)
      return fail(DA_ERR_INVALID_ARG, "kv_batch must be 1 or batch for a sparse plan, got %d",
                  p.kv_batch);
  } else if (p.kv_batch != 0 && p.kv_batch != p.batch) {
    return fail(DA_ERR_INVALID_ARG, "kv_batch must be 0 or batch for a dense plan, got %d",
                p.kv_batch);
  }
  if (p.ragged != 0 && p.ragged != 1)
    return fail(DA_ERR_INVALID_ARG, "ragged must be 0 or 1, got %d", p.ragged);
  if (p.ragged && p.topk_max > 0)
    return fail(DA_ERR_UNSUPPORTED, "ragged: per-sequence lengths are dense-only");
  if (p.page_size != 0) {
    if (p.topk_max > 0) return fail(DA_ERR_UNSUPPORTED, "page_size: paged caches are dense-only");
    if (p.page_size < 32 || p.page_size % 32 != 0)
      return fail(DA_ERR_INVALID_ARG, "page_size must be a positive multiple of 32, got %d",
                  p.page_size);
    if (p.max_pages_per_seq < 1 || p.num_pages < 1)
      return fail(DA_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
    if (p.capacity != (int64_t)p.page_size * p.max_pages_per_seq)
      return fail(DA_ERR_INVALID_ARG, "capacity must equal page_size * max_pages_per_seq");
  }
  if (p.force_chunk % 32 != 0 && p.page_size != 0)
    return fail(DA_ERR_INVALID_ARG, "force_chunk must be a multiple of 32 for a paged plan");
  if (p.num_cus < 0 || p.force_splits < 0 || p.force_chunk < 0)
    return fail(DA_ERR_INVALID_ARG, "num_cus, force_splits and force_chunk must be >= 0");
  // The kernels address a KV row by a 32-bit byte offset inside one (batch, kv
  // head) slab of capacity * head_dim bf16.
  if ((double)p.capacity * p.head_dim * 2.0 >= 4294967296.0)
    return fail(DA_ERR_UNSUPPORTED, "capacity: one kv head's rows must span less than 4 GiB");
  // Element counts must fit the 64-bit index arithmetic with ample margin.
  const double elems = (double)p.batch * p.num_kv_heads * (double)p.capacity * p.head_dim;
  if (elems > 9.0e15) return fail(DA_ERR_INVALID_ARG, "KV buffer too large");
  if ((int64_t)p.batch * p.num_q_heads * p.seq_q > 0x7fffffff)
    return fail(DA_ERR_INVALID_ARG, "batch * num_q_heads too large");
  return DA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

da::PartialLaunch base_launch(const decode_attn_plan_t& P, const void* q, const void* k,
                              const void* v, void* out, float scale, int64_t k_len,
                              void* workspace, int S) {
  const auto& p = P.prob;
  da::PartialLaunch L{};
  L.q = static_cast<const uint16_t*>(q);
  L.k = static_cast<const uint16_t*>(k);
  L.v = static_cast<const uint16_t*>(v);
  L.out = static_cast<uint16_t*>(out);
  L.B = p.batch;
  L.Hq = p.num_q_heads;
  L.Hkv = p.num_kv_heads;
  L.G = P.group;
  L.D = p.head_dim;
  L.kv_batch = p.kv_batch;
  L.capacity = p.capacity;
  L.k_len = k_len;
  L.S = S;
  L.heads_per_wg = heads_per_wg(P.group, p.seq_q);
  L.Sq = p.seq_q;
  L.causal = p.causal != 0;
  L.qscale = scale * 1.4426950408889634f;  // log2(e): the kernels use exp2
  const int64_t rows = (int64_t)p.batch * p.num_q_heads * p.seq_q;
  float* ws = static_cast<float*>(workspace);
  L.part_o = S > 1 ? ws : nullptr;
  L.part_m = S > 1 ? ws + rows * S * p.head_dim : nullptr;
  L.part_l = S > 1 ? ws + rows * S * (p.head_dim + 1) : nullptr;
  return L;
}

uint64_t workspace_for(const decode_attn_problem& p, int S) {
  if (S <= 1) return 0;
  return (uint64_t)p.batch * p.num_q_heads * p.seq_q * (uint64_t)S * (p.head_dim + 2) *
         sizeof(float);
}

// Length-balanced schedule: two partial slots of (heads per workgroup) x
// (tokens) rows per run, and up to one run per wave (4 per workgroup).
constexpr int kWavesPerWg = 4;
uint64_t balanced_workspace(const decode_attn_plan_t& P) {
  return (uint64_t)P.balanced_wgs * kWavesPerWg * 2 * heads_per_wg(P.group, P.prob.seq_q) *
         P.prob.seq_q * (P.prob.head_dim + 2) * sizeof(float);
}

decode_attn_status check_common(const decode_attn_plan_t* plan, int kind, const void* q,
                                const void* k, const void* v, void* out, float scale,
                                void* workspace, size_t workspace_bytes) {
  if (!plan) return fail(DA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->kind != kind)
    return fail(DA_ERR_INVALID_ARG, kind ? "plan is a dense plan; use decode_attn_dense"
                                         : "plan is a sparse plan; use decode_attn_sparse");
  if (!q || !k || !v || !out) return fail(DA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(DA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(DA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (plan->workspace_bytes > 0) {
    if (!workspace) return fail(DA_ERR_WORKSPACE, "workspace is NULL but the plan needs %llu bytes",
                                (unsigned long long)plan->workspace_bytes);
    if (workspace_bytes < plan->workspace_bytes)
      return fail(DA_ERR_WORKSPACE, "workspace has %zu bytes, the plan needs %llu", workspace_bytes,
                  (unsigned long long)plan->workspace_bytes);
    if (!aligned16(workspace)) return fail(DA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  return DA_OK;
}

decode_attn_status run(const da::PartialLaunch& L, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (g_ev_before) {
    e = hipEventRecord(g_ev_before, st);
    if (e != hipSuccess) return fail(DA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  }
  e = da::launch_partial(L, st);
  if (e != hipSuccess) return fail(DA_ERR_HIP, "partial kernel launch failed: %s", hipGetErrorString(e));
  if (g_ev_after) {
    e = hipEventRecord(g_ev_after, st);
    if (e != hipSuccess) return fail(DA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  }
  if (L.S > 1) {
    e = da::launch_combine(L, st);
    if (e != hipSuccess)
      return fail(DA_ERR_HIP, "combine kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}


decode_attn_status dense_with_lengths(const decode_attn_plan_t* plan, const void* q,
                                      const void* k, const void* v, const int32_t* block_table,
                                      const int32_t* k_lens, int32_t k_lens_stride, void* out,
                                      float softmax_scale, void* workspace,
                                      size_t workspace_bytes, void* stream,
                                      const void* k_new = nullptr, const void* v_new = nullptr) {
  decode_attn_status s =
      check_common(plan, 0, q, k, v, out, softmax_scale, workspace, workspace_bytes);
  if (s != DA_OK) return s;
  const bool paged = block_table != nullptr;
  if (paged != (plan->prob.page_size > 0))
    return fail(DA_ERR_INVALID_ARG, paged ? "a paged call needs a plan with page_size > 0"
                                          : "a paged plan needs decode_attn_dense_paged");
  if (plan->balanced_wgs < 1 || plan->workspace_bytes < balanced_workspace(*plan))
    return fail(DA_ERR_INVALID_ARG, "per-sequence lengths need a plan made with ragged = 1");
  if (!k_lens) return fail(DA_ERR_INVALID_ARG, "k_lens must be non-NULL");
  if (((uintptr_t)k_lens & 3u) || (paged && ((uintptr_t)block_table & 3u)))
    return fail(DA_ERR_INVALID_ARG, "k_lens and block_table must be 4-byte aligned");
  if (k_lens_stride < 1) return fail(DA_ERR_INVALID_ARG, "k_lens_stride must be >= 1");
  da::PartialLaunch L =
      base_launch(*plan, q, k, v, out, softmax_scale, plan->prob.max_k_len, nullptr, 1);
  L.k_len_dev = k_lens;
  L.k_lens_stride = k_lens_stride;
  L.sparse = false;
  L.balanced_wgs = plan->balanced_wgs;
  const int64_t slots = (int64_t)plan->balanced_wgs * kWavesPerWg * 2 * L.heads_per_wg * L.Sq;
  float* ws = static_cast<float*>(workspace);
  L.part_o = ws;
  L.part_m = ws + slots * plan->prob.head_dim;
  L.part_l = L.part_m + slots;
  if (paged) {
    L.block_table = block_table;
    L.page_size = plan->prob.page_size;
    L.max_pages = plan->prob.max_pages_per_seq;
    L.num_pages = plan->prob.num_pages;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (k_new) {
    // The pass's new rows first (one small kernel), then the attention reads
    // them from the cache like every other row.
    da::AppendRowsLaunch A{};
    A.k_cache = const_cast<uint16_t*>(static_cast<const uint16_t*>(k));
    A.v_cache = const_cast<uint16_t*>(static_cast<const uint16_t*>(v));
    A.k_new = static_cast<const uint16_t*>(k_new);
    A.v_new = static_cast<const uint16_t*>(v_new);
    A.k_lens = k_lens;
    A.k_lens_stride = k_lens_stride;
    A.max_len = plan->prob.max_k_len;
    A.block_table = block_table;
    A.page_size = plan->prob.page_size;
    A.max_pages = plan->prob.max_pages_per_seq;
    A.num_pages = plan->prob.num_pages;
    A.B = plan->prob.batch;
    A.Hkv = plan->prob.num_kv_heads;
    A.Sq = plan->prob.seq_q;
    A.D = plan->prob.head_dim;
    A.capacity = plan->prob.capacity;
    e = da::launch_append_rows(A, st);
    if (e != hipSuccess)
      return fail(DA_ERR_HIP, "append kernel launch failed: %s", hipGetErrorString(e));
  }
  if (g_ev_before) {
    e = hipEventRecord(g_ev_before, st);
    if (e != hipSuccess) return fail(DA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  }
  e = da::launch_balanced(L, st);
  if (e != hipSuccess)
    return fail(DA_ERR_HIP, "balanced kernel launch failed: %s", hipGetErrorString(e));
  if (g_ev_after) {
    e = hipEventRecord(g_ev_after, st);
    if (e != hipSuccess) return fail(DA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  }
  e = da::launch_balanced_combine(L, st);
  if (e != hipSuccess)
    return fail(DA_ERR_HIP, "balanced combine launch failed: %s", hipGetErrorString(e));
  return ok();
}

decode_attn_status select_launch(const decode_attn_select_problem* p, const float* scores,
                                 const int32_t* pos, int32_t* sel, da::SelectLaunch* L) {
  if (!p) return fail(DA_ERR_INVALID_ARG, "problem pointer must be non-NULL");
  if (p->batch < 1 || p->topk < 1 || p->n_idx < 0 || p->window < 0 || p->k_idx < 0)
    return fail(DA_ERR_INVALID_ARG, "batch and topk must be >= 1; n_idx, window, k_idx >= 0");
  if (p->k_idx > da::kSelectMaxK)
    return fail(DA_ERR_INVALID_ARG, "k_idx must be <= %d, got %d", da::kSelectMaxK, p->k_idx);
  if (p->n_idx > da::kSelectMaxCandidates)
    return fail(DA_ERR_UNSUPPORTED, "n_idx: at most %d index candidates per token, got %d",
                da::kSelectMaxCandidates, p->n_idx);
  if (p->score_stride < p->n_idx || p->score_stride < 1)
    return fail(DA_ERR_INVALID_ARG, "score_stride must be >= max(n_idx, 1)");
  if (p->win_base < 0 || p->win_base + p->window > 0x7fffffffLL)
    return fail(DA_ERR_INVALID_ARG, "window rows must lie in [0, 2^31)");
  if (p->n_idx > 0x7fffffff - 1 || (int64_t)p->batch * p->topk > 0x7fffffffLL)
    return fail(DA_ERR_INVALID_ARG, "selection too large");
  if (!pos || !sel) return fail(DA_ERR_INVALID_ARG, "pos and sel must be non-NULL");
  if (((uintptr_t)pos & 3u) || ((uintptr_t)sel & 3u))
    return fail(DA_ERR_INVALID_ARG, "pos and sel must be 4-byte aligned");
  if (p->k_idx > 0 && p->n_idx > 0) {
    if (!scores) return fail(DA_ERR_INVALID_ARG, "scores must be non-NULL when k_idx > 0");
    if (((uintptr_t)scores & 15u) || (p->score_stride & 3))
      return fail(DA_ERR_INVALID_ARG,
                  "scores must be 16-byte aligned with a row stride that is a multiple of 4");
  }
  *L = da::SelectLaunch{};
  L->scores = scores;
  L->score_stride = p->score_stride;
  L->pos = pos;
  L->sel = sel;
  L->B = p->batch;
  L->n_idx = p->n_idx;
  L->k_idx = p->k_idx;
  L->window = p->window;
  L->topk = p->topk;
  L->win_base = p->win_base;
  return DA_OK;
}

}  // namespace

extern "C" {

decode_attn_status decode_attn_plan(const decode_attn_problem* p, decode_attn_plan_t* out) {
  if (!p || !out) return fail(DA_ERR_INVALID_ARG, "problem and plan pointers must be non-NULL");
  decode_attn_status s = validate_problem(*p);
  if (s != DA_OK) return s;
  decode_attn_plan_t P;
  std::memset(&P, 0, sizeof P);
  P.prob = *p;
  P.group = p->num_q_heads / p->num_kv_heads;
  P.kind = p->topk_max > 0 ? 1 : 0;
  if (P.kind == 0 && p->force_splits == 0 && p->force_chunk == 0) {
    // Tuning runs only: DECODE_ATTN_SPLITS=<n> caps the dense split count as
    // force_splits would (anything but a positive integer is ignored).
    const char* e = std::getenv("DECODE_ATTN_SPLITS");
    if (e && e[0]) {
      char* end = nullptr;
      const long v = std::strtol(e, &end, 10);
      if (end && *end == '\0' && v >= 1 && v <= kMaxSplits) {
        P.prob.force_splits = (int32_t)v;
        if (log_enabled()) std::fprintf(stderr, "[decode_attn] DECODE_ATTN_SPLITS=%ld\n", v);
      }
    }
  }
  if (P.kind == 0) P.prob.kv_batch = p->batch;
  int cus = p->num_cus;
  if (cus == 0) {
    s = device_cus(&cus);
    if (s != DA_OK) return s;
  }
  P.num_cus = cus;
  const int gt = heads_per_wg(P.group, p->seq_q);
  const int64_t units = (int64_t)p->batch * p->num_kv_heads * (P.group / gt);
  if (P.kind == 0) {
    int S = 0, chunk = 0, bound = 0;
    dense_split(P, p->max_k_len, &S, &chunk, &bound);
    P.num_splits_max = bound;
    P.chunk = chunk;
  } else {
    // The chunk depends on the plan only (never on a call's topk), which is what
    // makes padding to any launch width bit-exact.
    int64_t chunk;
    if (p->force_chunk > 0) {
      chunk = p->force_chunk;
    } else {
      const int64_t per_unit = splits_for_occupancy(units, cus, kResidentPerCu);
      chunk = round_up(ceil_div(p->topk_max, per_unit), kKeyAlign);
      chunk = std::max<int64_t>(chunk, std::min<int64_t>(kMinSparseChunk, round_up(p->topk_max, kKeyAlign)));
    }
    const int64_t S = ceil_div(p->topk_max, chunk);
    if (S > kMaxSplits) return fail(DA_ERR_INVALID_ARG, "force_chunk gives too many splits");
    P.chunk = (int)chunk;
    P.num_splits_max = (int)S;
  }
  if (P.num_splits_max > kMaxSplits) return fail(DA_ERR_INVALID_ARG, "too many splits");
  P.workspace_bytes = workspace_for(P.prob, P.num_splits_max);
  if (P.kind == 0 && (p->ragged || p->page_size > 0)) {
    P.prob.ragged = 1;
    // Two workgroups per CU: the schedule's piece boundaries leave bubbles in
    // one workgroup's stream that the other fills (measured faster than one).
    P.balanced_wgs = kResidentPerCu * cus;
    P.workspace_bytes = std::max(P.workspace_bytes, balanced_workspace(P));
  }
  if (log_enabled())
    std::fprintf(stderr,
                 "[decode_attn] plan kind=%s B=%d Hq=%d Hkv=%d D=%d G=%d heads/wg=%d units=%lld "
                 "cus=%d splits_max=%d chunk=%d workspace=%llu\n",
                 P.kind ? "sparse" : "dense", p->batch, p->num_q_heads, p->num_kv_heads,
                 p->head_dim, P.group, gt, (long long)units, cus, P.num_splits_max, P.chunk,
                 (unsigned long long)P.workspace_bytes);
  *out = P;
  return ok();
}

decode_attn_status decode_attn_dense(const decode_attn_plan_t* plan, const void* q, const void* k,
                                     const void* v, void* out, float softmax_scale, int64_t k_len,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  decode_attn_status s =
      check_common(plan, 0, q, k, v, out, softmax_scale, workspace, workspace_bytes);
  if (s != DA_OK) return s;
  if (plan->prob.page_size > 0)
    return fail(DA_ERR_INVALID_ARG, "a paged plan needs decode_attn_dense_paged");
  if (k_len < 1 || k_len > plan->prob.max_k_len)
    return fail(DA_ERR_INVALID_ARG, "k_len must lie in [1, max_k_len = %lld], got %lld",
                (long long)plan->prob.max_k_len, (long long)k_len);
  if (plan->prob.causal && k_len < plan->prob.seq_q)
    return fail(DA_ERR_INVALID_ARG,
                "k_len (%lld) counts the %d query tokens and must be at least that many",
                (long long)k_len, plan->prob.seq_q);
  int S = 0, chunk = 0;
  dense_split(*plan, k_len, &S, &chunk, nullptr);
  if (S > plan->num_splits_max)
    return fail(DA_ERR_INVALID_ARG, "internal: %d splits exceed the plan's %d", S,
                plan->num_splits_max);
  da::PartialLaunch L = base_launch(*plan, q, k, v, out, softmax_scale, k_len, workspace, S);
  L.chunk = chunk;
  L.sparse = false;
  if (log_enabled())
    std::fprintf(stderr, "[decode_attn] dense k_len=%lld splits=%d chunk=%d\n", (long long)k_len, S,
                 chunk);
  return run(L, stream);
}

decode_attn_status decode_attn_dense_static(const decode_attn_plan_t* plan, const void* q,
                                            const void* k, const void* v, void* out,
                                            float softmax_scale, int64_t k_len, void* stream) {
  if (!plan) return fail(DA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->workspace_bytes > da::kStaticScratchBytes)
    return fail(DA_ERR_WORKSPACE,
                "the plan needs %llu bytes of workspace; the static workspace holds %zu "
                "(use decode_attn_dense with a caller-owned workspace)",
                (unsigned long long)plan->workspace_bytes, da::kStaticScratchBytes);
  void* ws = nullptr;
  if (plan->workspace_bytes > 0) {
    const hipError_t e = da::static_scratch(&ws);
    if (e != hipSuccess)
      return fail(DA_ERR_HIP, "looking up the static workspace failed: %s", hipGetErrorString(e));
  }
  return decode_attn_dense(plan, q, k, v, out, softmax_scale, k_len, ws,
                           ws ? (size_t)da::kStaticScratchBytes : 0, stream);
}

decode_attn_status decode_attn_dense_devlen(const decode_attn_plan_t* plan, const void* q,
                                            const void* k, const void* v, void* out,
                                            float softmax_scale, const int32_t* k_len_dev,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
  decode_attn_status s =
      check_common(plan, 0, q, k, v, out, softmax_scale, workspace, workspace_bytes);
  if (s != DA_OK) return s;
  if (plan->prob.page_size > 0)
    return fail(DA_ERR_INVALID_ARG, "a paged plan needs decode_attn_dense_paged");
  if (!k_len_dev) return fail(DA_ERR_INVALID_ARG, "k_len_dev must be non-NULL");
  if (((uintptr_t)k_len_dev & 3u) != 0)
    return fail(DA_ERR_INVALID_ARG, "k_len_dev must be 4-byte aligned");
  // The launch is sized once for max_k_len; the kernel spreads whatever length
  // the device holds over the same splits.
  const int S = plan->num_splits_max;
  da::PartialLaunch L =
      base_launch(*plan, q, k, v, out, softmax_scale, plan->prob.max_k_len, workspace, S);
  L.k_len_dev = k_len_dev;
  L.chunk = plan->chunk;
  L.sparse = false;
  if (log_enabled())
    std::fprintf(stderr, "[decode_attn] dense (device k_len) splits=%d\n", S);
  return run(L, stream);
}

decode_attn_status decode_attn_dense_ragged(const decode_attn_plan_t* plan, const void* q,
                                            const void* k, const void* v, void* out,
                                            float softmax_scale, const int32_t* k_lens,
                                            int32_t k_lens_stride, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return dense_with_lengths(plan, q, k, v, nullptr, k_lens, k_lens_stride, out, softmax_scale,
                            workspace, workspace_bytes, stream);
}

decode_attn_status decode_attn_dense_step(const decode_attn_plan_t* plan, const void* q,
                                          void* k_cache, void* v_cache, const void* k_new,
                                          const void* v_new, const int32_t* block_table,
                                          const int32_t* k_lens, int32_t k_lens_stride, void* out,
                                          float softmax_scale, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) return fail(DA_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(DA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  return dense_with_lengths(plan, q, k_cache, v_cache, block_table, k_lens, k_lens_stride, out,
                            softmax_scale, workspace, workspace_bytes, stream, k_new, v_new);
}

decode_attn_status decode_attn_dense_paged(const decode_attn_plan_t* plan, const void* q,
                                           const void* k_pages, const void* v_pages,
                                           const int32_t* block_table, const int32_t* k_lens,
                                           int32_t k_lens_stride, void* out, float softmax_scale,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (!block_table) return fail(DA_ERR_INVALID_ARG, "block_table must be non-NULL");
  return dense_with_lengths(plan, q, k_pages, v_pages, block_table, k_lens, k_lens_stride, out,
                            softmax_scale, workspace, workspace_bytes, stream);
}

decode_attn_status decode_attn_sparse(const decode_attn_plan_t* plan, const void* q, const void* k,
                                      const void* v, const int32_t* sel, int32_t topk, void* out,
                                      float softmax_scale, int64_t k_len, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  decode_attn_status s =
      check_common(plan, 1, q, k, v, out, softmax_scale, workspace, workspace_bytes);
  if (s != DA_OK) return s;
  if (!sel) return fail(DA_ERR_INVALID_ARG, "sel must be non-NULL");
  if (((uintptr_t)sel & 3u) != 0) return fail(DA_ERR_INVALID_ARG, "sel must be 4-byte aligned");
  if (topk < 1 || topk > plan->prob.topk_max)
    return fail(DA_ERR_INVALID_ARG, "topk must lie in [1, topk_max = %d], got %d",
                plan->prob.topk_max, topk);
  if (k_len < 1 || k_len > plan->prob.capacity)
    return fail(DA_ERR_INVALID_ARG, "k_len must lie in [1, capacity = %lld], got %lld",
                (long long)plan->prob.capacity, (long long)k_len);
  const int S = (int)ceil_div(topk, plan->chunk);
  da::PartialLaunch L = base_launch(*plan, q, k, v, out, softmax_scale, k_len, workspace, S);
  L.sel = sel;
  L.topk = topk;
  L.chunk = plan->chunk;
  L.sparse = true;
  if (log_enabled())
    std::fprintf(stderr, "[decode_attn] sparse topk=%d splits=%d chunk=%d\n", topk, S, plan->chunk);
  return run(L, stream);
}

decode_attn_status decode_attn_build_selection(const decode_attn_select_problem* p,
                                               const float* scores, const int32_t* pos,
                                               int32_t* sel, void* stream) {
  da::SelectLaunch L;
  const decode_attn_status s = select_launch(p, scores, pos, sel, &L);
  if (s != DA_OK) return s;
  const hipError_t e = da::launch_select(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(DA_ERR_HIP, "selection kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

decode_attn_status decode_attn_select_workspace(const decode_attn_select_problem* p,
                                                size_t* bytes) {
  if (!bytes) return fail(DA_ERR_INVALID_ARG, "bytes must be non-NULL");
  da::SelectLaunch L;
  // pointers are not needed for the size: validate the shape only
  static const int32_t dummy[4] = {0, 0, 0, 0};
  alignas(16) static const float dummy_scores[4] = {0.f, 0.f, 0.f, 0.f};
  const decode_attn_status s =
      select_launch(p, dummy_scores, dummy, const_cast<int32_t*>(dummy), &L);
  if (s != DA_OK) return s;
  *bytes = da::select_workspace_bytes(p->batch, p->n_idx);
  return ok();
}

decode_attn_status decode_attn_build_selection_ws(const decode_attn_select_problem* p,
                                                  const float* scores, const int32_t* pos,
                                                  int32_t* sel, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  da::SelectLaunch L;
  const decode_attn_status s = select_launch(p, scores, pos, sel, &L);
  if (s != DA_OK) return s;
  const size_t need = da::select_workspace_bytes(p->batch, p->n_idx);
  if (need > 0) {
    if (!workspace)
      return fail(DA_ERR_WORKSPACE, "workspace is NULL but the selection needs %zu bytes", need);
    if (workspace_bytes < need)
      return fail(DA_ERR_WORKSPACE, "workspace has %zu bytes, the selection needs %zu",
                  workspace_bytes, need);
    if (!aligned16(workspace)) return fail(DA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  L.ws = need > 0 ? workspace : nullptr;
  L.parts = need > 0 ? da::select_parts(p->n_idx) : 0;
  const hipError_t e = need > 0 ? da::launch_select_split(L, static_cast<hipStream_t>(stream))
                                : da::launch_select(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(DA_ERR_HIP, "selection kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

decode_attn_status decode_attn_append_kv(const decode_attn_append_problem* p, void* k_cache,
                                         void* v_cache, const void* k_new, const void* v_new,
                                         const int32_t* pos, void* stream) {
  if (!p) return fail(DA_ERR_INVALID_ARG, "problem pointer must be non-NULL");
  if (p->batch < 1 || p->num_kv_heads < 1)
    return fail(DA_ERR_INVALID_ARG, "batch and num_kv_heads must be >= 1");
  if (p->head_dim < 8 || p->head_dim > 512 || p->head_dim % 8 != 0)
    return fail(DA_ERR_INVALID_ARG, "head_dim must be a multiple of 8 in [8, 512], got %d",
                p->head_dim);
  if (p->capacity < 1) return fail(DA_ERR_INVALID_ARG, "capacity must be >= 1");
  if (p->window < 0 || p->win_base < 0 || p->win_base + p->window > p->capacity)
    return fail(DA_ERR_INVALID_ARG, "the window ring must lie inside [0, capacity)");
  if (!k_cache || !v_cache || !k_new || !v_new || !pos)
    return fail(DA_ERR_INVALID_ARG, "caches, new rows and pos must be non-NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
      ((uintptr_t)pos & 3u))
    return fail(DA_ERR_INVALID_ARG, "caches and new rows must be 16-byte aligned, pos 4-byte");
  da::AppendLaunch L{};
  L.k_cache = static_cast<uint16_t*>(k_cache);
  L.v_cache = static_cast<uint16_t*>(v_cache);
  L.k_new = static_cast<const uint16_t*>(k_new);
  L.v_new = static_cast<const uint16_t*>(v_new);
  L.pos = pos;
  L.B = p->batch;
  L.Hkv = p->num_kv_heads;
  L.D = p->head_dim;
  L.capacity = p->capacity;
  L.window = p->window;
  L.win_base = p->win_base;
  const hipError_t e = da::launch_append(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(DA_ERR_HIP, "append kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

decode_attn_status decode_attn_write_slots(const decode_attn_slot_problem* p, void* k_pages,
                                           void* v_pages, const void* k_rows, const void* v_rows,
                                           const int64_t* slot_mapping, void* stream) {
  if (!p) return fail(DA_ERR_INVALID_ARG, "problem pointer must be non-NULL");
  if (p->num_tokens < 0 || p->num_kv_heads < 1 || p->page_size < 1 || p->num_pages < 1)
    return fail(DA_ERR_INVALID_ARG,
                "num_tokens must be >= 0; num_kv_heads, page_size and num_pages >= 1");
  if (p->head_dim < 8 || p->head_dim > 512 || p->head_dim % 8 != 0)
    return fail(DA_ERR_INVALID_ARG, "head_dim must be a multiple of 8 in [8, 512], got %d",
                p->head_dim);
  if ((double)p->num_pages * p->num_kv_heads * p->page_size * p->head_dim > 9.0e15)
    return fail(DA_ERR_INVALID_ARG, "page pools too large");
  if ((int64_t)p->num_tokens * p->num_kv_heads * (p->head_dim / 8) * 2 > 0x7fffffffLL * 256)
    return fail(DA_ERR_INVALID_ARG, "too many rows for one launch");
  if (p->num_tokens == 0) return ok();  // nothing to write; no pointer is read
  if (!k_pages || !v_pages || !k_rows || !v_rows || !slot_mapping)
    return fail(DA_ERR_INVALID_ARG, "pools, rows and slot_mapping must be non-NULL");
  if (!aligned16(k_pages) || !aligned16(v_pages) || !aligned16(k_rows) || !aligned16(v_rows) ||
      ((uintptr_t)slot_mapping & 7u))
    return fail(DA_ERR_INVALID_ARG, "pools and rows must be 16-byte aligned, slot_mapping 8-byte");
  da::SlotWriteLaunch L{};
  L.k_pages = static_cast<uint16_t*>(k_pages);
  L.v_pages = static_cast<uint16_t*>(v_pages);
  L.k_rows = static_cast<const uint16_t*>(k_rows);
  L.v_rows = static_cast<const uint16_t*>(v_rows);
  L.slots = slot_mapping;
  L.N = p->num_tokens;
  L.Hkv = p->num_kv_heads;
  L.D = p->head_dim;
  L.page_size = p->page_size;
  L.num_pages = p->num_pages;
  const hipError_t e = da::launch_write_slots(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(DA_ERR_HIP, "slot write kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

decode_attn_status decode_attn_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                         void* stream) {
  if (!buf || !sink) return fail(DA_ERR_INVALID_ARG, "buf and sink must be non-NULL");
  if (!aligned16(buf) || ((uintptr_t)sink & 3u))
    return fail(DA_ERR_INVALID_ARG, "buf must be 16-byte and sink 4-byte aligned");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(DA_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  int cus = 0;
  decode_attn_status s = device_cus(&cus);
  if (s != DA_OK) return s;
  const hipError_t e =
      da::launch_read_probe(buf, (int64_t)bytes, sink, cus, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DA_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
  return ok();
}

decode_attn_status decode_attn_set_timing_events(void* ev_before, void* ev_after) {
  if ((ev_before == nullptr) != (ev_after == nullptr))
    return fail(DA_ERR_INVALID_ARG, "pass both timing events or neither");
  g_ev_before = static_cast<hipEvent_t>(ev_before);
  g_ev_after = static_cast<hipEvent_t>(ev_after);
  return ok();
}

const char* decode_attn_status_str(decode_attn_status s) {
  // A C caller may pass any int; read it as one (a C++ load of an out-of-range
  // enumeration value is undefined).
  int v = 0;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case DA_OK: return "DA_OK";
    case DA_ERR_INVALID_ARG: return "DA_ERR_INVALID_ARG";
    case DA_ERR_UNSUPPORTED: return "DA_ERR_UNSUPPORTED";
    case DA_ERR_WORKSPACE: return "DA_ERR_WORKSPACE";
    case DA_ERR_HIP: return "DA_ERR_HIP";
  }
  return "DA_ERR_UNKNOWN";
}

const char* decode_attn_last_error(void) { return g_last_error; }

}  // extern "C"
