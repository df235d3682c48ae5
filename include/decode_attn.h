/*
 * decode_attn.h -- decode attention on MI355X (gfx950), C ABI.
 *
 * The operation. For query token t of Sq (Sq = 1 in plain decode),
 *
 *     out[b, h, t, :] = sum_j softmax_j( softmax_scale * q[b, h, t, :] . K[b, hk, j, :] ) V[b, hk, j, :]
 *
 * over the keys j the token sees, with hk = h / (Hq / Hkv) (grouped-query
 * heads: each KV head serves a contiguous group of Hq / Hkv query heads). This
 * is the problem stated by the fuel-dispatch page "DecodeFlashSpec": q is
 * [B, Hq, Sq, D]; k and v are the capacity KV buffers [B, Hkv, capacity, D];
 * softmax_scale is an f32 (usually 1/sqrt(head_dim)); the query attends the
 * live prefix [0, k_len), which counts the Sq new tokens (field k_len); causal
 * is accepted and ignored for one token, which sees the whole prefix (field
 * causal), and for several tokens masks each to the positions up to its own
 * (the last Sq of the prefix); ALiBi slopes, left and right sliding windows
 * and a logit softcap are rejected (fields alibi, window_size_left,
 * window_size_right, softcap).
 *
 * The sparse variant follows the metrale page "AttnV41" (decode_fixed_topk,
 * decode_prep, decode_body): each token attends the KV rows listed in its
 * selection, padded with -1 to a fixed launch width topk; a pad contributes
 * to neither the softmax sum nor the weighted sum of values, so padding the
 * same valid entries to any width gives bit-identical output.
 *
 * Conventions (every call):
 *   - Every tensor is contiguous row-major. q, k, v and out are bfloat16
 *     (passed as raw device pointers); sel is int32; the workspace is raw
 *     bytes. All device pointers must be 16-byte aligned.
 *   - The caller owns every buffer and the stream. The library allocates and
 *     frees nothing, performs no host<->device copy and no synchronisation;
 *     both compute calls only enqueue kernels on `stream` (a hipStream_t, NULL
 *     for the default stream), so they can be captured into a HIP graph with
 *     fixed pointers. (Caller-owned, graph-stable buffers and no device-to-host
 *     validation sync are the conventions of the flashinfer page
 *     "packed_fused_kda_decode".)
 *   - Validation fails closed on host-visible arguments and returns a status;
 *     nothing is thrown across the ABI. Values that live in device memory
 *     (the selection entries) are caller-owned and are not validated.
 *   - decode_attn_last_error() returns a thread-local, human-readable message
 *     for the last failing call on the calling thread.
 *   - Environment (diagnostics and tuning runs only): DECODE_ATTN_LOG=1 prints
 *     each plan's decisions and each call's split count to stderr;
 *     DECODE_ATTN_SPLITS=<n> caps the dense split count (see force_splits).
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DA_OK = 0,
  DA_ERR_INVALID_ARG = 1, /* bad shape, range, pointer, alignment or plan mismatch */
  DA_ERR_UNSUPPORTED = 2, /* a feature the kernels do not implement (ALiBi, window, softcap) */
  DA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than plan.workspace_bytes */
  DA_ERR_HIP = 4          /* the HIP runtime reported an error (device query or launch) */
} decode_attn_status;

/*
 * The problem a plan serves. Host struct; mirrors the fields of the
 * "DecodeFlashSpec" statement (q/k/v shapes, causal, alibi, windows, softcap,
 * k_len) plus the fixed launch width of the sparse variant ("AttnV41",
 * decode_fixed_topk).
 */
typedef struct {
  int32_t batch;        /* B >= 1: sequences                                              */
  int32_t num_q_heads;  /* Hq >= 1, a multiple of num_kv_heads                            */
  int32_t num_kv_heads; /* Hkv >= 1                                                       */
  int32_t head_dim;     /* D: 64 or 128                                                   */
  int32_t seq_q;        /* Sq: query tokens per sequence, 1 (decode) to 16 (verification
                           rows: the AttnV41 page's forward runs m tokens at start_pos);
                           above 1 for dense plans only                                 */
  int64_t capacity;     /* rows per (kv batch, kv head) in K and V                        */
  int64_t max_k_len;    /* largest k_len a call may pass, 1 <= max_k_len <= capacity      */
  int32_t topk_max;     /* sparse plan: largest launch topk (>= 1); 0 = dense plan        */
  int32_t kv_batch;     /* sparse: 1 (rows shared by all tokens) or batch; dense: batch
                           (0 is read as batch)                                           */
  int32_t causal;       /* Sq = 1: accepted and ignored. Sq > 1: nonzero -> token t (of
                           Sq) sees rows [0, k_len - Sq + 1 + t), the new tokens being the
                           last Sq positions of the live prefix; 0 -> every token sees
                           [0, k_len)                                                    */
  int32_t has_alibi;    /* nonzero -> DA_ERR_UNSUPPORTED                                  */
  int64_t window_left;  /* -1 = none; any other value -> DA_ERR_UNSUPPORTED               */
  int64_t window_right; /* -1 = none; any other value -> DA_ERR_UNSUPPORTED               */
  int32_t has_softcap;  /* nonzero -> DA_ERR_UNSUPPORTED                                  */
  int32_t num_cus;      /* compute units to plan for; 0 = query the current HIP device    */
  int32_t force_splits; /* > 0: dense split count cap (tuning and tests); 0 = heuristic,
                           or for tuning runs the environment variable DECODE_ATTN_SPLITS
                           (a positive integer) when force_chunk is 0 too; the plan's
                           prob holds the value used                                     */
  int32_t force_chunk;  /* > 0: keys (dense) or selection entries (sparse) per split      */
  int32_t page_size;    /* 0: contiguous K/V; > 0: paged dense cache, a multiple of 32    */
  int32_t max_pages_per_seq; /* paged: block-table row length; capacity must equal
                                page_size * max_pages_per_seq                            */
  int64_t num_pages;    /* paged: pages in the K and V page pools                         */
  int32_t ragged;       /* 1: the plan also serves decode_attn_dense_ragged (one length per
                           sequence; implied by page_size > 0), 0: it does not             */
} decode_attn_problem;

/*
 * A plan: plain data, copyable, no device state. Produced by decode_attn_plan
 * and passed by pointer to every compute call.
 */
typedef struct {
  decode_attn_problem prob; /* the validated problem (kv_batch resolved)               */
  int32_t group;            /* Hq / Hkv                                                */
  int32_t num_splits_max;   /* most key splits any call of this plan launches          */
  int32_t chunk;            /* sparse: selection entries per split (fixed by the plan);
                               dense: keys per split at max_k_len                      */
  int32_t num_cus;          /* compute units the plan was made for                      */
  int32_t kind;             /* 0 dense, 1 sparse                                       */
  int32_t balanced_wgs;     /* ragged / paged plans: workgroups of the length-balanced
                               schedule (0 for other plans)                              */
  uint64_t workspace_bytes; /* bytes of workspace every call of this plan needs (may be 0) */
} decode_attn_plan_t;

/*
 * Validate a problem and choose the split-K decomposition.
 *   p    host pointer to the problem; out  host pointer that receives the plan.
 * Returns DA_OK, DA_ERR_INVALID_ARG (shapes/ranges), DA_ERR_UNSUPPORTED (ALiBi,
 * window, softcap, head_dim other than 64/128, seq_q outside 1..16 or above 1 in
 * a sparse plan, ragged or paged sparse plans), or DA_ERR_HIP when
 * num_cus is 0 and the device query fails. Touches the GPU only for that query.
 */
decode_attn_status decode_attn_plan(const decode_attn_problem* p, decode_attn_plan_t* out);

/*
 * Dense decode attention over the live prefix [0, k_len) of the capacity buffers.
 *   q    [B, Hq, Sq, D] bf16           k, v [B, Hkv, capacity, D] bf16
 *   out  [B, Hq, Sq, D] bf16 (written) softmax_scale  finite f32
 *   k_len  1 <= k_len <= plan->prob.max_k_len (and k_len >= Sq when causal); rows
 *          >= k_len are never read. It counts the Sq query tokens (DecodeFlashSpec,
 *          field k_len: cached length plus the tokens of the pass).
 *   workspace  device scratch of at least plan->workspace_bytes (may be NULL when
 *          that is 0); its contents on entry do not matter.
 * Enqueues one or two kernels on `stream` and returns without waiting.
 * Returns DA_OK, DA_ERR_INVALID_ARG, DA_ERR_WORKSPACE or DA_ERR_HIP (launch).
 */
decode_attn_status decode_attn_dense(const decode_attn_plan_t* plan, const void* q,
                                     const void* k, const void* v, void* out,
                                     float softmax_scale, int64_t k_len, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): decode_attn_dense with the split
 * workspace taken from a library-owned static device array of 16 MiB per
 * device (held until the process ends) instead of a caller-owned buffer.
 * Arguments as decode_attn_dense, without workspace and workspace_bytes.
 * Allocates nothing. Every call on one device shares that device's array, so
 * calls that overlap on one device (other streams, other threads) race and
 * must not be issued; the array's contents between calls do not matter.
 * Returns as decode_attn_dense; DA_ERR_WORKSPACE when plan->workspace_bytes
 * exceeds 16 MiB, DA_ERR_HIP if the array's device address cannot be found.
 */
decode_attn_status decode_attn_dense_static(const decode_attn_plan_t* plan, const void* q,
                                            const void* k, const void* v, void* out,
                                            float softmax_scale, int64_t k_len, void* stream);

/*
 * Dense decode attention with the live length read on the device (plan-once
 * decode: DecodeFlashSpec's k_len as a symbol bound to the live length each
 * token, fuel-dispatch page "DecodeFlashSpec", field k_len). Same arguments
 * as decode_attn_dense except:
 *   k_len_dev  device pointer to one int32, read by the kernel when it runs. The
 *          launch is sized once for plan->prob.max_k_len, so the call can be
 *          captured in a HIP graph and replayed while the caller rewrites the
 *          value between replays. The value is caller-owned and not validated on
 *          the host: a value above max_k_len is clamped to max_k_len, and a value
 *          <= 0 produces zero output. Rows at or beyond the clamped length are
 *          never read.
 * Returns DA_OK, DA_ERR_INVALID_ARG, DA_ERR_WORKSPACE or DA_ERR_HIP (launch).
 */
decode_attn_status decode_attn_dense_devlen(const decode_attn_plan_t* plan, const void* q,
                                            const void* k, const void* v, void* out,
                                            float softmax_scale, const int32_t* k_len_dev,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * Dense decode attention with one live length per sequence, read on the device
 * (ragged batch; the DflashScratch page of metrale keeps one [kv_len, q_offset,
 * q_rope_pos] u32 triple per band, read at kernel entry, so the lengths can be
 * read straight out of such an array). Same arguments as decode_attn_dense
 * except:
 *   k_lens  device int32; sequence b attends rows [0, k_lens[b * k_lens_stride]).
 *          Values are caller-owned: clamped to [0, max_k_len]; 0 gives zeros, and
 *          with causal Sq > 1 a token whose prefix is empty gets zeros.
 *   k_lens_stride  >= 1, in int32 elements (3 for the triples above).
 * The launch is sized once for max_k_len (capturable, like
 * decode_attn_dense_devlen). Returns as decode_attn_dense.
 */
decode_attn_status decode_attn_dense_ragged(const decode_attn_plan_t* plan, const void* q,
                                            const void* k, const void* v, void* out,
                                            float softmax_scale, const int32_t* k_lens,
                                            int32_t k_lens_stride, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * Dense decode attention over a paged KV cache (the DflashScratch page of
 * metrale addresses its paged cache through slot indices). Needs a plan with
 * page_size > 0.
 *   k_pages, v_pages  [num_pages, Hkv, page_size, D] bf16 page pools.
 *   block_table  device int32 [B, max_pages_per_seq]: logical row j of sequence b
 *          is row j % page_size of page block_table[b, j / page_size]. Entries for
 *          pages that cover [0, k_len_b) must be page ids in [0, num_pages); an id
 *          outside that range is never read (those keys are skipped). Entries past
 *          a sequence's length are ignored.
 *   k_lens, k_lens_stride  as decode_attn_dense_ragged.
 *   q, out, softmax_scale, workspace, stream  as decode_attn_dense.
 * Returns as decode_attn_dense; DA_ERR_INVALID_ARG for a contiguous plan.
 */
decode_attn_status decode_attn_dense_paged(const decode_attn_plan_t* plan, const void* q,
                                           const void* k_pages, const void* v_pages,
                                           const int32_t* block_table, const int32_t* k_lens,
                                           int32_t k_lens_stride, void* out, float softmax_scale,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/*
 * One whole dense decode pass in a single call: write the pass's new K and V
 * rows into the cache and attend (the append-then-attend step of plan-once
 * decode: the live length counts the new tokens, fuel-dispatch page
 * "DecodeFlashSpec", field k_len; the metrale page "DflashScratch" writes its
 * cache through slot indices). Needs a plan made with ragged = 1 (contiguous
 * cache, block_table NULL) or a paged plan (block_table as
 * decode_attn_dense_paged).
 *   k_cache, v_cache  the caches of decode_attn_dense_ragged / _paged (written).
 *   k_new, v_new  [B, Hkv, Sq, D] bf16: row t of sequence b belongs at cache row
 *          L_b - Sq + t, L_b = clamp(k_lens[b * k_lens_stride], 0, max_k_len).
 *          Those rows are written (a negative row, or one whose page id lies
 *          outside the pool, is not), and token t attends [0, L_b) or its
 *          causal part, reading them as written.
 *   the other arguments as decode_attn_dense_ragged / decode_attn_dense_paged.
 * Enqueues a small row-write kernel and then the attention kernels of
 * decode_attn_dense_ragged / _paged, so the result equals those calls made
 * after writing the rows, bit for bit. (Measured: folding the write into the
 * attention kernel cost more than the extra launch.)
 * Returns as decode_attn_dense.
 */
decode_attn_status decode_attn_dense_step(const decode_attn_plan_t* plan, const void* q,
                                          void* k_cache, void* v_cache, const void* k_new,
                                          const void* v_new, const int32_t* block_table,
                                          const int32_t* k_lens, int32_t k_lens_stride, void* out,
                                          float softmax_scale, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Index-selected sparse decode attention.
 *   q    [B, Hq, 1, D] bf16           k, v [kv_batch, Hkv, capacity, D] bf16
 *   sel  [B, topk] int32 (device): token b attends rows sel[b, t] of its KV set
 *        (set 0 when kv_batch == 1, set b otherwise), for every KV head; entries
 *        < 0 are pads. Valid entries must lie in [0, k_len): an entry >= k_len is
 *        a caller error, which the kernel does not report but never reads
 *        through (it is skipped like a pad). Duplicates count with multiplicity.
 *   topk 1 <= topk <= plan->prob.topk_max: the launch width (row stride of sel).
 *   out  [B, Hq, 1, D] bf16 (written). A token with no valid entry gets zeros.
 *   k_len rows usable by the selection, 1 <= k_len <= capacity.
 * The split of the selection into chunks is fixed by the plan and does not
 * depend on topk, so the same valid entries padded to any topk <= topk_max give
 * bit-identical output.
 * Returns DA_OK, DA_ERR_INVALID_ARG, DA_ERR_WORKSPACE or DA_ERR_HIP (launch).
 */
decode_attn_status decode_attn_sparse(const decode_attn_plan_t* plan, const void* q,
                                      const void* k, const void* v, const int32_t* sel,
                                      int32_t topk, void* out, float softmax_scale,
                                      int64_t k_len, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * The selection a sparse call reads, built on the device (metrale page
 * "AttnV41": decode_prep / decode_prep_role fill the selection buffer with the
 * window slots, then the shared index selection, then -1 up to the fixed width
 * of decode_fixed_topk; decode_body writes the window as a ring at
 * pos % window). Host struct.
 */
typedef struct {
  int32_t batch;        /* B >= 1 tokens                                              */
  int32_t n_idx;        /* index candidates 0 .. n_idx-1 per token, 0 .. 131072       */
  int64_t score_stride; /* floats between rows of scores: >= n_idx, a multiple of 4    */
  int32_t k_idx;        /* index entries to select per token, 0 .. 4096 (0: window only) */
  int32_t window;       /* window ring slots W (>= 0)                                 */
  int64_t win_base;     /* KV row of ring slot 0; the ring is rows win_base .. +W-1    */
  int32_t topk;         /* launch width of the selection (>= 1)                       */
} decode_attn_select_problem;

/*
 * Build sel [B, topk] int32 on `stream` from device scores [B, score_stride]
 * fp32 and device positions pos [B] int32 (0-based position of each token).
 * Row b holds: the window rows of positions max(0, pos-W+1) .. pos oldest first
 * (position p in row win_base + p % W; none when pos < 0); then the
 * min(k_idx, n_idx, topk - window entries) candidates with the largest scores
 * (ties to the lower index; scores ordered by IEEE 754 totalOrder), listed in
 * ascending row order; then -1. Device values are caller-owned (no host
 * validation). scores must be 16-byte aligned; pos and sel 4-byte aligned.
 * One kernel, no allocation, capturable.
 * Returns DA_OK, DA_ERR_INVALID_ARG (shapes, NULL or misaligned pointers,
 * k_idx > 4096), DA_ERR_UNSUPPORTED (n_idx > 131072) or DA_ERR_HIP (launch).
 */
decode_attn_status decode_attn_build_selection(const decode_attn_select_problem* p,
                                               const float* scores, const int32_t* pos,
                                               int32_t* sel, void* stream);

/*
 * The same selection built by several workgroups per token, for many index
 * candidates (AttnV41 page, decode_prep_role / decode_fixed_topk: the index
 * selection of a capturable step). Each workgroup filters a 4096-candidate part
 * of the row against a bound taken from a sample of it and keeps the keys above
 * the bound in a caller-owned workspace; one workgroup per token then selects
 * among the kept keys. The output is identical to decode_attn_build_selection
 * (exact whatever the scores: a token whose kept keys cannot hold the selection
 * is redone over all its candidates by its merge workgroup).
 *   workspace  device scratch of at least the bytes decode_attn_select_workspace
 *          reports for the problem (0 for fewer than 8192 candidates, which take
 *          the one-workgroup kernel); 16-byte aligned; contents on entry do not
 *          matter. Two kernels on `stream`, no allocation, capturable.
 * Returns as decode_attn_build_selection, and DA_ERR_WORKSPACE for a missing or
 * short workspace.
 */
decode_attn_status decode_attn_build_selection_ws(const decode_attn_select_problem* p,
                                                  const float* scores, const int32_t* pos,
                                                  int32_t* sel, void* workspace,
                                                  size_t workspace_bytes, void* stream);

/*
 * Workspace bytes decode_attn_build_selection_ws needs for problem p (host
 * only; validates the problem's shape like the build call). Returns DA_OK,
 * DA_ERR_INVALID_ARG or DA_ERR_UNSUPPORTED.
 */
decode_attn_status decode_attn_select_workspace(const decode_attn_select_problem* p,
                                                size_t* bytes);

/*
 * KV append / window ring write: the current token's K and V rows go into the
 * capacity cache before the attention call, at a row read on the device
 * (fuel-dispatch page "DecodeFlashSpec", field k_len: the live length counts
 * the new token; metrale page "AttnV41", decode_body: the window ring write at
 * pos % window with the slot read on the device). Host struct.
 */
typedef struct {
  int32_t batch;        /* B >= 1 tokens                                              */
  int32_t num_kv_heads; /* Hkv >= 1                                                   */
  int32_t head_dim;     /* D: a multiple of 8, at most 512                            */
  int64_t capacity;     /* rows per (token, kv head) in the caches                    */
  int32_t window;       /* 0: linear cache, row = pos; > 0: ring of `window` rows      */
  int64_t win_base;     /* first row of the ring (window > 0); ring within capacity   */
} decode_attn_append_problem;

/*
 * k_cache, v_cache [B, Hkv, capacity, D] bf16 (written); k_new, v_new
 * [B, Hkv, 1, D] bf16; pos [B] int32 device positions. Token b's rows go to row
 * pos[b] (window == 0) or win_base + pos[b] % window; a position that is
 * negative or lands outside [0, capacity) writes nothing (device values are
 * caller-owned, not validated on the host). One kernel on `stream`, no
 * allocation, capturable. Pointers 16-byte aligned (pos 4-byte).
 * Returns DA_OK, DA_ERR_INVALID_ARG or DA_ERR_HIP (launch).
 */
decode_attn_status decode_attn_append_kv(const decode_attn_append_problem* p, void* k_cache,
                                         void* v_cache, const void* k_new, const void* v_new,
                                         const int32_t* pos, void* stream);

/*
 * Slot-addressed KV write (metrale page "DflashScratch", field slot_mapping_dev:
 * one 64-bit paged-cache slot index per token of the pass, consumed by a
 * reshape-and-cache write into the paged cache). Host struct.
 */
typedef struct {
  int32_t num_tokens;   /* N >= 0 rows to write (0: nothing is enqueued or read)   */
  int32_t num_kv_heads; /* Hkv >= 1                                                */
  int32_t head_dim;     /* D: a multiple of 8, at most 512                         */
  int32_t page_size;    /* rows per page, >= 1                                     */
  int64_t num_pages;    /* pages in each pool, >= 1                                */
} decode_attn_slot_problem;

/*
 * k_pages, v_pages [num_pages, Hkv, page_size, D] bf16 (written): the page pools
 * of decode_attn_dense_paged (a contiguous cache [B, Hkv, capacity, D] is the
 * same layout with page_size = capacity and num_pages = B). k_rows, v_rows
 * [N, Hkv, D] bf16: token n's key and value rows, head-major inside a token.
 * slot_mapping [N] int64 (device): token n's rows go to row s % page_size of
 * page s / page_size, s = slot_mapping[n], for every kv head. A negative slot
 * (a padding token) writes nothing; a slot at or past num_pages * page_size is
 * a caller error that writes nothing. Two tokens naming one slot are a caller
 * error: each 16-byte piece of that slot's rows then holds the same piece of
 * one of those tokens' rows. Slot values are device-resident and not
 * validated on the host. One kernel on `stream`, no allocation, capturable.
 * Pools and rows 16-byte aligned, slot_mapping 8-byte aligned.
 * Returns DA_OK, DA_ERR_INVALID_ARG or DA_ERR_HIP (launch).
 */
decode_attn_status decode_attn_write_slots(const decode_attn_slot_problem* p, void* k_pages,
                                           void* v_pages, const void* k_rows, const void* v_rows,
                                           const int64_t* slot_mapping, void* stream);

/*
 * Diagnostics: time the split-K partial kernel (the kernel that streams K and V)
 * with caller-created HIP events. After this call, every compute call made on
 * the calling thread records `ev_before` on its stream immediately before
 * launching its partial kernel and `ev_after` immediately after it, so that
 * hipEventElapsedTime(ev_before, ev_after) is that kernel's duration. Events
 * are hipEvent_t handles owned by the caller; passing NULL for both stops the
 * recording. Returns DA_OK, or DA_ERR_INVALID_ARG if exactly one is NULL.
 * (Not part of the operation; for benchmarks and profilers.)
 */
decode_attn_status decode_attn_set_timing_events(void* ev_before, void* ev_after);

/*
 * Diagnostics: the measured streaming-read ceiling. Reads `bytes` (a positive
 * multiple of 16) of device memory at `buf` (16-byte aligned) with the
 * attention kernels' load style (16-byte non-temporal loads, one workgroup
 * per compute unit, each reading a contiguous share with sixteen loads in
 * flight per thread, the fastest shape measured) and XORs a fold of every
 * word into *sink (device, 4-byte aligned), so the reads cannot be dropped.
 * Time it with events on `stream` to get the achievable read bandwidth the
 * attention kernels are compared with. Returns DA_OK, DA_ERR_INVALID_ARG or
 * DA_ERR_HIP. (Not part of the operation; for benchmarks.)
 */
decode_attn_status decode_attn_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                          void* stream);

/* Static string naming a status code. */
const char* decode_attn_status_str(decode_attn_status s);

/* Message for the last failing call on this thread ("" if none). Host memory,
 * valid until the next call on this thread. */
const char* decode_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
