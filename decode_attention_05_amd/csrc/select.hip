// select.hip -- builds the padded sparse-attention selection on the device.
//
// For each token b the selection row holds (metrale page "AttnV41":
// decode_prep and decode_prep_role fill it with the window slots, then the
// shared index selection, then -1 up to decode_fixed_topk's launch width;
// decode_body writes the window as a ring at pos % window):
//   * the window rows of positions max(0, pos - W + 1) .. pos, oldest first,
//     position p living in KV row win_base + p % W;
//   * the k index candidates (0 .. n_idx - 1) with the largest scores, listed
//     in ascending row order, ties to the lower index, k = min(k_idx, n_idx,
//     topk - window entries), scores ordered as IEEE 754 totalOrder;
//   * -1 for the rest.
// Building it on the device removes the host score download that keeps a step
// with a host-side top-k out of a captured graph.
//
// One 1024-thread workgroup per token. Scores become 32-bit totalOrder keys.
//   0. Prefilter (at least 8192 candidates): 256 runs of 8 keys spread over
//      the row are sampled, and the lower end of the 16-bit bucket of the
//      sample key a few standard deviations beyond the expected rank of the
//      k-th largest key becomes a bound L0. One pass keeps every key >= L0 in
//      LDS (a wave scan and one LDS atomic per wave per chunk place them). If
//      at least k keys were kept (so the k-th largest key is >= L0 and the top
//      k are all among them) and they fit, steps 1-2 run on the kept keys,
//      otherwise on all keys: the result is exact either way.
//   1. Two histogram passes over the key set (8 bits each, from the top) find
//      the 16-bit key bucket that holds the k-th largest key, how many keys lie
//      above that bucket and how many inside it. Each thread keeps 8 16-byte
//      loads in flight; counts go to 16 lane-striped LDS histograms plus spare
//      bins for non-matching keys, so no count is conditional.
//   2. One more pass marks every row above the bucket in an LDS bitmap of the
//      candidate rows and collects the keys inside the bucket (a handful for
//      real-valued scores); a small LDS sort of those by (key desc, index asc)
//      (one wave, in registers, when there are at most 64) marks the rest of
//      the k, ties resolved to lower indices.
//   3. Per-thread popcounts and a block scan over the bitmap write the chosen
//      rows in ascending row order.
// When the bucket holds more keys than the candidate list (heavily tied
// scores), the workgroup finishes an exact 4-pass radix select instead, marks
// the keys equal to the threshold to find the cut index among them, and marks
// the final set from that.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "select.h"

namespace da {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kCopies = 16;                // histogram copies, chosen by lane % 16
constexpr int kBins = 256 + 32 + 1;        // 256 digits, 32 spare bins for non-matching
                                           // keys, 1 pad word: copies start on distinct banks
constexpr int kLoads = 8;                  // 16-byte loads in flight per thread in a pass
constexpr int kCandCap = 2048;             // candidate list (keys inside the threshold bucket)
constexpr int kWords = kSelectMaxCandidates / 32;  // bitmap of the candidate rows
constexpr int kSampleRuns = 256;           // the prefilter's sample: 256 runs of 8 keys
constexpr int kSample = 8 * kSampleRuns;
constexpr int kPreCap = 8192;              // keys kept by the prefilter
constexpr int kPreMinN = 8192;             // rows below this go straight to the exact path

// IEEE 754 totalOrder as an unsigned key: larger float -> larger key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  // negative: every bit flipped; otherwise the sign bit set (shift, or, xor)
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Sort item: ascending order = (score desc, index asc).
__device__ __forceinline__ uint64_t sort_item(uint32_t key, uint32_t idx) {
  return ((uint64_t)(~key) << 32) | idx;
}

struct Shared {
  uint32_t hist[kCopies][kBins];
  uint32_t bitmap[kWords];     // bit i: candidate row i is selected
  uint64_t cand[kCandCap];     // keys inside the threshold bucket
  uint64_t pre[kPreCap];       // prefilter: the (key, row) items at or above the bound
  uint32_t sample[kSample];    // prefilter: sampled keys
  uint32_t wsum[kSelWaves];
  uint32_t prefix, need, count, n_cand, cut, n_pre;
};

// A pass visits the scores in chunks of kSelThreads * kLoads * 4 elements: the
// thread loads 16-byte vectors (elements 4 v .. 4 v + 3 with v = vbase + tid +
// kSelThreads * u) for v < nv = n / 4, clamped to vector nv - 1 past the end (a
// valid address: the loads are unconditional); their keys are zeroed and
// `valid` cleared. for_each_key visits the last n % 4 elements separately.
struct Chunk {
  uint32_t key[kLoads][4];
  bool valid[kLoads];
};

__device__ __forceinline__ void load_chunk(const float* sc, int nv, int vbase, Chunk& c) {
  const int tid = threadIdx.x;
  float4 f[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int v = vbase + tid + kSelThreads * u;
    const int vc = v < nv ? v : nv - 1;
    f[u] = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(sc) + (uint32_t)vc * 16u);
  }
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int v = vbase + tid + kSelThreads * u;
    c.valid[u] = v < nv;
    const uint32_t m = 0u - (uint32_t)c.valid[u];
    c.key[u][0] = order_key(f[u].x) & m;
    c.key[u][1] = order_key(f[u].y) & m;
    c.key[u][2] = order_key(f[u].z) & m;
    c.key[u][3] = order_key(f[u].w) & m;
  }
}

// Visit every (key, index) of the row: fn(key, index, valid) with 16-byte loads
// for the body and scalar loads for the n % 4 tail (threads 0 .. n % 4 - 1).
template <class Fn>
__device__ __forceinline__ void for_each_key(const float* sc, int n, Fn fn) {
  const int tid = threadIdx.x;
  const int nv = n >> 2;
  for (int vbase = 0; vbase < nv; vbase += kSelThreads * kLoads) {
    Chunk c;
    load_chunk(sc, nv, vbase, c);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const uint32_t i0 = 4u * (uint32_t)(vbase + tid + kSelThreads * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) fn(c.key[u][e], i0 + e, c.valid[u]);
    }
  }
  const int tail = n & 3;
  if (tid < tail) {
    const int i = 4 * nv + tid;
    fn(order_key(sc[i]), (uint32_t)i, true);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips): within each row of 16 lanes by shifts
// of 1, 2, 4 and 8, then the rows' totals carried into the following rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return x;
}

// Digit histogram (bits shift .. shift+7) of the keys matching prefix under mask,
// then choice of the digit that holds the need-th largest matching key.
// Updates prefix/mask/need; returns the count of keys in the chosen digit.
// `visit(fn)` calls fn(key, row, live) for every key of the set.
template <class Visit>
__device__ uint32_t radix_pass(Visit&& visit, int shift, uint32_t& prefix, uint32_t& mask,
                               uint32_t& need, Shared& S) {
  const int tid = threadIdx.x;
  // Lane l counts into copy l % 16, so at most the 4 lanes l, l+16, l+32, l+48
  // of a wave instruction can collide on one bin; a score distribution puts
  // most keys into a few top-byte (exponent) digits, which a single histogram
  // would serialise.
  const int copy = tid & (kCopies - 1);
  for (int i = tid; i < kCopies * kBins; i += kSelThreads) (&S.hist[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t spare = 256u + (uint32_t)((tid >> 4) & 31);
  visit([&](uint32_t key, uint32_t, bool live) {
    const bool hit = live && (key & mask) == prefix;
    atomicAdd(&S.hist[copy][hit ? (key >> shift) & 255u : spare], 1u);
  });
  __syncthreads();
  // Wave 0 merges the histograms and picks the digit: lane l owns digits
  // 4l .. 4l+3; counts above a digit come from a suffix scan across lanes.
  if (tid < 64) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = 0u;
      for (int g = 0; g < kCopies; ++g) c[j] += S.hist[g][4 * tid + j];
    }
    const uint32_t t = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl_lo = wave_incl_scan(t);  // digits < 4 * (tid + 1)
    uint32_t above = __builtin_amdgcn_readlane(incl_lo, 63) - incl_lo;  // digits >= 4 * (tid + 1)
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      const uint32_t incl = above + c[j];
      if (above < need && incl >= need) {  // exactly one digit qualifies
        S.prefix = prefix | ((uint32_t)(4 * tid + j) << shift);
        S.need = need - above;
        S.count = c[j];
      }
      above = incl;
    }
  }
  __syncthreads();
  prefix = S.prefix;
  need = S.need;
  mask |= 255u << shift;
  return S.count;
}

// Block-wide exclusive scan of one value per thread (wave scans, then the
// wave totals through LDS); *total receives the block sum. The closing barrier
// lets a later scan reuse S.wsum; the last scan of a kernel (kLast) skips it.
template <bool kLast = false>
__device__ uint32_t block_exclusive_scan(uint32_t v, Shared& S, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) S.wsum[wave] = x;
  __syncthreads();
  uint32_t base = 0u, tot = 0u;
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t ws = S.wsum[w];
    base += w < wave ? ws : 0u;
    tot += ws;
  }
  if (!kLast) __syncthreads();
  *total = tot;
  return base + x - v;
}

// Ascending bitonic sort of a[0, P), P a power of two.
__device__ void bitonic_sort(uint64_t* a, int P) {
  const int tid = threadIdx.x;
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += kSelThreads) {
        const int i = 2 * stride * (t / stride) + (t % stride);
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const uint64_t x = a[i], y = a[j];
        if ((x > y) == up) {
          a[i] = y;
          a[j] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int k) {
  int P = 1;
  while (P < k) P <<= 1;
  return P;
}

// Set bit i of the LDS bitmap.
__device__ __forceinline__ void mark(Shared& S, uint32_t i) {
  atomicOr(&S.bitmap[i >> 5], 1u << (i & 31u));
}

// The k largest keys of the set `visit` enumerates (ties to the lower row)
// marked in the bitmap: two radix passes find the 16-bit bucket of the k-th
// largest key; rows above it are marked and the keys inside it are collected
// and sorted, unless the bucket holds more keys than the candidate list, in
// which case an exact 4-pass radix select finds the threshold key and the cut
// row among the keys equal to it. Every thread of the workgroup calls it.
template <class Visit>
__device__ void exact_select(Visit&& visit, int k, int nwords, Shared& S) {
  const int tid = threadIdx.x;
  // The 16-bit bucket of the k-th largest key.
  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)k;
  radix_pass(visit, 24, prefix, mask, need, S);
  const uint32_t in_bucket = radix_pass(visit, 16, prefix, mask, need, S);
  const uint32_t top16 = prefix >> 16;
  for (int w = tid; w < nwords; w += kSelThreads) S.bitmap[w] = 0u;
  if (tid == 0) S.n_cand = 0u;
  __syncthreads();

  if (in_bucket <= (uint32_t)kCandCap) {
    // Rows above the bucket are selected outright; keys inside it are candidates.
    visit([&](uint32_t key, uint32_t i, bool live) {
      if (!live) return;
      const uint32_t hi = key >> 16;
      if (hi > top16) mark(S, i);
      else if (hi == top16) S.cand[atomicAdd(&S.n_cand, 1u)] = sort_item(key, i);
    });
    __syncthreads();
    const int nc = (int)S.n_cand;  // = in_bucket >= need
    if (nc <= 64) {
      // One wave sorts the candidates in registers (no workgroup barriers).
      if (tid < 64) {
        uint64_t v = tid < nc ? S.cand[tid] : ~0ull;
        for (int size = 2; size <= 64; size <<= 1) {
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint32_t lo = __shfl_xor((uint32_t)v, stride);
            const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), stride);
            const uint64_t o = ((uint64_t)hi << 32) | lo;
            const bool up = (tid & size) == 0;
            const bool lower = (tid & stride) == 0;
            const uint64_t mn = v < o ? v : o, mx = v < o ? o : v;
            v = (lower == up) ? mn : mx;
          }
        }
        if (tid < (int)need) mark(S, (uint32_t)(v & 0xffffffffu));
      }
    } else {
      const int PC = pow2_at_least(nc);
      for (int i = nc + tid; i < PC; i += kSelThreads) S.cand[i] = ~0ull;
      __syncthreads();
      bitonic_sort(S.cand, PC);
      for (int j = tid; j < (int)need; j += kSelThreads)
        mark(S, (uint32_t)(S.cand[j] & 0xffffffffu));
    }
  } else {
    // Heavily tied scores: the exact threshold key T, then the cut index I, the
    // need-th lowest index among the keys equal to T.
    radix_pass(visit, 8, prefix, mask, need, S);
    radix_pass(visit, 0, prefix, mask, need, S);
    const uint32_t T = prefix;
    visit([&](uint32_t key, uint32_t i, bool live) {
      if (live && key == T) mark(S, i);
    });
    __syncthreads();
    const int per = (nwords + kSelThreads - 1) / kSelThreads;
    const int w0 = tid * per < nwords ? tid * per : nwords;
    const int w1 = w0 + per < nwords ? w0 + per : nwords;
    uint32_t cnt = 0u;
    for (int w = w0; w < w1; ++w) cnt += __popc(S.bitmap[w]);
    uint32_t tot;
    uint32_t off = block_exclusive_scan(cnt, S, &tot);
    if (off < need && need <= off + cnt) {
      for (int w = w0; w < w1; ++w) {
        uint32_t bits = S.bitmap[w];
        while (bits) {
          const uint32_t bit = __builtin_ctz(bits);
          bits &= bits - 1u;
          if (++off == need) S.cut = (uint32_t)(w * 32) + bit;
        }
      }
    }
    __syncthreads();
    const uint32_t I = S.cut;
    for (int w = tid; w < nwords; w += kSelThreads) S.bitmap[w] = 0u;
    __syncthreads();
    visit([&](uint32_t key, uint32_t i, bool live) {
      if (live && (key > T || (key == T && i <= I))) mark(S, i);
    });
  }
  __syncthreads();
}

// Window entries of token b (n_win) and the size k of its index part.
__device__ __forceinline__ void token_counts(const SelectLaunch& a, int pos, int* n_win_out,
                                             int* k_out) {
  int n_win = 0;
  if (a.window > 0 && pos >= 0) n_win = pos + 1 < a.window ? pos + 1 : a.window;
  if (n_win > a.topk) n_win = a.topk;
  int k = a.k_idx < a.n_idx ? a.k_idx : a.n_idx;
  if (k > a.topk - n_win) k = a.topk - n_win;
  if (k < 0) k = 0;
  *n_win_out = n_win;
  *k_out = k;
}

// Row b of the selection around its index part: the window rows, oldest
// first, then -1 after the n_win + k entries. Every thread of the workgroup
// calls it; returns n_win and k.
__device__ __forceinline__ void window_and_pads(const SelectLaunch& a, int b, int nthreads,
                                                int* n_win_out, int* k_out) {
  const int tid = threadIdx.x;
  int32_t* out = a.sel + (int64_t)b * a.topk;
  const int pos = a.pos[b];
  int n_win, k;
  token_counts(a, pos, &n_win, &k);
  for (int j = tid; j < a.topk; j += nthreads) {
    if (j < n_win) {
      const int p = pos - n_win + 1 + j;  // >= 0
      out[j] = (int32_t)(a.win_base + p % a.window);
    } else if (j >= n_win + k) {
      out[j] = -1;
    }
  }
  *n_win_out = n_win;
  *k_out = k;
}

// The index part of one token with one workgroup: the k (>= 1) best of the n
// scores of row `sc`, in ascending row order, into dst[0, k). The calling
// kernel ends right after it (its last scan has no closing barrier).
__device__ __forceinline__ void index_part(const float* sc, int n, int k, int32_t* dst, Shared& S) {
  const int tid = threadIdx.x;
  const int nwords = (n + 31) >> 5;

  // 1. Prefilter (rows >= kPreMinN): a sample of the keys gives a lower bound
  //    L0 meant to lie below the k-th largest key; one pass keeps every key
  //    >= L0. When at least k keys were kept (so the k-th largest key is
  //    >= L0 and the top k are all among them) and they fit, the exact
  //    selection runs on the kept keys in LDS; otherwise on all keys. Either
  //    way the result is exact; the sample only decides how fast.
  bool use_pre = false;
  if (n >= kPreMinN) {
    if (tid < 2 * kSampleRuns) {
      const int run = tid >> 1;
      const int64_t start = ((int64_t)run * (n - 8) / (kSampleRuns - 1)) & ~(int64_t)3;
      const float4 f = *reinterpret_cast<const float4*>(sc + start + 4 * (tid & 1));
      S.sample[4 * tid + 0] = order_key(f.x);
      S.sample[4 * tid + 1] = order_key(f.y);
      S.sample[4 * tid + 2] = order_key(f.z);
      S.sample[4 * tid + 3] = order_key(f.w);
    }
    if (tid == 0) S.n_pre = 0u;
    __syncthreads();
    // The k-th largest key sits near sample rank k * kSample / n; go four
    // standard deviations (plus a margin) deeper and take the lower end of
    // that key's 16-bit bucket.
    const int mu = (int)(((int64_t)k * kSample) / n);
    int r0 = mu + 4 * ((int)sqrtf((float)mu) + 1) + 8;
    if (r0 > kSample - 1) r0 = kSample - 1;
    if ((int64_t)(r0 + 1) * n <= (int64_t)kPreCap * kSample * 3 / 4) {  // expected keep fits
      auto visit_sample = [&](auto fn) {
        for (int i = tid; i < kSample; i += kSelThreads) fn(S.sample[i], (uint32_t)i, true);
      };
      uint32_t sp = 0u, sm = 0u, sneed = (uint32_t)(r0 + 1);
      radix_pass(visit_sample, 24, sp, sm, sneed, S);
      radix_pass(visit_sample, 16, sp, sm, sneed, S);
      const uint32_t L0 = sp;  // low 16 bits are zero: the bucket's smallest key
      const int lane = tid & 63;
      // Per chunk, each lane counts its kept keys, a wave scan gives each lane
      // its offset, and one LDS atomic per wave reserves the wave's space.
      const int nv = n >> 2;
      for (int vbase = 0; vbase < nv; vbase += kSelThreads * kLoads) {
        Chunk c;
        load_chunk(sc, nv, vbase, c);
        uint32_t cnt = 0u;
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) cnt += (c.valid[u] && c.key[u][e] >= L0) ? 1u : 0u;
        const uint32_t incl = wave_incl_scan(cnt);
        uint32_t base = 0u;
        if (lane == 63) base = atomicAdd(&S.n_pre, incl);
        uint32_t pos = __builtin_amdgcn_readlane(base, 63) + incl - cnt;
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
          const uint32_t i0 = 4u * (uint32_t)(vbase + tid + kSelThreads * u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (c.valid[u] && c.key[u][e] >= L0) {
              if (pos < (uint32_t)kPreCap) S.pre[pos] = sort_item(c.key[u][e], i0 + e);
              ++pos;
            }
          }
        }
      }
      const int tail = n & 3;
      if (tid < tail) {
        const int i = 4 * nv + tid;
        const uint32_t key = order_key(sc[i]);
        if (key >= L0) {
          const uint32_t pos = atomicAdd(&S.n_pre, 1u);
          if (pos < (uint32_t)kPreCap) S.pre[pos] = sort_item(key, (uint32_t)i);
        }
      }
      __syncthreads();
      const uint32_t kept = S.n_pre;
      use_pre = kept >= (uint32_t)k && kept <= (uint32_t)kPreCap;
    }
  }

  // 2. Exact selection of the top k of the chosen key set into the bitmap.
  if (use_pre) {
    const int kept = (int)S.n_pre;
    exact_select([&](auto fn) {
      for (int i = tid; i < kept; i += kSelThreads) {
        const uint64_t it = S.pre[i];
        fn(~(uint32_t)(it >> 32), (uint32_t)it, true);
      }
    }, k, nwords, S);
  } else {
    exact_select([&](auto fn) { for_each_key(sc, n, fn); }, k, nwords, S);
  }

  // 3. The chosen rows in ascending order.
  const int per = (nwords + kSelThreads - 1) / kSelThreads;
  const int w0 = tid * per < nwords ? tid * per : nwords;
  const int w1 = w0 + per < nwords ? w0 + per : nwords;
  uint32_t cnt = 0u;
  for (int w = w0; w < w1; ++w) cnt += __popc(S.bitmap[w]);
  uint32_t tot;
  uint32_t off = block_exclusive_scan<true>(cnt, S, &tot);  // index_part ends its kernel
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = S.bitmap[w];
    while (bits) {
      const uint32_t bit = __builtin_ctz(bits);
      bits &= bits - 1u;
      dst[off++] = (int32_t)((uint32_t)(w * 32) + bit);
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void build_selection_kernel(SelectLaunch a) {
  __shared__ Shared S;
  const int b = blockIdx.x;
  int n_win, k;
  window_and_pads(a, b, kSelThreads, &n_win, &k);
  if (k == 0) return;
  index_part(a.scores + (int64_t)b * a.score_stride, a.n_idx, k,
             a.sel + (int64_t)b * a.topk + n_win, S);
}

// --- split builder: several workgroups per token ----------------------------
//
// select_filter_kernel, workgroup (part p, token b): candidates
// [p * kSelectPartRows, (p + 1) * kSelectPartRows), 16 contiguous ones per
// thread, and the token's sample (the runs of the one-workgroup prefilter). A
// 12-bit histogram of the sample keys gives the bound L0: the lower edge of
// the key bucket holding the sample key of rank r0 from the top (r0 as in the
// one-workgroup prefilter). The part's keys >= L0 are written in row order as
// (key, row) items (the first kSelectPartCap of them) with their count.
//
// select_merge_kernel, one workgroup per token: every item slot is loaded as
// 16-byte vectors; the items go to LDS in part order (so in row order) while a
// first digit min((key - L0) >> 11, 4095) is counted; one wave finds the digit
// that holds the k-th largest key; the threads count the 11 bits below it over
// the items they hold in registers, and one wave finds the k-th largest key T
// and how many keys equal to T belong to the selection (the first ones in row
// order). When that digit is the open-ended last one, three radix passes (12,
// 12 and 8 bits from the top) over the keys at or above it find T instead. A
// block scan of (keys above T, keys equal to T) writes the chosen rows in
// ascending order. When a part kept more items than its capacity, fewer than k
// keys were kept in all (the k-th largest key lies below L0), or more than
// kPreCap, the token runs the one-workgroup index part instead. The result is
// exact either way.

constexpr int kFiltThreads = 256;
constexpr int kFiltRows = kSelectPartRows / kFiltThreads;  // contiguous candidates per thread
constexpr int kDigitBins = 4096;                           // 12-bit digits
constexpr int kLowBits = 11;                               // second digit: key bits below the first
constexpr int kHeadWords = 64;                             // a token's head: part counts, bound
constexpr int kBoundWord = 32;                             // head word holding the bound L0
constexpr int kMaxParts = kSelectMaxCandidates / kSelectPartRows;
constexpr uint32_t kNotFiltered = 0xffffffffu;             // count of a part that kept nothing

static_assert(kMaxParts <= kBoundWord && kMaxParts <= 64, "part counts: one word each, one wave");
static_assert(kFiltRows % 4 == 0, "a filter thread reads whole 16-byte vectors");
static_assert(kPreCap < (1 << 16), "the merge packs two item counts in one word");
static_assert(kDigitBins <= kCopies * kBins && (1 << kLowBits) <= kWords, "merge histograms in LDS");

__host__ __device__ __forceinline__ size_t token_ws_bytes(int parts) {
  return (size_t)kHeadWords * 4 + (size_t)parts * kSelectPartCap * 8;
}

// r0 of the prefilter: the sample rank (from the top) whose key bounds the
// kept set, or -1 when the expected keep would not fit the merge.
__device__ __forceinline__ int sample_rank(int k, int n) {
  const int mu = (int)(((int64_t)k * kSample) / n);
  int r0 = mu + 4 * ((int)sqrtf((float)mu) + 1) + 8;
  if (r0 > kSample - 1) r0 = kSample - 1;
  if ((int64_t)(r0 + 1) * n > (int64_t)kPreCap * kSample * 3 / 4) return -1;
  return r0;
}

// Exclusive scan of one value per thread over a workgroup of NT threads; *total
// receives the sum. wsum holds NT / 64 words of LDS, which are not reused (no
// closing barrier).
template <int NT>
__device__ __forceinline__ uint32_t wg_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t base = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t ws = wsum[w];
    base += w < wave ? ws : 0u;
    tot += ws;
  }
  *total = tot;
  return base + x - v;
}

// Wave 0 alone: the bin of an LDS histogram of 64 * PER bins (16-byte
// aligned) that holds the need-th largest counted key (need at most the
// count), and the rank left inside that bin. Two wave-wide suffix counts and no
// workgroup barrier: lane l sums bins PER l .. PER l + PER - 1 (its 16-byte
// reads rotated by lane, so the lanes start on different banks), a scan picks
// the lane range holding the key, then lane j reads bin j of that range and a
// second scan picks the bin. Every lane returns the same values.
template <int PER>
__device__ __forceinline__ void wave_find_bin(const uint32_t* hist, uint32_t need, uint32_t* bin,
                                              uint32_t* left) {
  static_assert(PER % 4 == 0 && PER <= 64 && (PER & (PER - 1)) == 0, "bins per lane");
  constexpr int NV = PER / 4;
  const int lane = threadIdx.x & 63;
  const uint4* hv = reinterpret_cast<const uint4*>(hist) + NV * lane;
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint4 v = hv[(i + lane) & (NV - 1)];
    c += v.x + v.y + v.z + v.w;
  }
  const uint32_t incl = wave_incl_scan(c);
  const uint32_t above = __builtin_amdgcn_readlane(incl, 63) - incl;  // keys in higher lanes
  const int L = __builtin_ctzll(__ballot(above < need && need <= above + c));
  const uint32_t need2 = need - __builtin_amdgcn_readlane(above, L);
  const uint32_t x = lane < PER ? hist[PER * L + lane] : 0u;
  const uint32_t incl2 = wave_incl_scan(x);
  const uint32_t above2 = __builtin_amdgcn_readlane(incl2, 63) - incl2;
  const int j = __builtin_ctzll(__ballot(above2 < need2 && need2 <= above2 + x));
  *bin = (uint32_t)(PER * L + j);
  *left = need2 - __builtin_amdgcn_readlane(above2, j);
}

__global__ __launch_bounds__(kFiltThreads) void select_filter_kernel(SelectLaunch a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kDigitBins];
  __shared__ uint32_t wsum[kFiltThreads / 64];
  __shared__ uint32_t s_bound;
  const int p = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  unsigned char* tws = static_cast<unsigned char*>(a.ws) + (size_t)b * token_ws_bytes(a.parts);
  uint32_t* head = reinterpret_cast<uint32_t*>(tws);
  uint2* items = reinterpret_cast<uint2*>(tws + kHeadWords * 4) + (size_t)p * kSelectPartCap;
  const int n = a.n_idx;  // >= kSelectMinSplitRows
  const float* sc = a.scores + (int64_t)b * a.score_stride;
  // This thread's sample run (8 keys) and its 16 candidates, loaded together
  // with the token's position. Vectors past the last candidate re-read the
  // last one (a valid address) and are masked.
  const int64_t start = ((int64_t)tid * (n - 8) / (kSampleRuns - 1)) & ~(int64_t)3;
  const float4 s0 = *reinterpret_cast<const float4*>(sc + start);
  const float4 s1 = *reinterpret_cast<const float4*>(sc + start + 4);
  const int row0 = p * kSelectPartRows + kFiltRows * tid;
  const int nv = (n + 3) >> 2;
  float4 f[kFiltRows / 4];
#pragma unroll
  for (int u = 0; u < kFiltRows / 4; ++u) {
    const int v = (row0 >> 2) + u;
    f[u] = *reinterpret_cast<const float4*>(sc + 4 * (int64_t)(v < nv ? v : nv - 1));
  }
  for (int i = tid; i < kDigitBins; i += kFiltThreads) hist[i] = 0u;
  int n_win, k;
  token_counts(a, a.pos[b], &n_win, &k);
  const int r0 = k > 0 ? sample_rank(k, n) : -1;
  if (r0 < 0) {  // nothing to select, or the merge takes the one-workgroup path
    if (tid == 0) head[p] = kNotFiltered;
    return;
  }
  __syncthreads();
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) atomicAdd(&hist[order_key(sv[e]) >> 20], 1u);
  __syncthreads();
  // The bucket of the (r0 + 1)-th largest sample key (2048 sample keys).
  if (tid < 64) {
    uint32_t bucket, left;
    wave_find_bin<kDigitBins / 64>(hist, (uint32_t)r0 + 1u, &bucket, &left);
    if (tid == 0) s_bound = bucket << 20;
  }
  __syncthreads();
  const uint32_t L0 = s_bound;  // the same in every part of the token
  // Keep the keys >= L0, in row order.
  uint32_t key[kFiltRows];
  uint32_t kept = 0u;
#pragma unroll
  for (int u = 0; u < kFiltRows / 4; ++u) {
    const float fv[4] = {f[u].x, f[u].y, f[u].z, f[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + 4 * u + e;
      key[4 * u + e] = order_key(fv[e]);
      kept |= (row < n && key[4 * u + e] >= L0) ? (1u << (4 * u + e)) : 0u;
    }
  }
  uint32_t total;
  uint32_t off = wg_exclusive_scan<kFiltThreads>((uint32_t)__popc(kept), wsum, &total);
#pragma unroll
  for (int j = 0; j < kFiltRows; ++j) {
    if ((kept >> j) & 1u) {
      if (off < (uint32_t)kSelectPartCap) items[off] = make_uint2(key[j], (uint32_t)(row0 + j));
      ++off;
    }
  }
  if (tid == 0) {
    head[p] = total;  // more than the part holds: the merge redoes the token
    if (p == 0) head[kBoundWord] = L0;
  }
}

// Find the digit of a histogram of nb digits (a power of two) that holds the
// need-th largest counted key: thread t owns digits per * t .. per * t + per - 1
// (per = nb / threads, or one digit for threads below nb); a block scan gives
// the keys above each range. S.prefix receives the digit and S.need the rank
// left inside it. Every thread calls it.
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nb, uint32_t need, Shared& S) {
  const int tid = threadIdx.x;
  const int per = nb >= kSelThreads ? nb / kSelThreads : 1;
  const int d0 = per * tid;
  uint32_t c = 0u;
  if (d0 < nb)
    for (int j = 0; j < per; ++j) c += hist[d0 + j];
  uint32_t tot;
  const uint32_t excl = block_exclusive_scan(c, S, &tot);
  uint32_t above = tot - excl - c;
  if (above < need && need <= above + c) {
    for (int j = per - 1; j >= 0; --j) {
      const uint32_t h = hist[d0 + j];
      if (above + h >= need) {
        S.prefix = (uint32_t)(d0 + j);
        S.need = need - above;
        break;
      }
      above += h;
    }
  }
  __syncthreads();
}

// The k largest (key, row) items of S.pre[0, total) (key in the high word,
// items in ascending row order, every key >= L0), ties to the lower row,
// written to dst as rows in ascending order. hist1 holds the counts of the
// first digit min((key - L0) >> kLowBits, kDigitBins - 1); hist2 is zero.
// mine(fn) calls fn(key) for the keys of S.pre this thread placed (the counting
// passes read them from registers).
template <class Mine>
__device__ __forceinline__ void select_items(Shared& S, int total, int k, uint32_t L0, const uint32_t* hist1,
                             uint32_t* hist2, int32_t* dst, Mine&& mine) {
  const int tid = threadIdx.x;
  constexpr uint32_t kLowMask = (1u << kLowBits) - 1u;
  if (tid < 64) {
    uint32_t d, left;
    wave_find_bin<kDigitBins / 64>(hist1, (uint32_t)k, &d, &left);
    if (tid == 0) {
      S.prefix = d;
      S.need = left;
    }
  }
  __syncthreads();
  const uint32_t d1 = S.prefix;
  uint32_t need = S.need;
  uint32_t T;
  if (d1 < (uint32_t)kDigitBins - 1u) {
    // the k-th largest key lies within 2^kLowBits of L0 + (d1 << kLowBits)
    mine([&](uint32_t key) {
      const uint32_t r = key - L0;
      if ((r >> kLowBits) == d1) atomicAdd(&hist2[r & kLowMask], 1u);
    });
    __syncthreads();
    if (tid < 64) {
      uint32_t d, left;
      wave_find_bin<(1 << kLowBits) / 64>(hist2, need, &d, &left);
      if (tid == 0) {
        S.prefix = d;
        S.need = left;
      }
    }
    __syncthreads();
    T = L0 + (d1 << kLowBits) + S.prefix;
    need = S.need;
  } else {
    // far above the bound (the last digit is a catch-all): radix over the keys
    // of that digit, 12, 12 and 8 bits from the top
    uint32_t prefix = 0u, mask = 0u;
    constexpr int kShift[3] = {20, 8, 0};
    constexpr int kBits[3] = {12, 12, 8};
#pragma unroll
    for (int ps = 0; ps < 3; ++ps) {
      const int shift = kShift[ps];
      const int nb = 1 << kBits[ps];
      for (int i = tid; i < nb; i += kSelThreads) hist2[i] = 0u;
      __syncthreads();
      mine([&](uint32_t key) {
        if (((key - L0) >> kLowBits) >= d1 && (key & mask) == prefix)
          atomicAdd(&hist2[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      });
      __syncthreads();
      find_digit(hist2, nb, need, S);
      prefix |= S.prefix << shift;
      need = S.need;
      mask |= (uint32_t)(nb - 1) << shift;
      __syncthreads();
    }
    T = prefix;
  }
  // The selection: every key above T and the first `need` keys equal to T in
  // row order. Thread t owns items [m t, m t + m), so one scan over threads of
  // (keys above T, keys equal to T), packed in one word, places every row.
  const int m = (total + kSelThreads - 1) / kSelThreads;
  const int i0 = m * tid < total ? m * tid : total;
  const int i1 = i0 + m < total ? i0 + m : total;
  uint32_t eq = 0u, gt = 0u;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = (uint32_t)(S.pre[i] >> 32);
    eq += key == T ? 1u : 0u;
    gt += key > T ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t pre = block_exclusive_scan<true>(gt << 16 | eq, S, &tot);  // counts < 2^14
  uint32_t rank = pre & 0xffffu;          // keys equal to T before this thread
  uint32_t off = (pre >> 16) + (rank < need ? rank : need);
  for (int i = i0; i < i1; ++i) {
    const uint64_t it = S.pre[i];
    const uint32_t key = (uint32_t)(it >> 32);
    bool take = key > T;
    if (key == T) take = rank++ < need;
    if (take) dst[off++] = (int32_t)(uint32_t)it;
  }
}

__global__ __launch_bounds__(kSelThreads) void select_merge_kernel(SelectLaunch a) {
  __shared__ __attribute__((aligned(16))) Shared S;
  __shared__ uint32_t part_cnt[kBoundWord];
  __shared__ uint32_t part_off[kBoundWord];
  __shared__ uint32_t s_total, s_fast;
  const int b = blockIdx.x, tid = threadIdx.x;
  const unsigned char* tws =
      static_cast<const unsigned char*>(a.ws) + (size_t)b * token_ws_bytes(a.parts);
  const uint32_t* head = reinterpret_cast<const uint32_t*>(tws);
  const uint4* items = reinterpret_cast<const uint4*>(tws + kHeadWords * 4);
  const int P = a.parts;
  const int pairs = P * kSelectPartCap / 2;  // 16-byte vectors of two (key, row) items
  // Every item slot, the part counts and the bound are loaded before any is
  // needed, together with the token's position: vector v = tid + 1024 u holds
  // slots 2 v and 2 v + 1.
  constexpr int kVecs = kMaxParts * kSelectPartCap / 2 / kSelThreads;
  uint4 it[kVecs];
#pragma unroll
  for (int u = 0; u < kVecs; ++u) {
    const int v = tid + kSelThreads * u;
    it[u] = v < pairs ? items[v] : make_uint4(0u, 0u, 0u, 0u);
  }
  const uint32_t c = tid < P ? head[tid] : 0u;
  const uint32_t L0 = head[kBoundWord];
  uint32_t* hist1 = &S.hist[0][0];
  uint32_t* hist2 = S.bitmap;
  for (int i = tid; i < kDigitBins; i += kSelThreads) hist1[i] = 0u;
  for (int i = tid; i < (1 << kLowBits); i += kSelThreads) hist2[i] = 0u;
  int n_win, k;
  window_and_pads(a, b, kSelThreads, &n_win, &k);
  if (k == 0) return;
  const float* sc = a.scores + (int64_t)b * a.score_stride;
  int32_t* dst = a.sel + (int64_t)b * a.topk + n_win;
  if (tid < 64) {
    const bool bad = tid < P && c > (uint32_t)kSelectPartCap;  // includes kNotFiltered
    const uint32_t x = wave_incl_scan(c);
    if (tid < kBoundWord) {
      part_cnt[tid] = c;
      part_off[tid] = x - c;
    }
    const bool any_bad = __any(bad);
    if (tid == 63) {
      s_total = x;
      s_fast = !any_bad && x >= (uint32_t)k && x <= (uint32_t)kPreCap;
    }
  }
  __syncthreads();
  if (!s_fast) {
    index_part(sc, a.n_idx, k, dst, S);
    return;
  }
  // Items to LDS in row order, counting the first digit on the way; bit 2 u + e
  // of `held` marks a slot that holds an item.
  uint32_t held = 0u;
#pragma unroll
  for (int u = 0; u < kVecs; ++u) {
    const int v = tid + kSelThreads * u;
    if (v < pairs) {
      const int p = 2 * v / kSelectPartCap, i = 2 * v % kSelectPartCap;  // i even
      const uint32_t cnt = part_cnt[p];
      const uint32_t key[2] = {it[u].x, it[u].z}, row[2] = {it[u].y, it[u].w};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if ((uint32_t)(i + e) < cnt) {
          held |= 1u << (2 * u + e);
          S.pre[part_off[p] + i + e] = ((uint64_t)key[e] << 32) | row[e];
          const uint32_t d = (key[e] - L0) >> kLowBits;
          atomicAdd(&hist1[d < (uint32_t)kDigitBins ? d : (uint32_t)kDigitBins - 1u], 1u);
        }
      }
    }
  }
  __syncthreads();
  select_items(S, (int)s_total, k, L0, hist1, hist2, dst, [&](auto fn) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      if ((held >> (2 * u)) & 1u) fn(it[u].x);
      if ((held >> (2 * u + 1)) & 1u) fn(it[u].z);
    }
  });
}

}  // namespace

hipError_t launch_select(const SelectLaunch& L, hipStream_t stream) {
  if (L.B <= 0 || L.k_idx > kSelectMaxK || L.n_idx > kSelectMaxCandidates) return hipErrorInvalidValue;
  hipLaunchKernelGGL(build_selection_kernel, dim3((unsigned)L.B), dim3(kSelThreads), 0, stream, L);
  return hipGetLastError();
}

}  // namespace da

namespace da {

int select_parts(int n_idx) {
  if (n_idx < kSelectMinSplitRows) return 0;
  return (n_idx + kSelectPartRows - 1) / kSelectPartRows;
}

size_t select_workspace_bytes(int B, int n_idx) {
  const int parts = select_parts(n_idx);
  return parts > 0 ? (size_t)B * token_ws_bytes(parts) : 0;
}

hipError_t launch_select_split(const SelectLaunch& L, hipStream_t stream) {
  if (L.B <= 0 || L.k_idx > kSelectMaxK || L.n_idx > kSelectMaxCandidates)
    return hipErrorInvalidValue;
  if (L.parts != select_parts(L.n_idx) || L.parts < 1 || !L.ws) return launch_select(L, stream);
  hipLaunchKernelGGL(select_filter_kernel, dim3((unsigned)L.parts, (unsigned)L.B), dim3(kFiltThreads),
                     0, stream, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_merge_kernel, dim3((unsigned)L.B), dim3(kSelThreads), 0, stream, L);
  return hipGetLastError();
}

}  // namespace da
