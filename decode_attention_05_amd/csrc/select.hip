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
    uint32_t x = t;  // inclusive suffix over lanes: digits >= 4 * tid
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(x, off);
      if (tid + off < 64) x += y;
    }
    uint32_t above = x - t;  // keys with digit >= 4 * (tid + 1)
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
// wave totals through LDS); *total receives the block sum.
__device__ uint32_t block_exclusive_scan(uint32_t v, Shared& S, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) S.wsum[wave] = x;
  __syncthreads();
  uint32_t base = 0u, tot = 0u;
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t ws = S.wsum[w];
    base += w < wave ? ws : 0u;
    tot += ws;
  }
  __syncthreads();
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

__global__ __launch_bounds__(kSelThreads) void build_selection_kernel(SelectLaunch a) {
  __shared__ Shared S;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const float* sc = a.scores + (int64_t)b * a.score_stride;
  int32_t* out = a.sel + (int64_t)b * a.topk;

  const int pos = a.pos[b];
  int n_win = 0;
  if (a.window > 0 && pos >= 0) n_win = pos + 1 < a.window ? pos + 1 : a.window;
  if (n_win > a.topk) n_win = a.topk;
  int k = a.k_idx < a.n_idx ? a.k_idx : a.n_idx;
  if (k > a.topk - n_win) k = a.topk - n_win;
  if (k < 0) k = 0;
  for (int j = tid; j < a.topk; j += kSelThreads) {
    if (j < n_win) {
      const int p = pos - n_win + 1 + j;  // >= 0
      out[j] = (int32_t)(a.win_base + p % a.window);
    } else if (j >= n_win + k) {
      out[j] = -1;
    }
  }
  if (k == 0) return;
  const int n = a.n_idx;
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
        uint32_t incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        uint32_t base = 0u;
        if (lane == 63) base = atomicAdd(&S.n_pre, incl);
        uint32_t pos = __shfl(base, 63) + incl - cnt;
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
  uint32_t off = block_exclusive_scan(cnt, S, &tot);
  int32_t* dst = out + n_win;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = S.bitmap[w];
    while (bits) {
      const uint32_t bit = __builtin_ctz(bits);
      bits &= bits - 1u;
      dst[off++] = (int32_t)((uint32_t)(w * 32) + bit);
    }
  }
}

}  // namespace

hipError_t launch_select(const SelectLaunch& L, hipStream_t stream) {
  if (L.B <= 0 || L.k_idx > kSelectMaxK || L.n_idx > kSelectMaxCandidates) return hipErrorInvalidValue;
  hipLaunchKernelGGL(build_selection_kernel, dim3((unsigned)L.B), dim3(kSelThreads), 0, stream, L);
  return hipGetLastError();
}

}  // namespace da
