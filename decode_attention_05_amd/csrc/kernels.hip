// kernels.hip -- split-K decode attention kernels for gfx950.
//
// The operation is softmax(scale * q . K^T) V for one query token per sequence
// (fuel-dispatch page "DecodeFlashSpec": q [B, Hq, 1, D] against the capacity
// buffers [B, Hkv, capacity, D] over the live prefix [0, k_len)), and its
// index-selected form (metrale page "AttnV41", decode_fixed_topk: rows named
// by a -1-padded selection, a pad adding exactly zero).
//
// Decomposition (split-K over keys, a.k.a. flash-decoding): one workgroup owns
// a (batch, kv head, head tile, split) and streams its chunk of keys once.
//   - The GQA query rows of the head tile are staged through LDS as fp32,
//     pre-multiplied by scale * log2(e) so the softmax runs in base 2.
//   - A KV row of D bf16 is read by D/8 lanes with one 16-byte load each (a
//     "row group"); a wave covers 64/(D/8) rows per load instruction, so every
//     load instruction of a wave reads 1 KiB of contiguous KV memory.
//   - Each row group keeps its own online-softmax state (running max m, sum l,
//     unnormalised output o) over the rows it visits. q.k partial dot products
//     are summed over the row group with a DPP butterfly.
//   - At the end the row groups of the workgroup are merged (in a fixed order:
//     deterministic), and the workgroup either writes the normalised bf16
//     output (one split) or its (o, m, l) partial for the combine kernel.
// Pads and tail rows are never loaded: their score is -inf, their weight +0
// and their value -0, so they leave every accumulator bit-for-bit unchanged.
#include "device_common.h"
#include "launch.h"

namespace da {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kUnroll = 2;     // rows per row group per iteration


template <int D, int GT, bool SPARSE>
__global__ __launch_bounds__(kThreads) void partial_kernel(PartialLaunch a) {
  constexpr int LPR = D / 8;     // lanes per KV row (16 bytes each)
  constexpr int RPW = 64 / LPR;  // rows per wave per load instruction
  constexpr int NRG = 4 * RPW;   // row groups per workgroup
  constexpr int STEP = NRG * kUnroll;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int rg = wave * RPW + lane / LPR;
  const int sub = lane % LPR;

  // Workgroup coordinates: split fastest, then head tile, then (b, kv head).
  const int tiles = a.G / GT;
  int wg = blockIdx.x;
  const int s = wg % a.S;
  wg /= a.S;
  const int ht = wg % tiles;
  const int bh = wg / tiles;
  const int b = bh / a.Hkv, hkv = bh % a.Hkv;
  const int h0 = hkv * a.G + ht * GT;  // first query head of this tile

  __shared__ float q_lds[GT][D];
  __shared__ float o_lds[4][GT][D];
  __shared__ float m_lds[4][GT];
  __shared__ float l_lds[4][GT];

  for (int i = tid; i < GT * D; i += kThreads) {
    const int g = i / D, d = i % D;
    const uint16_t raw = a.q[((int64_t)b * a.Hq + h0 + g) * D + d];
    q_lds[g][d] = __uint_as_float((uint32_t)raw << 16) * a.qscale;
  }
  __syncthreads();

  float qr[GT][8];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[g][e] = q_lds[g][sub * 8 + e];

  float m[GT], l[GT], o[GT][8];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }

  const int bk = SPARSE ? (a.kv_batch == 1 ? 0 : b) : b;
  const int64_t kv_off = ((int64_t)bk * a.Hkv + hkv) * a.capacity * D + sub * 8;
  const uint4* __restrict__ kp = reinterpret_cast<const uint4*>(a.k + kv_off);
  const uint4* __restrict__ vp = reinterpret_cast<const uint4*>(a.v + kv_off);
  constexpr int ROW_U4 = D / 8;  // uint4 per KV row

  // Key range of this split: rows [j0, j1) (dense) or selection entries [j0, j1).
  const int64_t j0 = (int64_t)s * a.chunk;
  const int64_t j_end = SPARSE ? (int64_t)a.topk : a.k_len;
  const int64_t j1 = (j0 + a.chunk < j_end) ? j0 + a.chunk : j_end;
  const int32_t* sel_row = SPARSE ? a.sel + (int64_t)b * a.topk : nullptr;

  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
  const uint4 negzero4 = make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u);

  for (int64_t base = j0; base < j1; base += STEP) {
    uint4 kr[kUnroll], vr[kUnroll];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = base + rg + NRG * u;
      int64_t row = j;
      bool ok = j < j1;
      if constexpr (SPARSE) {
        const int32_t r = ok ? sel_row[j] : -1;
        ok = r >= 0 && (int64_t)r < a.k_len;
        row = r;
      }
      valid[u] = ok;
      if (ok) {
        kr[u] = kp[row * ROW_U4];
        vr[u] = vp[row * ROW_U4];
      } else {
        kr[u] = zero4;
        vr[u] = negzero4;  // -0: adding p * (-0) leaves any accumulator unchanged
      }
    }

    float sc[kUnroll][GT];
    float vf[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      unpack8(kr[u], kf);
      unpack8(vr[u], vf[u]);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = fmaf(qr[g][e], kf[e], p);
        p = group_sum<LPR>(p);
        sc[u][g] = valid[u] ? p : kNegInf;
      }
    }

#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mb = m[g];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) mb = fmaxf(mb, sc[u][g]);
      if (mb == kNegInf) continue;  // nothing valid seen yet by this row group
      const float alpha = exp2_fast(m[g] - mb);
      float p[kUnroll];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        p[u] = exp2_fast(sc[u][g] - mb);
        ps += p[u];
      }
      l[g] = l[g] * alpha + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = o[g][e] * alpha;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc = fmaf(p[u], vf[u][e], acc);
        o[g][e] = acc;
      }
      m[g] = mb;
    }
  }

  // Merge the row groups of each wave (lanes that hold the same d slice).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      float oo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) oo[e] = __shfl_xor(o[g][e], off);
      if (mo == kNegInf) continue;  // partner empty: keep ours
      if (m[g] == kNegInf) {        // we are empty: take the partner's
        m[g] = mo;
        l[g] = lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = oo[e];
        continue;
      }
      const float M = fmaxf(m[g], mo);
      const float wa = exp2_fast(m[g] - M), wb = exp2_fast(mo - M);
      l[g] = l[g] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = o[g][e] * wa + oo[e] * wb;
      m[g] = M;
    }
  }

  // Row group 0 of every wave publishes the wave's state.
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o_lds[wave][g][sub * 8 + e] = o[g][e];
      if (sub == 0) {
        m_lds[wave][g] = m[g];
        l_lds[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  // Merge the four waves in order 0..3 and emit: thread t owns head t / LPR and
  // the 8 values at d = (t % LPR) * 8.
  if (tid < GT * LPR) {
    const int g = tid / LPR, d0 = (tid % LPR) * 8;
    float M = kNegInf, L = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = m_lds[w][g];
      if (mw == kNegInf) continue;
      if (M == kNegInf) {
        M = mw;
        L = l_lds[w][g];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = o_lds[w][g][d0 + e];
        continue;
      }
      const float Mn = fmaxf(M, mw);
      const float wa = exp2_fast(M - Mn), wb = exp2_fast(mw - Mn);
      L = L * wa + l_lds[w][g] * wb;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * wa + o_lds[w][g][d0 + e] * wb;
      M = Mn;
    }
    const int64_t row = (int64_t)b * a.Hq + h0 + g;
    if (a.S == 1) {
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      uint4 r;
      r.x = pack2_bf16(acc[0] * inv, acc[1] * inv);
      r.y = pack2_bf16(acc[2] * inv, acc[3] * inv);
      r.z = pack2_bf16(acc[4] * inv, acc[5] * inv);
      r.w = pack2_bf16(acc[6] * inv, acc[7] * inv);
      *reinterpret_cast<uint4*>(a.out + row * D + d0) = r;
    } else {
      float* po = a.part_o + (row * a.S + s) * D + d0;
      reinterpret_cast<float4*>(po)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(po)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      if (d0 == 0) {
        a.part_m[row * a.S + s] = M;
        a.part_l[row * a.S + s] = L;
      }
    }
  }
}

// Log-sum-exp combine of S partials per output row. Splits with no valid key
// (m = -inf) are skipped; the first non-empty split initialises the sums, so a
// single non-empty split reproduces the one-split output bit for bit.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(PartialLaunch a) {
  constexpr int PER = D / 64;  // outputs per lane
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const float* pm = a.part_m + row * a.S;
  const float* pl = a.part_l + row * a.S;
  const float* po = a.part_o + row * a.S * D;

  float M = kNegInf;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, pm[s]);

  float L = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  bool first = true;
  if (M != kNegInf) {
    for (int s = 0; s < a.S; ++s) {
      const float ms = pm[s];
      if (ms == kNegInf) continue;
      const float w = exp2_fast(ms - M);
      if (first) {
        L = pl[s] * w;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = po[s * D + lane * PER + e] * w;
        first = false;
      } else {
        L = L + pl[s] * w;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = acc[e] + po[s * D + lane * PER + e] * w;
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  uint16_t* dst = a.out + row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[e] = (uint16_t)f32_to_bf16_rne(acc[e] * inv);
}

template <int D, bool SPARSE>
hipError_t launch_partial_d(const PartialLaunch& L, hipStream_t stream) {
  const int tiles = L.G / L.heads_per_wg;
  const int64_t grid = (int64_t)L.B * L.Hkv * tiles * L.S;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(kThreads);
  switch (L.heads_per_wg) {
    case 1: hipLaunchKernelGGL((partial_kernel<D, 1, SPARSE>), g, blk, 0, stream, L); break;
    case 2: hipLaunchKernelGGL((partial_kernel<D, 2, SPARSE>), g, blk, 0, stream, L); break;
    case 4: hipLaunchKernelGGL((partial_kernel<D, 4, SPARSE>), g, blk, 0, stream, L); break;
    case 8: hipLaunchKernelGGL((partial_kernel<D, 8, SPARSE>), g, blk, 0, stream, L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partial(const PartialLaunch& L, hipStream_t stream) {
  if (L.D == 128) return L.sparse ? launch_partial_d<128, true>(L, stream)
                                  : launch_partial_d<128, false>(L, stream);
  if (L.D == 64) return L.sparse ? launch_partial_d<64, true>(L, stream)
                                 : launch_partial_d<64, false>(L, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const PartialLaunch& L, hipStream_t stream) {
  const int64_t rows = (int64_t)L.B * L.Hq;
  if (rows <= 0 || rows > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (L.D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)rows), dim3(64), 0, stream, L);
  else if (L.D == 64)
    hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)rows), dim3(64), 0, stream, L);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace da
