// kernels.hip -- decode attention kernels for gfx950 (CDNA4).
//
// The operation is softmax(scale * q . K^T) V for the query tokens of each
// sequence (fuel-dispatch page "DecodeFlashSpec": q [B, Hq, Sq, D] against the
// capacity buffers [B, Hkv, capacity, D] over the live prefix [0, k_len),
// grouped-query heads; Sq = 1 in decode, up to 16 with a causal mask over the
// last Sq positions), and its index-selected form (metrale page "AttnV41",
// decode_fixed_topk: rows named by a -1-padded selection; pads contribute
// nothing).
//
// Decompositions. attend_partial (split-K): one workgroup owns a (batch, kv
// head, head tile, split). attend_balanced (one live length per sequence):
// workgroup w owns an equal run of 32-key tiles of all (sequence, kv head,
// head tile) key streams laid end to end. Either way the workgroup calls
// attend_range on a key range, whose four waves each stream every fourth
// 32-key tile and keep their own base-2 online-softmax state, merged at the
// end. attend_balanced_waves (batches with more streams than the grid has
// waves): each wave owns a run and streams it alone (wave_stream).
// combine_splits / combine_balanced merge the partials (log-sum-exp).
//
// Per 32-key tile, for the (up to 16) query rows (heads x tokens) of the tile:
//   S^T[32 keys x 16 rows] = K_tile . Q^T  two v_mfma_f32_16x16x32_bf16 chains over D.
//       K is loaded from HBM straight into the A-operand layout: lane l holds
//       16 bytes of key row (l % 16); a wave instruction reads 64 contiguous
//       bytes of each of 16 rows, and the D/64 instructions cover the rows.
//   softmax: scores * scale * log2(e); per-row running max m (wave-reduced),
//       weights p = 2^(s - m) rounded to bf16 (the same rounded weights feed the
//       denominator l and the output), rescale of l and O by 2^(m_old - m_new).
//   O^T[D x 16 rows] += V_tile^T . P^T   D/16 MFMAs, one per 16-wide d tile.
//       V is staged through LDS (coalesced 1 KiB-per-instruction loads, XOR-
//       swizzled 16-byte chunks) and read back transposed with
//       ds_read_b64_tr_b16, which hands each lane 4 keys of one d column.
// The next tile's K and V loads are issued before the current tile is
// processed (register double buffering), so every wave keeps 16 KiB in flight.
//
// Keys outside the range, past k_len, hidden by the causal mask, or (sparse)
// pads and out-of-range entries get score -inf, so their weight is exactly 0;
// a slot without a valid key reads an allowed row (never one at or past k_len)
// and its V row is zeroed in LDS before use. A tile with no valid key is
// skipped.
#include "device_common.h"
#include "launch.h"

namespace da {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 32;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load with the non-temporal hint (K and V are read exactly
// once per call): measured on MI355X at ~7 TB/s for a plain read stream, against
// ~6 TB/s with the default cache policy.
__device__ __forceinline__ uint4 load_stream(const unsigned char* base, uint32_t off) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Reductions over lane pairs l, l ^ 16 and l, l ^ 32 with the gfx950 permlane
// swaps (VALU, no LDS round trip): with both operands the same register, each
// lane ends up holding its own value in one result and its partner's in the
// other, so a symmetric operation of the two results reduces the pair.
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ shortx4 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (shortx4 __attribute__((address_space(3)))*)(p));
}

template <int D>
struct Geometry {
  static constexpr int ROWB = D * 2;                 // bytes per KV row
  static constexpr int RU4 = D / 8;                  // 16-byte chunks per row
  static constexpr int NC = D / 32;                  // k-chunks of the q.k contraction
  static constexpr int NDT = D / 16;                 // 16-wide d tiles of the output
  static constexpr int VLD = kTileKeys * RU4 / 64;   // V loads per lane per tile
  static constexpr int SWZ = (D == 128) ? 7 : 3;     // key bits used by the LDS swizzle
  static constexpr int VTILE = kTileKeys * ROWB;     // LDS bytes per wave tile
  static constexpr int OSTRIDE = D + 4;              // floats per head row of the merge area
  static constexpr int MERGE = kWaves * 16 * OSTRIDE * 4;
  static constexpr int LDS = (kWaves * VTILE > MERGE ? kWaves * VTILE : MERGE);
};

// Physical LDS byte offset of 16-byte chunk `chunk` of key row `key` in a V tile.
template <int D>
__device__ __forceinline__ int v_off(int key, int chunk) {
  using Gm = Geometry<D>;
  return key * Gm::ROWB + ((chunk ^ (2 * (key & Gm::SWZ))) << 4);
}

template <int D>
struct TileRegs {
  uint4 k[2][Geometry<D>::NC];   // A operands: key rows (lane % 16) of the two 16-key halves
  uint4 v[Geometry<D>::VLD];     // V tile in natural order, destined for LDS
  uint32_t mask;                 // bit i: key i of the tile is valid
  int tau;                       // tile index within the range
};

// One 32-key tile of the online softmax for the wave's 16 query rows (lane
// group g = lane / 16, row r16 = lane % 16): V into this wave's LDS tile `vt`
// (slots outside R.mask zeroed), the score MFMAs against the query operand qop,
// the base-2 online softmax over the keys row r16 may see, and the P.V MFMAs
// into O. Row r16 sees the keys of R.mask, and with `cut` only the first
// rel - row_off of them (a causal row of several tokens). With R.mask = 0 the
// state is left as it is (every score -inf, every V row zeroed).
template <int D>
__device__ __forceinline__ void tile_step(const TileRegs<D>& R, bool cut, int rel, int row_off,
                                          const bf16x8 (&qop)[Geometry<D>::NC], unsigned char* vt,
                                          floatx4 (&O)[Geometry<D>::NDT], float& m, float& l,
                                          float qscale, int lane) {
  using Gm = Geometry<D>;
  constexpr int NC = Gm::NC, NDT = Gm::NDT, VLD = Gm::VLD, RU4 = Gm::RU4;
  const int g = lane >> 4, r16 = lane & 15;
  const uint32_t mask = R.mask;
  // V tile -> LDS (swizzled), for the transposed reads below. Rows of masked
  // slots are zeroed so that a non-finite value there cannot reach the output.
  if (mask == 0xffffffffu) {
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      *reinterpret_cast<uint4*>(vt + v_off<D>(idx / RU4, idx % RU4)) = R.v[r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      const bool ok = (mask >> (idx / RU4)) & 1u;
      *reinterpret_cast<uint4*>(vt + v_off<D>(idx / RU4, idx % RU4)) =
          ok ? R.v[r] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // S^T halves: keys 4g+i (first) and 16+4g+i (second) for head r16.
  floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k[0][c]), qop[c], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k[1][c]), qop[c], s1, 0, 0, 0);
  }
  uint32_t lm = mask;  // keys this lane's row may see
  if (cut) {
    const int n = rel - row_off;
    lm &= n >= 32 ? 0xffffffffu : (n <= 0 ? 0u : ((1u << n) - 1u));
  }
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k0 = 4 * g + i, k1 = 16 + 4 * g + i;
    sc[i] = ((lm >> k0) & 1u) ? s0[i] * qscale : kNegInf;
    sc[4 + i] = ((lm >> k1) & 1u) ? s1[i] * qscale : kNegInf;
  }
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
  mx = pair16_max(mx);
  mx = pair32_max(mx);
  const float m_new = fmaxf(m, mx);
  // -inf only for a row that has seen no key yet (causal rows): then every
  // weight below is exp2(-inf) = 0 and the state stays empty.
  const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = exp2_fast(m - m_ref);
  uint32_t pw[4];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pw[i] = pack_bf16(exp2_fast(sc[2 * i] - m_ref), exp2_fast(sc[2 * i + 1] - m_ref));
    psum += __uint_as_float(pw[i] << 16) + __uint_as_float(pw[i] & 0xffff0000u);
  }
  l = l * alpha + psum;
  m = m_new;
  const bf16x8 pop = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
  // O^T[d tile] = alpha * O^T + V^T P^T. Transposed V reads: lane (g, j = r16)
  // addresses key 4g + (j >> 2) (+16 for the second half), d = 16 dt + 4 (j & 3);
  // it receives V[4g + e][16 dt + j] for e = 0..3 (+16), the keys of its P slots.
  const int jk = 4 * g + (r16 >> 2);
  const int q4 = r16 & 3;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int chunk = 2 * dt + (q4 >> 1);
    const int sub = (q4 & 1) * 8;
    const shortx4 lo = lds_read_tr(vt + v_off<D>(jk, chunk) + sub);
    const shortx4 hi = lds_read_tr(vt + v_off<D>(16 + jk, chunk) + sub);
    const bf16x8 vop = __builtin_bit_cast(
        bf16x8, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                           __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))));
    O[dt] *= alpha;
    O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, O[dt], 0, 0, 0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
}

// Where attend_range leaves the result of its GT heads: the bf16 output rows
// (direct: head hh at out + hh * D), or fp32 unnormalised partials with their
// running max (base 2) and denominator (head hh at po + hh * po_stride and
// pm / pl + hh * pm_stride).
struct RangeOut {
  bool direct;
  uint16_t* out;
  float* po;
  float* pm;
  float* pl;
  int64_t po_stride;
  int64_t pm_stride;
};

// The whole workgroup attends the RT query rows row0 .. row0 + RT - 1 (rows of
// q [B, Hq, Sq, D] flattened: heads h0 .. h0 + RT / Sq - 1 of sequence b, every
// token of each) through kv head hkv over keys [j0, j1) of its KV stream
// (dense: rows of the cache; sparse: entries of the selection), k_len bounding
// the usable rows, and writes the merged result of its four waves to `ro`.
// With causal masking and several tokens, token t sees only keys below
// k_len - Sq + 1 + t. Every thread of the workgroup must call it with the same
// arguments; it synchronises the workgroup and uses all of `lds`, so a caller
// that calls it again first synchronises.
template <int D, bool SPARSE>
__device__ __forceinline__ void attend_range(const PartialLaunch& a, unsigned char* lds,
                                             float (&mrg_m)[kWaves][16],
                                             float (&mrg_l)[kWaves][16], int b, int hkv,
                                             int64_t row0, int RT, int64_t k_len, int64_t j0,
                                             int64_t j1, const RangeOut& ro) {
  using Gm = Geometry<D>;
  constexpr int NC = Gm::NC, NDT = Gm::NDT, VLD = Gm::VLD, RU4 = Gm::RU4;

  // Opaque copy of the thread id: the per-lane offsets derived from it are
  // rebuilt in each call rather than hoisted out of a caller's loop (where they
  // would stay live, and spill, across calls).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar addressing
  const int g = lane >> 4;   // lane group: which 8 bf16 of a 32-wide k slice
  const int r16 = lane & 15; // A-operand row / C-operand column

  // B operand of S^T = K Q^T: lane holds q row row0 + r16, elements 8 (4c + g) .. + 7.
  bf16x8 qop[NC];
  {
    const bool hv = r16 < RT;
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + (row0 + (hv ? r16 : 0)) * D);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qop[c] = as_bf16x8(hv ? qrow[4 * c + g] : make_uint4(0u, 0u, 0u, 0u));
  }

  const int bk = SPARSE ? (a.kv_batch == 1 ? 0 : b) : b;
  const int64_t kv_base = ((int64_t)bk * a.Hkv + hkv) * a.capacity * D;
  const uint4* __restrict__ kp = reinterpret_cast<const uint4*>(a.k + kv_base);
  const uint4* __restrict__ vp = reinterpret_cast<const uint4*>(a.v + kv_base);

  const int ntiles = (j1 > j0) ? (int)((j1 - j0 + kTileKeys - 1) / kTileKeys) : 0;
  // Causal masking of several tokens: keys from k_len - (Sq - 1) on are
  // visible to some rows only; row r16 (token t = r16 % Sq) sees keys below
  // k_len - (Sq - 1 - t). Offsets relative to j0 (a range spans < 2^31 keys):
  // tiles from tail_tau on need per-row masks; lim_rel is k_len - j0.
  int tail_tau = 0x7fffffff;
  int lim_rel = 0;
  if (!SPARSE && a.causal && a.Sq > 1) {
    const int64_t t0 = k_len - (a.Sq - 1) - j0;  // first key seen by some rows only
    tail_tau = t0 <= 0 ? 0 : (int)(t0 / kTileKeys);  // tile tau ends at 32 (tau + 1)
    lim_rel = (int)(k_len - j0);
  }
  const int row_off = a.Sq - 1 - r16 % a.Sq;
  const int32_t* sel_row = SPARSE ? a.sel + (int64_t)b * a.topk : nullptr;

  unsigned char* vt = lds + wave * Gm::VTILE;  // this wave's V tile

  // Issue the loads of tile `tau` (tile index within the split) into R. Every
  // load is unconditional, so the compiler can count them and wait only for the
  // tile being processed: a slot without a valid key reads an allowed row (the
  // last key of the split, or row 0 for a sparse pad), and its score and value
  // are masked off before use. No row at or beyond k_len is ever read.
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kp);
  const unsigned char* vbytes = reinterpret_cast<const unsigned char*>(vp);
  // Paged cache: the block-table entries of logical pages pg_first ..
  // pg_first + 63 of sequence b, one per lane (-1 past the row), so a tile
  // takes its page id with a lane read instead of a dependent load.
  int pg_first = 0;
  int pg_ids = -1;
  auto load_page_ids = [&](int first) {
    pg_first = first;
    const int lp = first + lane;
    pg_ids = lp < a.max_pages ? a.block_table[(int64_t)b * a.max_pages + lp] : -1;
  };
  if (!SPARSE && a.block_table) load_page_ids((int)((uint32_t)j0 / (uint32_t)a.page_size));
  auto load_tile = [&](TileRegs<D>& R, int tau) {
    const int64_t kt = j0 + (int64_t)tau * kTileKeys;
    R.tau = tau;
    const unsigned char* kb;
    const unsigned char* vb;
    int row_lane = 0;  // sparse: row of key (lane & 31) of the tile (0 for a pad)
    int last = 0;      // dense: last valid slot of the tile
    if constexpr (SPARSE) {
      const int64_t t = kt + (lane & 31);
      const int32_t r = (tau < ntiles && t < j1) ? sel_row[t] : -1;
      const bool ok = r >= 0 && (int64_t)r < k_len;
      row_lane = ok ? (int)r : 0;
      R.mask = (uint32_t)__ballot(ok);
      kb = kbytes;
      vb = vbytes;
    } else {
      const int64_t n = (tau < ntiles) ? j1 - kt : 0;
      R.mask = n >= 32 ? 0xffffffffu : (n <= 0 ? 0u : ((1u << n) - 1u));
      // A tile past the end re-reads the split's last key (cached, never used),
      // or row 0 when the sequence is empty (k_len = 0 leaves j1 = 0).
      const int64_t base = n > 0 ? kt : (j1 > 0 ? j1 - 1 : 0);
      last = n >= 32 ? 31 : (n > 0 ? (int)n - 1 : 0);
      if (a.block_table) {
        // Paged cache: a 32-key tile lies inside one page (tiles start at
        // multiples of 32, pages hold a multiple of 32 rows). A page id outside
        // [0, num_pages) is never read: the tile is dropped and its loads go to
        // page 0, as do the loads of a tile with no key.
        int64_t page = 0;
        int in_page = 0;
        if (n > 0) {
          const int lp = (int)((uint32_t)kt / (uint32_t)a.page_size);  // kt < 2^31
          in_page = (int)(kt - (int64_t)lp * a.page_size);
          if (lp < pg_first || lp >= pg_first + 64) load_page_ids(lp);
          page = __builtin_amdgcn_readlane(pg_ids, lp - pg_first);
          if (page < 0 || page >= a.num_pages) {
            page = 0;
            R.mask = 0u;
          }
        }
        const int64_t off = ((page * a.Hkv + hkv) * a.page_size + in_page) * Gm::ROWB;
        kb = reinterpret_cast<const unsigned char*>(a.k) + off;
        vb = reinterpret_cast<const unsigned char*>(a.v) + off;
      } else {
        kb = kbytes + base * Gm::ROWB;
        vb = vbytes + base * Gm::ROWB;
      }
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int slot = 16 * sb + r16;
      uint32_t row;
      if constexpr (SPARSE) row = (uint32_t)__shfl(row_lane, slot);
      else row = (uint32_t)(slot < last ? slot : last);
      const uint32_t off = row * (uint32_t)Gm::ROWB + (uint32_t)g * 16u;  // uniform base + 32-bit offset
#pragma unroll
      for (int c = 0; c < NC; ++c) R.k[sb][c] = load_stream(kb, off + 64u * c);
    }
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      const int slot = idx / RU4, chunk = idx % RU4;
      uint32_t row;
      if constexpr (SPARSE) row = (uint32_t)__shfl(row_lane, slot);
      else row = (uint32_t)(slot < last ? slot : last);
      R.v[r] = load_stream(vb, row * (uint32_t)Gm::ROWB + (uint32_t)chunk * 16u);
    }
  };

  floatx4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;  // running max (base 2) of head r16, same in every lane group
  float l = 0.f;      // this lane's share of the denominator of head r16
  const float qscale = a.qscale;

  // The tile update is written out here rather than shared with tile_step:
  // through the shared function the compiler scheduled this kernel's loop
  // differently and the long-context workload ran 1.2 % slower (same box).
  auto process_tile = [&](const TileRegs<D>& R) {
    const uint32_t mask = R.mask;
    if (mask == 0u) return;  // nothing valid: the state is left untouched
    // V tile -> LDS (swizzled), for the transposed reads below. Rows of masked
    // slots are zeroed so that a non-finite value there cannot reach the output.
    if (mask == 0xffffffffu) {
#pragma unroll
      for (int r = 0; r < VLD; ++r) {
        const int idx = r * 64 + lane;
        *reinterpret_cast<uint4*>(vt + v_off<D>(idx / RU4, idx % RU4)) = R.v[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < VLD; ++r) {
        const int idx = r * 64 + lane;
        const bool ok = (mask >> (idx / RU4)) & 1u;
        *reinterpret_cast<uint4*>(vt + v_off<D>(idx / RU4, idx % RU4)) =
            ok ? R.v[r] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // S^T halves: keys 4g+i (first) and 16+4g+i (second) for head r16.
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k[0][c]), qop[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k[1][c]), qop[c], s1, 0, 0, 0);
    }
    uint32_t lm = mask;  // keys this lane's row may see
    if (R.tau >= tail_tau) {
      const int rel = lim_rel - kTileKeys * R.tau - row_off;  // keys of this tile it sees
      lm &= rel >= 32 ? 0xffffffffu : (rel <= 0 ? 0u : ((1u << rel) - 1u));
    }
    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = 4 * g + i, k1 = 16 + 4 * g + i;
      sc[i] = ((lm >> k0) & 1u) ? s0[i] * qscale : kNegInf;
      sc[4 + i] = ((lm >> k1) & 1u) ? s1[i] * qscale : kNegInf;
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
    mx = pair16_max(mx);
    mx = pair32_max(mx);
    const float m_new = fmaxf(m, mx);
    // -inf only for a row that has seen no key yet (causal rows): then every
    // weight below is exp2(-inf) = 0 and the state stays empty.
    const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_ref);
    uint32_t pw[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = pack_bf16(exp2_fast(sc[2 * i] - m_ref), exp2_fast(sc[2 * i + 1] - m_ref));
      psum += __uint_as_float(pw[i] << 16) + __uint_as_float(pw[i] & 0xffff0000u);
    }
    l = l * alpha + psum;
    m = m_new;
    const bf16x8 pop = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    // O^T[d tile] = alpha * O^T + V^T P^T. Transposed V reads: lane (g, j = r16)
    // addresses key 4g + (j >> 2) (+16 for the second half), d = 16 dt + 4 (j & 3);
    // it receives V[4g + e][16 dt + j] for e = 0..3 (+16), the keys of its P slots.
    const int jk = 4 * g + (r16 >> 2);
    const int q4 = r16 & 3;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int chunk = 2 * dt + (q4 >> 1);
      const int sub = (q4 & 1) * 8;
      const shortx4 lo = lds_read_tr(vt + v_off<D>(jk, chunk) + sub);
      const shortx4 hi = lds_read_tr(vt + v_off<D>(16 + jk, chunk) + sub);
      const bf16x8 vop = __builtin_bit_cast(
          bf16x8, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                             __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))));
      O[dt] *= alpha;
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, O[dt], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  };

  // Wave `wave` takes tiles wave, wave + 4, ...; the next tile's loads are in
  // flight while the current one is processed.
  constexpr int kStep = kWaves;
  {
    TileRegs<D> A, B;
    int tau = wave;
    load_tile(A, tau);
    while (tau < ntiles) {
      load_tile(B, tau + kStep);
      process_tile(A);
      tau += kStep;
      if (tau >= ntiles) break;
      load_tile(A, tau + kStep);
      process_tile(B);
      tau += kStep;
    }
  }

  // Denominator of head r16 over the four lane groups.
  l = pair16_sum(l);
  l = pair32_sum(l);

  __syncthreads();  // every wave is done with its V tile: reuse LDS for the merge
  float* mo = reinterpret_cast<float*>(lds);
  if (g == 0) {
    mrg_m[wave][r16] = m;
    mrg_l[wave][r16] = l;
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    *reinterpret_cast<floatx4*>(mo + (wave * 16 + r16) * Gm::OSTRIDE + 16 * dt + 4 * g) = O[dt];
  __syncthreads();

  // Merge the waves in order 0..3. Thread t owns head t / 16 and D/16 values.
  constexpr int PER = D / 16;
  const int hh = tid >> 4, d0 = (tid & 15) * PER;
  if (hh < RT) {
    float M = kNegInf, L = 0.f, acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = mrg_m[w][hh];
      if (mw == kNegInf) continue;
      const float* src = mo + (w * 16 + hh) * Gm::OSTRIDE + d0;
      if (M == kNegInf) {
        M = mw;
        L = mrg_l[w][hh];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = src[e];
        continue;
      }
      const float Mn = fmaxf(M, mw);
      const float wa = exp2_fast(M - Mn), wb = exp2_fast(mw - Mn);
      L = L * wa + mrg_l[w][hh] * wb;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = acc[e] * wa + src[e] * wb;
      M = Mn;
    }
    if (ro.direct) {
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      uint32_t w4[PER / 2];
#pragma unroll
      for (int e = 0; e < PER / 2; ++e) w4[e] = pack_bf16(acc[2 * e] * inv, acc[2 * e + 1] * inv);
      uint16_t* dst = ro.out + (int64_t)hh * D + d0;
      if constexpr (PER == 8)
        *reinterpret_cast<uint4*>(dst) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      else
        *reinterpret_cast<uint2*>(dst) = make_uint2(w4[0], w4[1]);
    } else {
      float* po = ro.po + hh * ro.po_stride + d0;
#pragma unroll
      for (int e = 0; e < PER; e += 4)
        *reinterpret_cast<float4*>(po + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
      if (d0 == 0) {
        ro.pm[hh * ro.pm_stride] = M;
        ro.pl[hh * ro.pm_stride] = L;
      }
    }
  }
}

// Split-K pass: one workgroup per (batch, kv head, head tile, split), split
// fastest. Writes the bf16 output directly when the plan does not split (S = 1).
template <int D, bool SPARSE>
__global__ __launch_bounds__(kThreads, 2) void attend_partial(PartialLaunch a) {
  using Gm = Geometry<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Gm::LDS];
  __shared__ float mrg_m[kWaves][16];
  __shared__ float mrg_l[kWaves][16];

  const int GT = a.heads_per_wg;
  const int tiles_h = a.G / GT;
  int wg = blockIdx.x;
  const int s = wg % a.S;
  wg /= a.S;
  const int ht = wg % tiles_h;
  const int bh = wg / tiles_h;
  const int b = bh / a.Hkv, hkv = bh % a.Hkv;
  const int h0 = hkv * a.G + ht * GT;  // first query head of this tile

  // Live length and split size. With a device-resident length (plan-once
  // decode) the S splits share [0, k_len) evenly for whatever k_len the device
  // holds; a value outside [0, max_k_len] is clamped, and k_len = 0 yields zeros.
  int64_t k_len = a.k_len;
  int64_t chunk = a.chunk;
  if constexpr (!SPARSE) {
    if (a.k_len_dev) {
      const int64_t raw =
          __builtin_amdgcn_readfirstlane(a.k_len_dev[(int64_t)b * a.k_lens_stride]);
      k_len = raw < 0 ? 0 : (raw > a.k_len ? a.k_len : raw);
      chunk = (k_len + a.S - 1) / a.S;
      chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
      if (chunk == 0) chunk = kTileKeys;
    }
  }

  // This split: keys (dense) or selection entries (sparse) [j0, j1).
  const int64_t j0 = (int64_t)s * chunk;
  const int64_t j_end = SPARSE ? (int64_t)a.topk : k_len;
  const int64_t j1 = (j0 + chunk < j_end) ? j0 + chunk : j_end;

  const int64_t row0 = ((int64_t)b * a.Hq + h0) * a.Sq;
  RangeOut ro;
  ro.direct = a.S == 1;
  ro.out = a.out + row0 * D;
  ro.po = a.S > 1 ? a.part_o + (row0 * a.S + s) * D : nullptr;
  ro.pm = a.S > 1 ? a.part_m + row0 * a.S + s : nullptr;
  ro.pl = a.S > 1 ? a.part_l + row0 * a.S + s : nullptr;
  ro.po_stride = (int64_t)a.S * D;
  ro.pm_stride = a.S;
  attend_range<D, SPARSE>(a, lds, mrg_m, mrg_l, b, hkv, row0, GT * a.Sq, k_len, j0, j1, ro);
}

// --- length-balanced schedule (one live length per sequence) ----------------
//
// Key streams: one per (sequence b, kv head, head tile), of tiles_of(len_b)
// 32-key tiles, laid end to end sequence by sequence (shortest first for up to
// 64 sequences, see length_order; index order beyond), then kv head, then head
// tile.
// Run w (a workgroup, or a wave when streams are many, see runs_per_wave) takes
// tiles [w * per_run, (w + 1) * per_run) of that concatenation, so every run
// streams the same number of tiles whatever the mix of lengths. A stream that
// lies inside one run is finished there (bf16 output); a stream cut by a run
// boundary leaves one fp32 partial per run that touches it, in slot 0 of the
// run (the first stream of the run) or slot 1 (the last), and the combine
// merges them. Both kernels derive the schedule from the lengths alone, with
// the same integer arithmetic.

constexpr int64_t kMinTilesPerRun = 8;

__device__ __forceinline__ int64_t seq_len(const PartialLaunch& a, int b) {
  const int64_t raw = a.k_len_dev[(int64_t)b * a.k_lens_stride];
  return raw < 0 ? 0 : (raw > a.k_len ? a.k_len : raw);
}

__device__ __forceinline__ int64_t tiles_of(int64_t len) {
  return (len + kTileKeys - 1) / kTileKeys;
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// A value known to be equal in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Tiles per run for `total` tiles over all streams cut into `runs` runs.
__device__ __forceinline__ int64_t run_tiles(int64_t total, int64_t runs) {
  const int64_t even = (total + runs - 1) / runs;
  return even > kMinTilesPerRun ? even : kMinTilesPerRun;
}

// Runs: one per workgroup, or one per wave when the batch has at least as many
// key streams as the grid has waves. With many short streams a workgroup's run
// cuts through several of them, and every piece costs the four waves a merge
// behind a barrier; one wave per run streams its pieces alone (wave_stream),
// with the next piece's loads in flight while it finishes one, and writes its
// own rows. Decided from the shapes alone, the same way on the host (which
// kernel to launch) and in the merge.
__host__ __device__ __forceinline__ bool runs_per_wave(const PartialLaunch& a) {
  return (int64_t)a.B * a.Hkv * (a.G / a.heads_per_wg) >= (int64_t)a.balanced_wgs * kWaves;
}

// More than 64 sequences are read kLenGroup at a time, kLenGroup / 64 per
// lane (sequence base + 64 i + lane in slot i), all loads issued before any is
// used; 0 past the batch.
constexpr int kLenSlots = 8;
constexpr int kLenGroup = 64 * kLenSlots;

__device__ __forceinline__ void load_lengths(const PartialLaunch& a, int base,
                                             int (&len)[kLenSlots]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kLenSlots; ++i) {
    const int bb = base + 64 * i + lane;
    len[i] = bb < a.B ? (int)seq_len(a, bb) : 0;
  }
}

// Tiles over all streams (more than 64 sequences).
__device__ __forceinline__ int64_t total_tiles(const PartialLaunch& a, int streams_per_seq) {
  int64_t mine = 0;
  for (int base = 0; base < a.B; base += kLenGroup) {
    int len[kLenSlots];
    load_lengths(a, base, len);
#pragma unroll
    for (int i = 0; i < kLenSlots; ++i) {
      mine += tiles_of(len[i]);
    }
  }
  return uniform_i64(wave_sum_i64(mine)) * streams_per_seq;
}

// Up to 64 sequences are laid end to end shortest first (ties in index order).
// The two workgroups a CU holds do not stream at the same pace: the one
// dispatched first (the lower half of the grid) wins the CU's memory
// arbitration and finishes well ahead of the other, which then streams alone.
// A run cut into many short pieces pays a pipeline fill and a merge per piece;
// in the first half of the grid those bubbles are filled by the other
// workgroup, in the second half they are not. Shortest-first puts the runs of
// many pieces at the start of the concatenation, in the first half (measured
// on 32 sequences of 581 to 32768 keys: 162 us for the slowest CU in index
// order, 153 us shortest first, 152 us for equal lengths).
struct SeqOrder {
  int len;         // lane i: live length of sequence i (0 past the batch)
  int next;        // lane i: the sequence after i in the order (B after the last)
  int64_t before;  // lane i: tiles of every stream of the sequences before i
  int64_t total;   // tiles over all streams (the same in every lane)
};

__device__ __forceinline__ SeqOrder length_order(const PartialLaunch& a, int streams_per_seq) {
  const int lane = threadIdx.x & 63;
  SeqOrder o;
  o.len = lane < a.B ? (int)seq_len(a, lane) : 0;
  int rank = 0;
  int64_t before = 0;
  for (int j = 0; j < a.B; ++j) {
    const int lj = __builtin_amdgcn_readlane(o.len, j);
    const bool earlier = lj < o.len || (lj == o.len && j < lane);
    rank += earlier ? 1 : 0;
    before += earlier ? tiles_of(lj) : 0;
  }
  if (lane >= a.B) rank = lane;  // ranks stay a permutation of the 64 lanes
  o.before = before * streams_per_seq;
  o.total = uniform_i64(wave_sum_i64(lane < a.B ? tiles_of(o.len) : 0)) * streams_per_seq;
  const int order = __builtin_amdgcn_ds_permute(rank * 4, lane);  // order[rank] = sequence
  const int after = __builtin_amdgcn_ds_bpermute(((rank + 1) & 63) * 4, order);
  o.next = rank + 1 < a.B ? after : a.B;
  return o;
}

// The sequence whose streams hold tile t0 (< total) of the concatenation, and
// the first tile of its streams. Returns false only if no sequence does, which
// the schedule rules out.
__device__ __forceinline__ bool locate(const PartialLaunch& a, int64_t t0, int per_seq,
                                       bool by_length, const SeqOrder& o, int& b,
                                       int64_t& seq_start) {
  const int lane = threadIdx.x & 63;
  b = 0;
  seq_start = 0;
  if (by_length) {
    const int64_t n = tiles_of(o.len) * per_seq;
    const uint64_t hit = __ballot(lane < a.B && n > 0 && o.before <= t0 && t0 < o.before + n);
    if (hit == 0) return false;
    b = __builtin_ctzll(hit);
    seq_start = uniform_i64(__shfl(o.before, b));
    return true;
  }
  // Index order: the first b with per_seq * (tiles before b) <= t0 <
  // per_seq * (tiles up to b), 64 sequences per step, lane-parallel scan.
  int64_t acc = 0;
  bool found = false;
  for (int base = 0; base < a.B && !found; base += kLenGroup) {
    int len[kLenSlots];
    load_lengths(a, base, len);
#pragma unroll
    for (int i = 0; i < kLenSlots; ++i) {
      if (found) break;
      const int64_t n = tiles_of(len[i]) * per_seq;
      int64_t inc = n;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      inc += acc;
      const int64_t exc = inc - n;
      const uint64_t hit = __ballot(n > 0 && exc <= t0 && t0 < inc);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        b = base + 64 * i + src;
        seq_start = uniform_i64(__shfl(exc, src));
        found = true;
      }
      acc = uniform_i64(__shfl(inc, 63));
    }
  }
  b = __builtin_amdgcn_readfirstlane(b);
  return found;
}

// Live length of sequence bb as a wave-uniform value: from the lanes of the
// length order (up to 64 sequences) or from memory.
__device__ __forceinline__ int64_t uniform_len(const PartialLaunch& a, bool by_length,
                                               const SeqOrder& o, int bb) {
  return by_length ? (int64_t)__builtin_amdgcn_readlane(o.len, bb)
                   : (int64_t)__builtin_amdgcn_readfirstlane(seq_len(a, bb));
}

// The pieces of workgroup run `run` (tiles [run * per_run, (run + 1) * per_run)
// of the concatenation), one attend_range call per piece.
template <int D>
__device__ __forceinline__ void run_pieces(const PartialLaunch& a, unsigned char* lds,
                                           float (&mrg_m)[kWaves][16],
                                           float (&mrg_l)[kWaves][16], int64_t run,
                                           int64_t per_run, int64_t total, int per_seq,
                                           bool by_length, const SeqOrder& o) {
  const int GT = a.heads_per_wg;
  const int RT = GT * a.Sq;             // query rows of one stream
  const int tiles_h = a.G / GT;
  const int64_t t0 = run * per_run;
  if (t0 >= total) return;  // the whole workgroup leaves together
  const int64_t t1 = (t0 + per_run < total) ? t0 + per_run : total;

  int b;
  int64_t seq_start;  // first tile of sequence b's streams
  if (!locate(a, t0, per_seq, by_length, o, b, seq_start)) return;
  int64_t len = uniform_len(a, by_length, o, b);
  int64_t nb = tiles_of(len);  // tiles of each stream of sequence b
  if (nb == 0) return;         // unreachable: t0 < total lies in a non-empty sequence
  const int64_t rel = t0 - seq_start;
  int r = (int)(rel / nb);     // stream of sequence b: kv head * tiles_h + head tile
  int64_t jt = rel - (int64_t)r * nb;
  int64_t x = t0;
  for (;;) {
    const int64_t left = t1 - x;
    const int64_t nt = (nb - jt < left) ? nb - jt : left;
    const int hkv = r / tiles_h, ht = r % tiles_h;
    const int64_t row0 = ((int64_t)b * a.Hq + hkv * a.G + ht * GT) * a.Sq;
    RangeOut ro;
    ro.direct = (jt == 0 && nt == nb);  // the whole stream is in this run
    ro.out = a.out + row0 * D;
    const int64_t slot = (run * 2 + (x == t0 ? 0 : 1)) * RT;
    ro.po = a.part_o + slot * D;
    ro.pm = a.part_m + slot;
    ro.pl = a.part_l + slot;
    ro.po_stride = D;
    ro.pm_stride = 1;
    const int64_t j1 = (jt + nt) * kTileKeys;
    attend_range<D, false>(a, lds, mrg_m, mrg_l, b, hkv, row0, RT, len, jt * kTileKeys,
                           j1 < len ? j1 : len, ro);
    x += nt;
    if (x >= t1) break;
    // the merge area is read before the next range's V tiles land there
    __syncthreads();
    // Next stream: the next head tile / kv head, else the next non-empty sequence.
    jt = 0;
    if (++r == per_seq) {
      r = 0;
      do {
        b = by_length ? __builtin_amdgcn_readlane(o.next, b) : b + 1;
        if (b >= a.B) break;
        len = uniform_len(a, by_length, o, b);
        nb = tiles_of(len);
      } while (nb == 0);
      if (b >= a.B) break;  // unreachable: tiles remain before t1 <= total
    }
  }
}

// LDS bytes per wave that hold finished pieces of a run until the run ends. A
// record is a 16-byte header (first query row, flags, record bytes) and then
// either the bf16 output rows of a whole stream or the fp32 partial rows
// followed by (m, l) per row, the rows padded (rows a multiple of 256 bytes
// apart would put every row's lanes on the same LDS banks); the largest (16
// partial rows at D = 128) fits. Four waves' buffers and V tiles
// take 80 KiB at D = 128, so two workgroups share a CU's 160 KiB.
constexpr int kPieceBufBytes = 12288;

// Per-tile facts of the wave streamer (uniform across the wave).
constexpr int kTileFirst = 1;    // first tile of its piece: the softmax state starts empty
constexpr int kTileLast = 2;     // last tile of its piece: the piece's rows are written
constexpr int kTileDirect = 4;   // the piece is its whole stream: bf16 output
constexpr int kTileSlot1 = 8;    // the piece starts after the run does: partial slot 1
constexpr int kTileReal = 16;    // a tile of the run (else a re-read past its end)

template <int D>
struct StreamTile {
  TileRegs<D> t;                 // K, V and the key mask
  bf16x8 q[Geometry<D>::NC];     // the piece's query rows (B operand of the scores)
  int row0;                      // first query row of the tile's stream (q / out rows)
  int lim;                       // keys from the tile's first to its sequence's length,
                                 // at most 64 (several causal tokens; 64: no mask)
  int flags;
};

// Run `run` of one wave (tiles [t0, t1) of the concatenation) streamed as one
// tile sequence: the loads of the next tile are in flight while the current one
// is processed, across stream boundaries too. Every tile carries its own copy
// of its stream's query rows (loaded with its K and V, cached), so every load
// is unconditional and no register that a queued tile still needs is
// overwritten. A piece (the part of a stream inside the run) starts from an
// empty softmax state at its first tile and ends with a record of its rows:
// bf16 output for a whole stream, else an fp32 partial for slot 0 (the piece
// that starts the run) or 1 (the one that ends it) of the run.
// The records wait in the wave's LDS buffer `pb` and are written out when it
// is full and when the run ends. A global store issued between tile loads sits
// in the same in-order memory counter as the loads, so the wait for every tile
// loaded after it also waits for the store's acknowledgement, which under a
// full read stream takes about one loaded memory latency.
template <int D>
__device__ __forceinline__ void wave_stream(const PartialLaunch& a, unsigned char* vt,
                                            unsigned char* pb, int64_t run, int64_t per_run,
                                            int64_t total, int per_seq, bool by_length,
                                            const SeqOrder& o) {
  using Gm = Geometry<D>;
  constexpr int NC = Gm::NC, NDT = Gm::NDT, VLD = Gm::VLD, RU4 = Gm::RU4;
  const int64_t t0 = run * per_run;
  if (t0 >= total) return;  // the wave leaves
  const int64_t t1 = (t0 + per_run < total) ? t0 + per_run : total;

  // The per-lane values of the process step are derived afresh in every step
  // from an opaque copy of the lane id, so that they are not kept live (and
  // spilled) across the whole tile loop; the load addresses are derived once.
  auto fresh_lane = []() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t & 63;
  };
  const int GT = a.heads_per_wg, RT = GT * a.Sq, tiles_h = a.G / GT;
  const bool causal_rows = a.causal && a.Sq > 1;
  const float qscale = a.qscale;
  // Per-lane byte offset inside the query rows of a stream, fixed for the run.
  // Query lanes past the stream's RT rows read its last row: their columns of
  // the score and output tiles are never written out.
  const int lane_ld = threadIdx.x & 63;
  const uint32_t q_lane =
      (uint32_t)((lane_ld & 15) < RT ? (lane_ld & 15) : RT - 1) * Gm::ROWB + (uint32_t)(lane_ld >> 4) * 16u;

  // The load cursor: tile x of the concatenation, tile jt of stream r of
  // sequence cb (length clen, cnb tiles per stream). Past the run it stays on
  // the run's last tile, which the extra load at the end re-reads.
  int cb;
  int64_t seq_start;
  if (!locate(a, t0, per_seq, by_length, o, cb, seq_start)) return;
  // More than 64 sequences: the lengths of sequences len_base .. len_base + 63,
  // one per lane (0 past the batch), so that moving to the next sequence reads
  // a lane instead of waiting on a load (which would drain every tile load in
  // flight); reloaded once per 64 sequences.
  int len_base = cb & ~63;
  int len_win = 0;
  auto load_len_win = [&]() {
    const int bb = len_base + lane_ld;
    len_win = bb < a.B ? (int)seq_len(a, bb) : 0;
  };
  if (!by_length) load_len_win();
  auto next_len = [&](int bb) -> int64_t {
    if (by_length) return (int64_t)__builtin_amdgcn_readlane(o.len, bb);
    if (bb >= len_base + 64) {
      len_base = bb & ~63;
      load_len_win();
    }
    return (int64_t)__builtin_amdgcn_readlane(len_win, bb - len_base);
  };
  int64_t clen = next_len(cb);
  int64_t cnb = tiles_of(clen);
  if (cnb == 0) return;  // unreachable: t0 < total lies in a non-empty sequence
  int cr = (int)((t0 - seq_start) / cnb);
  int64_t cjt = (t0 - seq_start) - (int64_t)cr * cnb;
  int64_t cx = t0;

  auto advance = [&]() {
    if (cx + 1 >= t1) {
      cx = t1;
      return;
    }
    ++cx;
    if (++cjt < cnb) return;
    if (cr + 1 < per_seq) {
      ++cr;
      cjt = 0;
      return;
    }
    int nbq = cb;
    int64_t nlen = 0, nnb = 0;
    for (;;) {
      nbq = by_length ? __builtin_amdgcn_readlane(o.next, nbq) : nbq + 1;
      if (nbq >= a.B) {  // unreachable: tiles remain before t1 <= total
        cx = t1;
        cjt = cnb - 1;
        return;
      }
      nlen = next_len(nbq);
      nnb = tiles_of(nlen);
      if (nnb > 0) break;
    }
    cb = nbq;
    clen = nlen;
    cnb = nnb;
    cr = 0;
    cjt = 0;
  };

  // Paged cache: block-table entries pg_first .. pg_first + 63 of sequence
  // pg_b, one per lane.
  int pg_b = -1, pg_first = 0, pg_ids = -1;

  auto load = [&](StreamTile<D>& T) {
    const int lane = lane_ld;
    const int g = lane >> 4, r16 = lane & 15;
    const bool real = cx < t1;
    const int hkv = cr / tiles_h, ht = cr - hkv * tiles_h;
    const int64_t kt = cjt * kTileKeys;
    const int64_t left = clen - kt;  // >= 1: the cursor is on a tile of the stream
    const int nv = left >= kTileKeys ? kTileKeys : (int)left;
    // The re-read past the run reads only the last tile's last key row.
    const int last = real ? nv - 1 : 0;
    const int64_t row0_ld = real ? kt : kt + nv - 1;
    T.t.mask = real ? (nv == kTileKeys ? 0xffffffffu : ((1u << nv) - 1u)) : 0u;
    T.row0 = (int)(((int64_t)cb * a.Hq + hkv * a.G + ht * GT) * a.Sq);
    T.lim = causal_rows ? (left >= 64 ? 64 : (int)left) : 64;
    const int64_t sfirst = cx - cjt;  // the stream's first tile in the concatenation
    T.flags = (real ? kTileReal : 0) | ((cjt == 0 || cx == t0) ? kTileFirst : 0) |
              ((cjt == cnb - 1 || cx == t1 - 1) ? kTileLast : 0) |
              ((sfirst >= t0 && sfirst + cnb <= t1) ? kTileDirect : 0) |
              (sfirst > t0 ? kTileSlot1 : 0);
    {
      const unsigned char* qb = reinterpret_cast<const unsigned char*>(a.q + (int64_t)T.row0 * D);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        T.q[c] = as_bf16x8(*reinterpret_cast<const uint4*>(qb + q_lane + 64u * c));
    }
    const unsigned char* kb;
    const unsigned char* vb;
    if (a.block_table) {
      // A 32-key tile lies inside one page; a page id outside [0, num_pages) is
      // never read (the tile is dropped and its loads go to page 0).
      const int lp = (int)((uint32_t)kt / (uint32_t)a.page_size);  // kt < 2^31
      int64_t page;
      if (cb != pg_b || lp < pg_first || lp >= pg_first + 64) {
        pg_b = cb;
        pg_first = lp;
        const int e = lp + lane;
        pg_ids = e < a.max_pages ? a.block_table[(int64_t)cb * a.max_pages + e] : -1;
        page = __builtin_amdgcn_readlane(pg_ids, 0);
      } else {
        page = __builtin_amdgcn_readlane(pg_ids, lp - pg_first);
      }
      if (page < 0 || page >= a.num_pages) {
        page = 0;
        T.t.mask = 0u;
      }
      const int64_t in_page = row0_ld - (int64_t)lp * a.page_size;  // same page as kt
      const int64_t off = ((page * a.Hkv + hkv) * a.page_size + in_page) * Gm::ROWB;
      kb = reinterpret_cast<const unsigned char*>(a.k) + off;
      vb = reinterpret_cast<const unsigned char*>(a.v) + off;
    } else {
      const int64_t off = (((int64_t)cb * a.Hkv + hkv) * a.capacity + row0_ld) * Gm::ROWB;
      kb = reinterpret_cast<const unsigned char*>(a.k) + off;
      vb = reinterpret_cast<const unsigned char*>(a.v) + off;
    }
    // Slots past the stream's last key (its last tile) re-read that key.
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int slot = 16 * sb + r16;
      const uint32_t row = (uint32_t)(slot < last ? slot : last);
      const uint32_t off = row * (uint32_t)Gm::ROWB + (uint32_t)g * 16u;
#pragma unroll
      for (int c = 0; c < NC; ++c) T.t.k[sb][c] = load_stream(kb, off + 64u * c);
    }
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      const int slot = idx / RU4, chunk = idx % RU4;
      const uint32_t row = (uint32_t)(slot < last ? slot : last);
      T.t.v[r] = load_stream(vb, row * (uint32_t)Gm::ROWB + (uint32_t)chunk * 16u);
    }
  };

  // Records of finished pieces held in pb (pb_used bytes), written out by
  // flush: bf16 rows for a whole stream, else the fp32 partial with its (m, l)
  // in the run's slot.
  // Record rows padded so that the rows of one write instruction fall on
  // distinct LDS banks (for up to 8 bf16 or 4 fp32 rows).
  constexpr int kDirRow = D * 2 + 32, kPartRow = D * 4 + 64;
  const int direct_bytes = 16 + RT * kDirRow;
  const int partial_bytes = (16 + RT * kPartRow + RT * 8 + 15) & ~15;  // headers 16-byte aligned
  int pb_used = 0;
  auto flush = [&]() {
    const int lane = fresh_lane();
    const int g = lane >> 4, r16 = lane & 15;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int at = 0; at < pb_used;) {
      const unsigned char* rec = pb + at;
      const int4 h = *reinterpret_cast<const int4*>(rec);
      const int row0 = __builtin_amdgcn_readfirstlane(h.x);
      const int fl = __builtin_amdgcn_readfirstlane(h.y);
      at += __builtin_amdgcn_readfirstlane(h.z);
      if (r16 < RT) {
        if (fl & kTileDirect) {
          const uint2* src = reinterpret_cast<const uint2*>(rec + 16 + r16 * kDirRow + 8 * g);
          uint16_t* dst = a.out + ((int64_t)row0 + r16) * D + 4 * g;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            *reinterpret_cast<uint2*>(dst + 16 * dt) = src[4 * dt];
        } else {
          const float4* src = reinterpret_cast<const float4*>(rec + 16 + r16 * kPartRow + 16 * g);
          const float2 ml = *reinterpret_cast<const float2*>(rec + 16 + RT * kPartRow + r16 * 8);
          const int64_t slot = (run * 2 + ((fl & kTileSlot1) ? 1 : 0)) * RT + r16;
          float* po = a.part_o + slot * D + 4 * g;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<float4*>(po + 16 * dt) = src[4 * dt];
          if (g == 0) {
            a.part_m[slot] = ml.x;
            a.part_l[slot] = ml.y;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    pb_used = 0;
  };

  floatx4 O[NDT];
  float m = kNegInf, l = 0.f;
  auto process = [&](const StreamTile<D>& T) {
    const int lane = fresh_lane();
    const int g = lane >> 4, r16 = lane & 15;
    if (T.flags & kTileFirst) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      m = kNegInf;
      l = 0.f;
    }
    // Every processed tile goes through the update, also one without a valid
    // key (a page id out of range), which leaves the state as it is (its V
    // rows are zeroed and every score is -inf): one path, on which every load
    // of the tile is consumed.
    // row r16 sees T.lim - row_off keys of this tile (later tokens see more)
    tile_step<D>(T.t, T.lim < 64, T.lim, a.Sq - 1 - r16 % a.Sq, T.q, vt, O, m, l, qscale, lane);
    if (T.flags & kTileLast) {
      // The piece's record: lane (g, r16) holds values 16 dt + 4 g .. + 3 of row r16.
      float lt = pair16_sum(l);
      lt = pair32_sum(lt);
      const bool direct = (T.flags & kTileDirect) != 0;
      const int bytes = direct ? direct_bytes : partial_bytes;
      if (pb_used + bytes > kPieceBufBytes) flush();
      unsigned char* rec = pb + pb_used;
      if (lane == 0) *reinterpret_cast<int4*>(rec) = make_int4(T.row0, T.flags, bytes, 0);
      if (r16 < RT) {
        if (direct) {
          const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
          uint2* dst = reinterpret_cast<uint2*>(rec + 16 + r16 * kDirRow + 8 * g);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            dst[4 * dt] = make_uint2(pack_bf16(O[dt][0] * inv, O[dt][1] * inv),
                                     pack_bf16(O[dt][2] * inv, O[dt][3] * inv));
        } else {
          float4* dst = reinterpret_cast<float4*>(rec + 16 + r16 * kPartRow + 16 * g);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            dst[4 * dt] = make_float4(O[dt][0], O[dt][1], O[dt][2], O[dt][3]);
          if (g == 0)
            *reinterpret_cast<float2*>(rec + 16 + RT * kPartRow + r16 * 8) = make_float2(m, lt);
        }
      }
      pb_used += bytes;
    }
  };

  // Two tiles in flight: each one's registers are refilled right after it is
  // processed (a tile past the run is loaded but never processed).
  StreamTile<D> A, B;
  load(A);
  advance();
  load(B);
  advance();
  for (;;) {
    process(A);
    if (!(B.flags & kTileReal)) break;
    load(A);
    advance();
    process(B);
    if (!(A.flags & kTileReal)) break;
    load(B);
    advance();
  }
  flush();
}

// Length-balanced pass, one run per workgroup.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void attend_balanced(PartialLaunch a) {
  using Gm = Geometry<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Gm::LDS];
  __shared__ float mrg_m[kWaves][16];
  __shared__ float mrg_l[kWaves][16];

  const int per_seq = a.Hkv * (a.G / a.heads_per_wg);  // streams per sequence
  const bool by_length = a.B <= 64;
  SeqOrder o{};
  int64_t total;
  if (by_length) {
    o = length_order(a, per_seq);
    total = o.total;
  } else {
    total = total_tiles(a, per_seq);
  }
  run_pieces<D>(a, lds, mrg_m, mrg_l, (int64_t)blockIdx.x, run_tiles(total, a.balanced_wgs),
                total, per_seq, by_length, o);
}

// Length-balanced pass, one run per wave (runs_per_wave).
template <int D>
__global__ __launch_bounds__(kThreads, 2) void attend_balanced_waves(PartialLaunch a) {
  using Gm = Geometry<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kWaves * (Gm::VTILE + kPieceBufBytes)];

  const int per_seq = a.Hkv * (a.G / a.heads_per_wg);  // streams per sequence
  const bool by_length = a.B <= 64;
  SeqOrder o{};
  int64_t total;
  if (by_length) {
    o = length_order(a, per_seq);
    total = o.total;
  } else {
    total = total_tiles(a, per_seq);
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t runs = (int64_t)a.balanced_wgs * kWaves;
  wave_stream<D>(a, lds + wave * Gm::VTILE, lds + kWaves * Gm::VTILE + wave * kPieceBufBytes,
                 (int64_t)blockIdx.x * kWaves + wave, run_tiles(total, runs), total, per_seq,
                 by_length, o);
}

// Merge of the partials of one stream (b, kv head, head tile) cut by the
// balanced schedule; one workgroup per stream (16 threads per row: 64, 128 or
// 256 threads), thread t owns row t / 16 of the stream and
// D/16 values. Streams inside one run were finished by attend_balanced and are
// left alone; an empty sequence gets zeros. Partials are merged in run order
// with weights 2^(m - M).
template <int D>
__global__ __launch_bounds__(256) void combine_balanced(PartialLaunch a) {
  constexpr int PER = D / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int GT = a.heads_per_wg;
  const int tiles_h = a.G / GT;
  const int per_seq = a.Hkv * tiles_h;
  const int RT = GT * a.Sq;
  const int b = blockIdx.x / per_seq, r = blockIdx.x % per_seq;
  const int h0 = (r / tiles_h) * a.G + (r % tiles_h) * GT;
  const int hh = tid >> 4, t16 = tid & 15, d0 = t16 * PER;  // row hh of the stream
  uint16_t* out = a.out + (((int64_t)b * a.Hq + h0) * a.Sq + hh) * D + d0;

  // The schedule of attend_balanced: every tile, and the tiles laid before
  // sequence b's streams (shortest first up to 64 sequences, else index order).
  int64_t total, before_b;
  if (a.B <= 64) {
    // the sequences laid before b: shorter ones, and equal ones of lower index
    const int len = lane < a.B ? (int)seq_len(a, lane) : 0;
    const int len_b = __builtin_amdgcn_readlane(len, b);
    const bool earlier = lane < a.B && (len < len_b || (len == len_b && lane < b));
    total = uniform_i64(wave_sum_i64(lane < a.B ? tiles_of(len) : 0)) * per_seq;
    before_b = uniform_i64(wave_sum_i64(earlier ? tiles_of(len) : 0)) * per_seq;
  } else {
    int64_t all = 0, before = 0;
    for (int base = 0; base < a.B; base += kLenGroup) {
      int len[kLenSlots];
      load_lengths(a, base, len);
#pragma unroll
      for (int i = 0; i < kLenSlots; ++i) {
        const int64_t n = tiles_of(len[i]);
        all += n;
        before += base + 64 * i + lane < b ? n : 0;
      }
    }
    total = uniform_i64(wave_sum_i64(all)) * per_seq;
    before_b = uniform_i64(wave_sum_i64(before)) * per_seq;
  }
  const int64_t runs = runs_per_wave(a) ? (int64_t)a.balanced_wgs * kWaves
                                                      : (int64_t)a.balanced_wgs;
  const int64_t per_run = run_tiles(total, runs);
  const int64_t nb = tiles_of(seq_len(a, b));
  if (nb == 0) {
    if (hh < RT) {
      if constexpr (PER == 8)
        *reinterpret_cast<uint4*>(out) = make_uint4(0u, 0u, 0u, 0u);
      else
        *reinterpret_cast<uint2*>(out) = make_uint2(0u, 0u);
    }
    return;
  }
  const int64_t ts = before_b + (int64_t)r * nb;
  const int64_t ws = ts / per_run, we = (ts + nb - 1) / per_run;
  if (ws == we || hh >= RT) return;

  auto slot_of = [&](int64_t w) -> int64_t {
    const int first = (w > ws || ts == w * per_run) ? 0 : 1;
    return (w * 2 + first) * RT + hh;
  };
  // M over the pieces: the 16 threads of a head take every 16th piece.
  float M = kNegInf;
  for (int64_t w = ws + t16; w <= we; w += 16) M = fmaxf(M, a.part_m[slot_of(w)]);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if (M != kNegInf) {
#pragma unroll 4
    for (int64_t w = ws; w <= we; ++w) {
      const int64_t sl = slot_of(w);
      const float mw = a.part_m[sl];
      const float wt = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
      L += a.part_l[sl] * wt;
      const float4* src = reinterpret_cast<const float4*>(a.part_o + sl * D + d0);
#pragma unroll
      for (int e = 0; e < PER / 4; ++e) {
        const float4 o = src[e];
        acc[4 * e] += o.x * wt;
        acc[4 * e + 1] += o.y * wt;
        acc[4 * e + 2] += o.z * wt;
        acc[4 * e + 3] += o.w * wt;
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  uint32_t w4[PER / 2];
#pragma unroll
  for (int e = 0; e < PER / 2; ++e) w4[e] = pack_bf16(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  if constexpr (PER == 8)
    *reinterpret_cast<uint4*>(out) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  else
    *reinterpret_cast<uint2*>(out) = make_uint2(w4[0], w4[1]);
}

// Log-sum-exp merge of the S split partials: one wave per output row, four rows
// per workgroup, lane l owning D/64 output values. With at most kFastSplits
// splits every load (the running maxima, denominators and partial outputs of
// all splits, in NS register slots, the next power of two of S; slots past the
// last split re-read it and get weight 0) is issued before any is used, so the
// merge costs about one memory round trip; more
// splits run the same arithmetic in a loop. M = max_s m_s, weights 2^(m_s - M)
// (exactly 0 for an empty split, whose partial holds zeros), sums in split
// order. With one non-empty split its weight is exactly 1 and every other term
// an exact 0, so the result equals the one-split output bit for bit.
constexpr int kFastSplits = 16;

template <int D, int NS>
__global__ __launch_bounds__(256) void combine_splits(PartialLaunch a) {
  constexpr int PER = D / 64;  // outputs per lane
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves leave
  const int S = a.S;
  const float* pm = a.part_m + row * S;
  const float* pl = a.part_l + row * S;
  const float* po = a.part_o + row * S * D + lane * PER;

  float M = kNegInf, L = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if constexpr (NS > 0) {
    float m[NS], l[NS], o[NS][PER];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = s < S ? s : S - 1;
      m[s] = pm[j];
      l[s] = pl[j];
      if constexpr (PER == 2) {
        const float2 v = *reinterpret_cast<const float2*>(po + (int64_t)j * D);
        o[s][0] = v.x;
        o[s][1] = v.y;
      } else {
        o[s][0] = po[(int64_t)j * D];
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s >= S) m[s] = kNegInf;
      M = fmaxf(M, m[s]);
    }
    if (M != kNegInf) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float w = exp2_fast(m[s] - M);
        L += l[s] * w;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += o[s][e] * w;
      }
    }
  } else {
    for (int j = lane; j < S; j += 64) M = fmaxf(M, pm[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (M != kNegInf) {
#pragma unroll 8
      for (int j = 0; j < S; ++j) {
        const float w = exp2_fast(pm[j] - M);
        L += pl[j] * w;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += po[(int64_t)j * D + e] * w;
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  if constexpr (PER == 2)
    *reinterpret_cast<uint32_t*>(a.out + row * D + lane * 2) = pack_bf16(acc[0] * inv, acc[1] * inv);
  else
    a.out[row * D + lane] = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xffffu);
}

template <int D, bool SPARSE>
hipError_t launch_partial_d(const PartialLaunch& L, hipStream_t stream) {
  const int tiles = L.G / L.heads_per_wg;
  const int64_t grid = (int64_t)L.B * L.Hkv * tiles * L.S;
  if (grid <= 0 || grid > 0x7fffffff || L.heads_per_wg < 1 || L.heads_per_wg * L.Sq > 16 ||
      (SPARSE && L.Sq != 1))
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attend_partial<D, SPARSE>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     L);
  return hipGetLastError();
}

template <int D>
hipError_t launch_balanced_d(const PartialLaunch& L, hipStream_t stream) {
  if (runs_per_wave(L))
    hipLaunchKernelGGL(attend_balanced_waves<D>, dim3((unsigned)L.balanced_wgs), dim3(kThreads),
                       0, stream, L);
  else
    hipLaunchKernelGGL(attend_balanced<D>, dim3((unsigned)L.balanced_wgs), dim3(kThreads), 0,
                       stream, L);
  return hipGetLastError();
}

template <int D>
hipError_t launch_balanced_combine_d(const PartialLaunch& L, hipStream_t stream) {
  const int64_t streams = (int64_t)L.B * L.Hkv * (L.G / L.heads_per_wg);
  // 16 threads per row of the stream, whole waves: 64 threads for up to 4 rows
  const int rows = L.heads_per_wg * L.Sq;
  const int threads = rows <= 4 ? 64 : (rows <= 8 ? 128 : 256);
  hipLaunchKernelGGL(combine_balanced<D>, dim3((unsigned)streams), dim3(threads), 0, stream, L);
  return hipGetLastError();
}

bool balanced_ok(const PartialLaunch& L) {
  const int64_t streams = (int64_t)L.B * L.Hkv * (L.G / L.heads_per_wg);
  return !L.sparse && L.k_len_dev && L.balanced_wgs > 0 && L.heads_per_wg >= 1 && L.Sq >= 1 &&
         L.heads_per_wg * L.Sq <= 16 && streams > 0 && streams <= 0x7fffffff && L.part_o && L.part_m &&
         L.part_l;
}

}  // namespace

hipError_t launch_balanced(const PartialLaunch& L, hipStream_t stream) {
  if (!balanced_ok(L)) return hipErrorInvalidConfiguration;
  if (L.D == 128) return launch_balanced_d<128>(L, stream);
  if (L.D == 64) return launch_balanced_d<64>(L, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_balanced_combine(const PartialLaunch& L, hipStream_t stream) {
  if (!balanced_ok(L)) return hipErrorInvalidConfiguration;
  if (L.D == 128) return launch_balanced_combine_d<128>(L, stream);
  if (L.D == 64) return launch_balanced_combine_d<64>(L, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_partial(const PartialLaunch& L, hipStream_t stream) {
  if (L.D == 128) return L.sparse ? launch_partial_d<128, true>(L, stream)
                                  : launch_partial_d<128, false>(L, stream);
  if (L.D == 64) return L.sparse ? launch_partial_d<64, true>(L, stream)
                                 : launch_partial_d<64, false>(L, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const PartialLaunch& L, hipStream_t stream) {
  const int64_t rows = (int64_t)L.B * L.Hq * L.Sq;
  if (rows <= 0 || rows > 0x7fffffff || L.S < 1) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)((rows + 3) / 4);  // one wave per row
  // The register-resident merge is sized to the next power of two of the split
  // count (up to kFastSplits); more splits take the looped merge.
  const int ns = L.S <= 2 ? 2 : (L.S <= 4 ? 4 : (L.S <= 8 ? 8 : (L.S <= kFastSplits ? 16 : 0)));
#define DA_COMBINE(DD, NN) \
  hipLaunchKernelGGL((combine_splits<DD, NN>), dim3(grid), dim3(256), 0, stream, L)
  if (L.D != 128 && L.D != 64) return hipErrorInvalidValue;
  if (L.D == 128) {
    if (ns == 2) DA_COMBINE(128, 2);
    else if (ns == 4) DA_COMBINE(128, 4);
    else if (ns == 8) DA_COMBINE(128, 8);
    else if (ns == 16) DA_COMBINE(128, 16);
    else DA_COMBINE(128, 0);
  } else {
    if (ns == 2) DA_COMBINE(64, 2);
    else if (ns == 4) DA_COMBINE(64, 4);
    else if (ns == 8) DA_COMBINE(64, 8);
    else if (ns == 16) DA_COMBINE(64, 16);
    else DA_COMBINE(64, 0);
  }
#undef DA_COMBINE
  return hipGetLastError();
}

}  // namespace da
