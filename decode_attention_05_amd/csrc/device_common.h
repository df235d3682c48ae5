// device_common.h -- small gfx950 device helpers shared by the decode-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// bfloat16 is the top half of an IEEE binary32, so widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& r, float (&f)[8]) {
  f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
  f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
  f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
  f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
}

// binary32 -> bfloat16 with IEEE round-to-nearest-even; NaN becomes the quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// 2^x on the transcendental unit (v_exp_f32): exp2(-inf) = 0, exp2(0) = 1 exactly.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside a row of 16 lanes. Each one pairs lane i with lane
// i ^ mask, so a butterfly over a basis of masks leaves the same sum in every lane.
enum : int {
  DPP_XOR1 = 0xB1,   // quad_perm [1,0,3,2]
  DPP_XOR2 = 0x4E,   // quad_perm [2,3,0,1]
  DPP_XOR7 = 0x141,  // row_half_mirror: i -> 7 - i inside 8 lanes
  DPP_XOR15 = 0x140, // row_mirror:      i -> 15 - i inside 16 lanes
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the LANES consecutive lanes (8 or 16) that share one KV row; every lane
// of the group ends with the identical value.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 8 || LANES == 16, "row groups are 8 or 16 lanes");
  if constexpr (LANES == 16) x += dpp_f32<DPP_XOR15>(x);
  x += dpp_f32<DPP_XOR7>(x);
  x += dpp_f32<DPP_XOR2>(x);
  x += dpp_f32<DPP_XOR1>(x);
  return x;
}

constexpr float kNegInf = -__builtin_inff();

}  // namespace da
