// device_common.h -- small gfx950 device helpers shared by the decode-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// 2^x on the transcendental unit (v_exp_f32): exp2(-inf) = 0, exp2(0) = 1 exactly.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_inff();

}  // namespace da
