// Device helpers shared by the SDM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16 / float32 values
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two float32 values -> two bfloat16 in one word (lo in bits 15:0), rounded to nearest even
// by gfx950's packed conversion instruction (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ------------------------------------------------------------------ wave primitives
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Exchange with lane ^ mask, for mask a power of two up to 32, without going through LDS
// addressing: DPP for masks 1, 2, 4 (half-row mirror then quad reversal), 8 (row rotate),
// ds_swizzle for 16, v_permlane32_swap for 32. `mask` must fold to a constant.
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  switch (mask) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    case 4: return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false), 0x1B,
                                                      0xF, 0xF, false);                // half mirror, quad reverse
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
    case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);              // swap 16
    case 32: {
      auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return __lane_id() < 32 ? r[1] : r[0];
    }
    default: return (uint32_t)__shfl_xor((int)v, mask, kWave);
  }
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = shfl_xor_u32((uint32_t)v, mask);
  uint32_t hi = shfl_xor_u32((uint32_t)(v >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
  return __uint_as_float(shfl_xor_u32(__float_as_uint(v), mask));
}

// v + (v of lane ^ mask), for mask a power of two up to 32 (fold to a constant). Within a
// row of 16 lanes the partner's value reaches the add through its DPP operand (one fused
// v_add_f32_dpp; every partner lies inside the row, so the zero that bound_ctrl gives an
// invalid source never occurs); mask 4 takes a half-row mirror first. The sum equals
// v + shfl_xor_f32(v, mask) bit for bit.
__device__ __forceinline__ float add_xor_f32(float v, int mask) {
  const int x = __float_as_int(v);
  switch (mask) {
    case 1: return v + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
    case 2: return v + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
    case 4: {
      const int t = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);                            // half mirror
      return v + __int_as_float(__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, true));         // quad reverse
    }
    case 8: return v + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true));  // row_ror:8
    default: return v + shfl_xor_f32(v, mask);
  }
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = add_xor_f32(v, m);
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }
// number of set bits of m in lanes below this lane
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

}  // namespace sdm
