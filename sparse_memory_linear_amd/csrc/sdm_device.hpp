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

// ------------------------------------------------------------------ ordered keys
// Maps float32 to uint32 so that unsigned comparison follows the float order.
__device__ __forceinline__ uint32_t ordered_u32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_u32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
// 64-bit rank key: larger key = earlier rank. Orders by score descending, then index
// ascending (the complement of the index in the low word). Key 0 marks "no element".
__device__ __forceinline__ uint64_t rank_key(float score, uint32_t index) {
  return ((uint64_t)ordered_u32(score) << 32) | (uint64_t)(~index);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~(uint32_t)k; }
__device__ __forceinline__ float key_score(uint64_t k) { return from_ordered_u32((uint32_t)(k >> 32)); }

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

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f32(v, m);
  return v;
}

// Bitonic sort of one key per lane across the wave, descending (lane 0 = largest). At each
// step a lane keeps the larger of its key and its partner's when it is the lower lane of a
// descending block or the upper lane of an ascending one, else the smaller: one compare,
// folded with that lane pattern, and one select per word. Equal keys are interchangeable.
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t key) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t other = shfl_xor_u64(key, j);
      const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
      key = ((key > other) == take_max) ? key : other;
    }
  }
  return key;
}
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t key) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t other = shfl_xor_u32(key, j);
      const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
      key = ((key > other) == take_max) ? key : other;
    }
  }
  return key;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }
// number of set bits of m in lanes below this lane
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Exact top-`count` (count <= 64) of E keys per lane (E*64 candidates; key 0 = empty),
// returned one per lane in rank order: lane i < count holds the i-th largest key, lanes
// >= count hold 0. `buf` is 64 words of LDS private to the calling wave.
//
// Fast path: the count-th largest lane maximum (score word only) is a lower bound of the
// count-th largest key; if at most 64 keys reach it they are compacted and sorted.
// Otherwise the keys are extracted one by one (exact, slower).
template <int E>
__device__ uint64_t wave_topk(const uint64_t (&keys)[E], int count, uint64_t* buf) {
  const int lane = lane_id();
  uint32_t lmax = (uint32_t)(keys[0] >> 32);  // score words only
#pragma unroll
  for (int e = 1; e < E; ++e) lmax = max(lmax, (uint32_t)(keys[e] >> 32));
  uint32_t sorted_hi = wave_sort_desc_u32(lmax);
  uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)sorted_hi, count - 1);
  uint64_t masks[E];
  int total = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bool p = keys[e] != 0 && (uint32_t)(keys[e] >> 32) >= tau;
    masks[e] = ballot(p);
    total += popc64(masks[e]);
  }
  if (total <= kWave) {
    int base = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((masks[e] >> lane) & 1ull) buf[base + mbcnt(masks[e])] = keys[e];
      base += popc64(masks[e]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    uint64_t mine = lane < total ? buf[lane] : 0ull;
    __builtin_amdgcn_wave_barrier();
    uint64_t s = wave_sort_desc_u64(mine);
    return lane < count ? s : 0ull;
  }
  // exact slow path: repeated wave-wide maximum extraction
  uint64_t work[E];
#pragma unroll
  for (int e = 0; e < E; ++e) work[e] = keys[e];
  uint64_t out = 0;
  for (int i = 0; i < count; ++i) {
    uint64_t m = work[0];
#pragma unroll
    for (int e = 1; e < E; ++e) m = work[e] > m ? work[e] : m;
    uint64_t g = wave_max_u64(m);
    if (lane == i) out = g;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (work[e] == g) work[e] = 0;  // keys are unique (index in the low word)
  }
  return out;
}

}  // namespace sdm
