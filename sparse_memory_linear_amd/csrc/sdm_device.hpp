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

// Bitonic sort of one float per lane, descending (scores only: used for thresholds).
__device__ __forceinline__ float wave_sort_desc_f32(float s) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float other = shfl_xor_f32(s, j);
      const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
      s = ((s > other) == take_max) ? s : other;
    }
  }
  return s;
}
// The same sort moving a 32-bit payload with each score. Equal scores are left in no
// particular order, and two equal scores that meet may leave with the same payload: the
// caller checks the sorted scores for equal neighbours before it trusts the payloads.
__device__ __forceinline__ void wave_sort_desc_f32_payload(float& s, uint32_t& p) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float os = shfl_xor_f32(s, j);
      const uint32_t op = shfl_xor_u32(p, j);
      const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
      const bool keep = (s > os) == take_max;
      s = keep ? s : os;
      p = keep ? p : op;
    }
  }
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

// Exact top-`count` (count <= 64) of E (score, index) pairs per lane, ranked by score
// descending, then index ascending; a score of -inf marks an absent entry, and at least
// `count` lanes must hold a finite score. Lane i < count receives the pair of rank i.
// `buf` is 64 words of LDS private to the calling wave.
//
// The count-th largest lane maximum tau bounds the answer from below: every pair of the
// top `count` scores at least tau (otherwise `count` lane maxima would beat it), so the
// pairs scoring >= tau hold the answer. When at most 64 do, they are compacted and sorted
// on their float scores alone, each carrying its index; if two sorted neighbours up to
// rank `count` score equal, their index order is not known and the candidates are sorted
// again on exact 64-bit keys (score, complemented index). More than 64 candidates take the
// exact extraction, one rank at a time. Only the candidates ever get a 64-bit key. With one
// entry per lane the lanes are sorted directly, with the same tie check.
template <int E>
__device__ __forceinline__ void wave_topk_f32(const float (&sc)[E], const uint32_t (&ix)[E], int count, uint64_t* buf,
                              float* out_s, uint32_t* out_i) {
  const int lane = lane_id();
  if constexpr (E == 1) {
    // one entry per lane: no threshold and no compaction, the lanes themselves are sorted
    float s = sc[0];
    uint32_t p = ix[0];
    wave_sort_desc_f32_payload(s, p);
    const float next = __shfl_down(s, 1, kWave);
    if (ballot(lane < count && lane < kWave - 1 && s == next) == 0ull) {
      *out_s = s;
      *out_i = p;
      return;
    }
    const uint64_t key = wave_sort_desc_u64(sc[0] > -INFINITY ? rank_key(sc[0], ix[0]) : 0ull);
    *out_s = key_score(key);
    *out_i = key_index(key);
    return;
  }
  float lmax = sc[0];
#pragma unroll
  for (int e = 1; e < E; ++e) lmax = fmaxf(lmax, sc[e]);
  const float tau = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sort_desc_f32(lmax)), count - 1));
  uint64_t masks[E];
  int total = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    masks[e] = ballot(sc[e] >= tau);
    total += popc64(masks[e]);
  }
  if (tau > -INFINITY && total <= kWave) {
    int base = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (sc[e] >= tau) buf[base + mbcnt(masks[e])] = ((uint64_t)ix[e] << 32) | (uint64_t)__float_as_uint(sc[e]);
      base += popc64(masks[e]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const uint64_t mine = lane < total ? buf[lane] : (0xFFFFFFFFull << 32) | (uint64_t)__float_as_uint(-INFINITY);
    __builtin_amdgcn_wave_barrier();
    float s = __uint_as_float((uint32_t)mine);
    uint32_t p = (uint32_t)(mine >> 32);
    wave_sort_desc_f32_payload(s, p);
    const float next = __shfl_down(s, 1, kWave);
    if (ballot(lane < count && lane < kWave - 1 && s == next) == 0ull) {
      *out_s = s;
      *out_i = p;
      return;
    }
    const uint64_t key = wave_sort_desc_u64(lane < total ? rank_key(__uint_as_float((uint32_t)mine), (uint32_t)(mine >> 32)) : 0ull);
    *out_s = key_score(key);
    *out_i = key_index(key);
    return;
  }
  // exact slow path: repeated wave-wide maximum extraction on 64-bit keys
  uint64_t work[E];
#pragma unroll
  for (int e = 0; e < E; ++e) work[e] = sc[e] > -INFINITY ? rank_key(sc[e], ix[e]) : 0ull;
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
  *out_s = key_score(out);
  *out_i = key_index(out);
}

}  // namespace sdm
