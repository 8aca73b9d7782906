// Wave-level product-key selection shared by the addressing and decode kernels.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Product Key Memory"; atlas.scime.ai
// summary, "Approach"): the best kappa sub-keys of each half are kept, and the best n_sel of
// the kappa x kappa sums are the token's slots. Every ranking orders by float32 score
// descending, then by index ascending.
#pragma once

#include "sdm_device.hpp"

namespace sdm {

// ---------------------------------------------------------------- per-half selection
// Top-kappa sub-keys of one token-half: lanes < kappa receive (index, score) in rank order.
// Score i of the row sits at row[i ^ swz] (swz < 32 permutes within aligned groups of 32).
template <int E>
__device__ __forceinline__ void select_half(const float* row, int swz, int s, int kappa, uint64_t* wbuf, int16_t* out_idx,
                            float* out_sc) {
  const int lane = lane_id();
  // i ^ swz = (lane ^ swz) + 64 e for i = lane + 64 e, since swz < 32
  const float* rp = row + (lane ^ swz);
  float sc[E];
  uint32_t ix[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + kWave * e;
    sc[e] = i < s ? rp[kWave * e] : -INFINITY;
    ix[e] = (uint32_t)i;
  }
  float ts;
  uint32_t ti;
  wave_topk_f32<E>(sc, ix, kappa, wbuf, &ts, &ti);
  if (lane < kappa) {
    out_idx[lane] = (int16_t)ti;
    out_sc[lane] = ts;
  }
}

// ---------------------------------------------------------------- merge
// Rank pairs (a, b) of the staircase {(a, b): (a+1)(b+1) <= n_sel, a, b < kappa}, enumerated
// row by row: this lane's pairs p = lane + 64 e, packed a << 8 | b, or -1 past the end.
// *bdiv receives n_sel / (lane + 1) (the first rank b past row `lane`), which merge_token
// takes. Depends only on (kappa, n_sel): computed once per wave, outside the token loop.
template <int EM>
__device__ __forceinline__ void stair_pairs(int kappa, int n_sel, int (&pr)[EM], int* bdiv) {
  const int lane = lane_id();
#pragma unroll
  for (int e = 0; e < EM; ++e) pr[e] = -1;
  // row a's length min(kappa, n_sel / (a + 1)) is computed on lane a (one division for the
  // whole wave) and read back row by row
  const int q = n_sel / (lane + 1);
  *bdiv = q;
  int rowlen = 0;
  if (lane < kappa) rowlen = q < kappa ? q : kappa;
  int base = 0;
  for (int a = 0; a < kappa; ++a) {
    const int cnt = __builtin_amdgcn_readlane(rowlen, a);
    if (cnt <= 0) break;
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      const int p = lane + kWave * e;
      if (p >= base && p < base + cnt) pr[e] = (a << 8) | (p - base);
    }
    base += cnt;
  }
}

__device__ __forceinline__ uint64_t cand_key(const int16_t* i1, const float* s1, const int16_t* i2, const float* s2,
                                             int a, int b, int s) {
  float sc = s1[a] + s2[b];
  uint32_t slot = (uint32_t)i1[a] * (uint32_t)s + (uint32_t)i2[b];
  return rank_key(sc, slot);
}

// Top n_sel of the kappa x kappa candidates for one token: lanes < n_sel get their key.
template <int EM>
__device__ __forceinline__ uint64_t merge_token(const int16_t* i1, const float* s1, const int16_t* i2, const float* s2, int s,
                                int kappa, int n_sel, const int (&pr)[EM], int bdiv, uint64_t* wbuf) {
  const int lane = lane_id();
  // 1. exact top n_sel of the staircase pairs (every pair outside it is dominated by at
  //    least n_sel pairs inside it up to float32 rounding ties, which step 2 catches)
  float sc[EM];
  uint32_t ix[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int a = pr[e] >> 8, b = pr[e] & 255;
    sc[e] = pr[e] >= 0 ? s1[a] + s2[b] : -INFINITY;
    ix[e] = pr[e] >= 0 ? (uint32_t)i1[a] * (uint32_t)s + (uint32_t)i2[b] : 0xFFFFFFFFu;
  }
  float ts;
  uint32_t ti;
  wave_topk_f32<EM>(sc, ix, n_sel, wbuf, &ts, &ti);
  const uint64_t top = lane < n_sel ? rank_key(ts, ti) : 0ull;
  // 2. a pair (a, b) outside the staircase has b >= n_sel/(a+1), so its score is at most that
  //    of the boundary pair (a, n_sel/(a+1)) of its row. If no boundary pair reaches the
  //    n_sel-th score, nothing outside the staircase can rank above it (a float32 rounding
  //    tie would need an equal score); otherwise fall back to the exact extraction.
  const float tau_score = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ts), n_sel - 1));
  bool viol = false;
  if (lane < kappa && bdiv < kappa && s1[lane] + s2[bdiv] >= tau_score) viol = true;
  const int all = kappa * kappa;
  if (ballot(viol) == 0ull) return top;
  // 3. exact extraction over all kappa^2 pairs, largest first
  uint64_t out = 0ull, prev = ~0ull;
  for (int i = 0; i < n_sel; ++i) {
    uint64_t m = 0ull;
    for (int p = lane; p < all; p += kWave) {
      uint64_t k = cand_key(i1, s1, i2, s2, p / kappa, p % kappa, s);
      if (k < prev && k > m) m = k;
    }
    uint64_t g = wave_max_u64(m);
    if (lane == i) out = g;
    prev = g;
  }
  return out;
}

}  // namespace sdm
