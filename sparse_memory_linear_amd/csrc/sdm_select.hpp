// Wave-level product-key selection shared by the addressing and decode kernels.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Product Key Memory"; atlas.scime.ai
// summary, "Approach"): the best kappa sub-keys of each half are kept, and the best n_sel of
// the kappa x kappa sums are the token's slots. Every ranking orders by float32 score
// descending, then by index ascending.
#pragma once

#include "sdm_device.hpp"

namespace sdm {

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

// The value of lane (lane ^ m) for the partners a descending bitonic sort of the wave uses:
// m = 2^i (the steps inside a stage) and m = 2^i - 1 (the mirror that opens stage 2^i), with
// DPP, ds_swizzle and v_permlane32_swap. `m` must fold to a constant.
__device__ __forceinline__ uint32_t xchg_u32(uint32_t v, int m) {
  switch (m) {
    case 3: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, false);    // quad_perm [3,2,1,0]
    case 7: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);   // row_half_mirror
    case 15: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);  // row_mirror
    case 31: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x7C1F);              // xor 31 in 32 lanes
    case 63: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)shfl_xor_u32(v, 32), 0x7C1F);
    default: return shfl_xor_u32(v, m);
  }
}
__device__ __forceinline__ uint64_t xchg_u64(uint64_t v, int m) {
  return ((uint64_t)xchg_u32((uint32_t)(v >> 32), m) << 32) | xchg_u32((uint32_t)v, m);
}
__device__ __forceinline__ float xchg_f32(float v, int m) { return __uint_as_float(xchg_u32(__float_as_uint(v), m)); }

// Bitonic sort of one value per lane across the wave, descending (lane 0 = largest). Stage k
// (k = 2, 4, ..., 64) opens by comparing each lane with its mirror in its block of k lanes
// (lane ^ (k - 1)), which merges the two sorted halves of the block into two bitonic halves,
// every value of the lower above every value of the upper; steps j = k/4 .. 1 (lane ^ j)
// then sort those halves. Every block is sorted in the same direction, so at each step the
// lower lane of a pair keeps the larger value: the lane pattern depends on one lane bit (six
// patterns in all, where a direction that alternates between blocks needs 21). Equal values
// are interchangeable. `step` performs one compare-exchange with partner lane ^ m, the lower
// lane being the one whose bit `bit` is clear.
template <typename Step>
__device__ __forceinline__ void bitonic_desc(Step step) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
    step(k - 1, k >> 1);
#pragma unroll
    for (int j = k >> 2; j > 0; j >>= 1) step(j, j);
  }
}
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t key) {
  const int lane = lane_id();
  bitonic_desc([&](int m, int bit) {
    const uint64_t other = xchg_u64(key, m);
    const bool lower = (lane & bit) == 0;
    key = ((key > other) == lower) ? key : other;
  });
  return key;
}
// Scores only: used for thresholds.
__device__ __forceinline__ float wave_sort_desc_f32(float s) {
  const int lane = lane_id();
  bitonic_desc([&](int m, int bit) {
    const float other = xchg_f32(s, m);
    const bool lower = (lane & bit) == 0;
    s = ((s > other) == lower) ? s : other;
  });
  return s;
}
// The same sort moving a 32-bit payload with each score. Equal scores are left in no
// particular order, and two equal scores that meet may leave with the same payload: the
// caller checks the sorted scores for equal neighbours before it trusts the payloads.
__device__ __forceinline__ void wave_sort_desc_f32_payload(float& s, uint32_t& p) {
  const int lane = lane_id();
  bitonic_desc([&](int m, int bit) {
    const float os = xchg_f32(s, m);
    const uint32_t op = xchg_u32(p, m);
    const bool keep = (s > os) == ((lane & bit) == 0);
    s = keep ? s : os;
    p = keep ? p : op;
  });
}

// Two independent sorts in one pass: each step exchanges and compares both, so one chain's
// dependent instructions fill the other's latency.
__device__ __forceinline__ void wave_sort_desc_f32x2(float& a, float& b) {
  const int lane = lane_id();
  bitonic_desc([&](int m, int bit) {
    const float oa = xchg_f32(a, m), ob = xchg_f32(b, m);
    const bool lower = (lane & bit) == 0;
    a = ((a > oa) == lower) ? a : oa;
    b = ((b > ob) == lower) ? b : ob;
  });
}
__device__ __forceinline__ void wave_sort_desc_f32_payload2(float& s0, uint32_t& p0, float& s1, uint32_t& p1) {
  const int lane = lane_id();
  bitonic_desc([&](int m, int bit) {
    const float o0 = xchg_f32(s0, m), o1 = xchg_f32(s1, m);
    const uint32_t q0 = xchg_u32(p0, m), q1 = xchg_u32(p1, m);
    const bool lower = (lane & bit) == 0;
    const bool k0 = (s0 > o0) == lower, k1 = (s1 > o1) == lower;
    s0 = k0 ? s0 : o0;
    p0 = k0 ? p0 : q0;
    s1 = k1 ? s1 : o1;
    p1 = k1 ? p1 : q1;
  });
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
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


// Two independent top-`count` selections (as wave_topk_f32) in one wave, their threshold
// sorts, compactions and candidate sorts interleaved. Results equal two calls of
// wave_topk_f32; a selection whose candidates do not fit the fast path is redone by it.
// bufa and bufb are 64 words of LDS each, private to the calling wave.
template <int E>
__device__ __forceinline__ void wave_topk_f32_x2(const float (&sa)[E], const uint32_t (&ia)[E], const float (&sb)[E],
                                                 const uint32_t (&ib)[E], int count, uint64_t* bufa, uint64_t* bufb,
                                                 float* oa_s, uint32_t* oa_i, float* ob_s, uint32_t* ob_i) {
  const int lane = lane_id();
  const uint64_t none = (0xFFFFFFFFull << 32) | (uint64_t)__float_as_uint(-INFINITY);
  uint64_t ma, mb;  // this lane's candidate of each selection, (index << 32) | score bits
  int na, nb;       // candidates of each selection
  if constexpr (E == 1) {
    ma = sa[0] > -INFINITY ? ((uint64_t)ia[0] << 32) | __float_as_uint(sa[0]) : none;
    mb = sb[0] > -INFINITY ? ((uint64_t)ib[0] << 32) | __float_as_uint(sb[0]) : none;
    na = nb = kWave;
  } else {
    float xa = sa[0], xb = sb[0];
#pragma unroll
    for (int e = 1; e < E; ++e) {
      xa = fmaxf(xa, sa[e]);
      xb = fmaxf(xb, sb[e]);
    }
    wave_sort_desc_f32x2(xa, xb);
    const float ta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xa), count - 1));
    const float tb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xb), count - 1));
    // compaction, optimistic: positions past 64 are not written, and such a selection is
    // redone below
    na = nb = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ca = sa[e] >= ta, cb = sb[e] >= tb;
      const uint64_t ka = ballot(ca), kb = ballot(cb);
      const int qa = na + mbcnt(ka), qb = nb + mbcnt(kb);
      if (ca && qa < kWave) bufa[qa] = ((uint64_t)ia[e] << 32) | (uint64_t)__float_as_uint(sa[e]);
      if (cb && qb < kWave) bufb[qb] = ((uint64_t)ib[e] << 32) | (uint64_t)__float_as_uint(sb[e]);
      na += popc64(ka);
      nb += popc64(kb);
    }
    if (!(ta > -INFINITY && na <= kWave && tb > -INFINITY && nb <= kWave)) {
      wave_topk_f32<E>(sa, ia, count, bufa, oa_s, oa_i);
      wave_topk_f32<E>(sb, ib, count, bufb, ob_s, ob_i);
      return;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    ma = lane < na ? bufa[lane] : none;
    mb = lane < nb ? bufb[lane] : none;
    __builtin_amdgcn_wave_barrier();
  }
  float s0 = __uint_as_float((uint32_t)ma), s1 = __uint_as_float((uint32_t)mb);
  uint32_t p0 = (uint32_t)(ma >> 32), p1 = (uint32_t)(mb >> 32);
  wave_sort_desc_f32_payload2(s0, p0, s1, p1);
  const float n0 = __shfl_down(s0, 1, kWave), n1 = __shfl_down(s1, 1, kWave);
  const bool ok = lane < count && lane < kWave - 1;
  *oa_s = s0;
  *oa_i = p0;
  *ob_s = s1;
  *ob_i = p1;
  // equal neighbours up to rank `count`: that selection's order is redone on exact keys
  if (ballot(ok && s0 == n0)) {
    const uint64_t key = wave_sort_desc_u64(ma != none ? rank_key(__uint_as_float((uint32_t)ma), (uint32_t)(ma >> 32)) : 0ull);
    *oa_s = key_score(key);
    *oa_i = key_index(key);
  }
  if (ballot(ok && s1 == n1)) {
    const uint64_t key = wave_sort_desc_u64(mb != none ? rank_key(__uint_as_float((uint32_t)mb), (uint32_t)(mb >> 32)) : 0ull);
    *ob_s = key_score(key);
    *ob_i = key_index(key);
  }
}

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

// Two token-halves in one wave (as two select_half calls), their selections interleaved.
template <int E>
__device__ __forceinline__ void select_half_x2(const float* rowa, int swza, const float* rowb, int swzb, int s, int kappa,
                                               uint64_t* bufa, uint64_t* bufb, int16_t* oia, float* osa, int16_t* oib,
                                               float* osb) {
  const int lane = lane_id();
  const float* ra = rowa + (lane ^ swza);
  const float* rb = rowb + (lane ^ swzb);
  float sa[E], sb[E];
  uint32_t ix[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + kWave * e;
    sa[e] = i < s ? ra[kWave * e] : -INFINITY;
    sb[e] = i < s ? rb[kWave * e] : -INFINITY;
    ix[e] = (uint32_t)i;
  }
  float ta, tb;
  uint32_t ja, jb;
  wave_topk_f32_x2<E>(sa, ix, sb, ix, kappa, bufa, bufb, &ta, &ja, &tb, &jb);
  if (lane < kappa) {
    oia[lane] = (int16_t)ja;
    osa[lane] = ta;
    oib[lane] = (int16_t)jb;
    osb[lane] = tb;
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

// Exact top n_sel of all kappa^2 pairs, extracted largest first: lanes < n_sel get their key.
__device__ __forceinline__ uint64_t merge_exact(const int16_t* i1, const float* s1, const int16_t* i2, const float* s2,
                                                int s, int kappa, int n_sel) {
  const int lane = lane_id();
  const int all = kappa * kappa;
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
  if (ballot(viol) == 0ull) return top;
  return merge_exact(i1, s1, i2, s2, s, kappa, n_sel);
}

// Two tokens' merges in one wave (as two merge_token calls), their selections interleaved.
template <int EM>
__device__ __forceinline__ void merge_token_x2(const int16_t* i1a, const float* s1a, const int16_t* i2a,
                                               const float* s2a, const int16_t* i1b, const float* s1b,
                                               const int16_t* i2b, const float* s2b, int s, int kappa, int n_sel,
                                               const int (&pr)[EM], int bdiv, uint64_t* bufa, uint64_t* bufb,
                                               uint64_t* ka, uint64_t* kb) {
  const int lane = lane_id();
  float sa[EM], sb[EM];
  uint32_t xa[EM], xb[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int a = pr[e] >> 8, b = pr[e] & 255;
    sa[e] = pr[e] >= 0 ? s1a[a] + s2a[b] : -INFINITY;
    sb[e] = pr[e] >= 0 ? s1b[a] + s2b[b] : -INFINITY;
    xa[e] = pr[e] >= 0 ? (uint32_t)i1a[a] * (uint32_t)s + (uint32_t)i2a[b] : 0xFFFFFFFFu;
    xb[e] = pr[e] >= 0 ? (uint32_t)i1b[a] * (uint32_t)s + (uint32_t)i2b[b] : 0xFFFFFFFFu;
  }
  float ta, tb;
  uint32_t ja, jb;
  wave_topk_f32_x2<EM>(sa, xa, sb, xb, n_sel, bufa, bufb, &ta, &ja, &tb, &jb);
  *ka = lane < n_sel ? rank_key(ta, ja) : 0ull;
  *kb = lane < n_sel ? rank_key(tb, jb) : 0ull;
  const float tua = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ta), n_sel - 1));
  const float tub = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tb), n_sel - 1));
  const bool row = lane < kappa && bdiv < kappa;
  if (ballot(row && s1a[lane] + s2a[bdiv] >= tua)) *ka = merge_exact(i1a, s1a, i2a, s2a, s, kappa, n_sel);
  if (ballot(row && s1b[lane] + s2b[bdiv] >= tub)) *kb = merge_exact(i1b, s1b, i2b, s2b, s, kappa, n_sel);
}

}  // namespace sdm
