// Chunkwise two-phase form of the sparse gated-delta recurrence (written-rows rule).
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, App. A.1 "Phase 1" / "Phase 2" and
// App. A.2's sparse inner products between tokens' slot lists): inside a chunk of C tokens
// a row changes only at the tokens that write it, so every quantity is the chunk-start
// table plus a combination of the chunk's write residuals delta_t = beta_t (v_t - rho_t).
// With dec(n; tau, t) the product of alpha over the chunk's writers of slot n strictly
// between tokens tau and t:
//   K[t][tau] = alpha_t sum_{j: n_tj written by tau} a_tj dec(n_tj; tau, t) a_{tau,n_tj}
//   Q[t][tau] = sum_{r: m_tr written by tau <= t} u_tr dec(m_tr; tau, t+1) a_{tau,m_tr}
//   P[t] = alpha_t sum_j a_tj dec(n_tj; start, t) M0[n_tj];   O0[t] = sum_r u_tr dec(m_tr; start, t+1) M0[m_tr]
//   (I + diag(beta) K) delta = diag(beta) (V - P);   o = O0 + Q delta
//   M[n] = dec(n; start, end) M0[n] + sum_{writers tau of n} dec(n; tau, end) a_{tau,n} delta_tau
//
// With W of N slots per token, K and Q are almost empty (two tokens couple only through a
// shared slot), so both are kept as sparse lists sorted by row and the unit lower-triangular
// system is solved by a forward sweep over the nonzeros only.
//
// Phase 1 (chunk_prep_kernel, one workgroup per (unit, chunk), every chunk in parallel): the
// chunk's write occurrences go into an LDS hash of per-slot linked lists and a bit filter;
// each write and read occurrence walks its slot's list for its couplings (accumulated
// densely in LDS, with a bit mask per row of the pairs that occur), its decay coefficient
// and its write-back terms (a read whose slot the filter rules out, or a slot's only
// writer, takes a short path). The product over a slot's writers between two tokens is a
// product over a set, so the list order does not matter. The couplings then leave as
// row-sorted lists.
//
// Phase 2 (chunk_apply_kernel, one workgroup per (unit, block of row dwords), the chunks of
// a unit in order): the lanes of a token split its occurrences into groups and the block
// into quads, so that each lane gathers a few whole row pieces at once and the lanes of one
// occurrence read contiguous bytes; P and O0 are summed across the groups; delta starts as
// beta (V - P) in LDS, the chunk's lists are staged in LDS and a few lanes sweep K's rows;
// then o = O0 + Q delta and the last writer of each slot writes its piece back once,
// rounded to the table dtype there.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kC = 64;                   // tokens per chunk
constexpr int kMaxList = 32;             // W, R <= 32 on this path
constexpr int kBuckets = 4096;           // LDS hash: at most 2048 distinct slots, at most half full
constexpr uint32_t kFree = 0xFFFFFFFFu;
constexpr int kFilterWords = 512;        // 16K-bit filter of the chunk's written slots
constexpr int kKMax = kC * (kC - 1) / 2;  // distinct (t, tau < t) pairs
constexpr int kQMax = kC * (kC + 1) / 2;  // distinct (t, tau <= t) pairs
constexpr int kXcd = 8;                  // workgroups are dealt round-robin to this many L2 domains
constexpr uint32_t kNoneByte = 0x7FFFFFF0u;  // byte offset past every table (tables < 2^31 - 16 bytes)

// Per-(unit, chunk) block of Phase 1 results, in 4-byte words. Per-occurrence arrays are
// [kC][LIST] (LIST >= W, R; unused entries hold zeros and wb = -1). The list area holds the
// K and Q row starts, the K rows by dependency level and, from word kLa0 on, the write-back
// lists, then K's and Q's entries.
constexpr int kLev = 8;                  // dependency levels of K's rows kept as row masks
constexpr int kLevAt = 130;              // list-area word: number of levels (kLev + 1: more)
constexpr int kLa0 = 132 + 2 * kLev;
struct MetaLayout {
  int list;
  size_t gw, wc, ge, wb, gr, hdr, la, words;
};
__host__ __device__ inline MetaLayout meta_layout(int list) {
  MetaLayout m;
  m.list = list;
  const size_t occ = (size_t)kC * list;
  m.gw = 0;               // alpha_t a_tj dec(n_tj; start, t)
  m.wc = m.gw + occ;      // a_tj dec(n_tj; t, end): the occurrence's own write-back coefficient
  m.ge = m.wc + occ;      // dec(n_tj; start, end) for the slot's last writer
  m.wb = m.ge + occ;      // -1, or for the slot's last writer (start << 8 | count) of its other writers
  m.gr = m.wb + occ;      // u_tr dec(m_tr; start, t+1)
  m.hdr = m.gr + occ;     // [0] write-back entries, [1] K entries, [2] Q entries, [3..4] rows with K entries
  m.la = m.hdr + 8;       // [0, 65) K row starts, [65, 130) Q row starts, [kLevAt] levels, [132 + 2l, +2) rows
                          // of level l + 1, [kLa0, ...) entries (tau, coef):
                          // write-back lists, then K (coef beta_t K[t][tau]), then Q, each sorted by t
  m.words = (m.la + kLa0 + 2 * (occ + kKMax + kQMax) + 63) & ~(size_t)63;
  return m;
}
inline int list_for(const sdm_shape& S) {
  const int m = S.W > S.R ? S.W : S.R;
  return m <= 8 ? 8 : m <= 16 ? 16 : 32;
}

struct ChunkArgs {
  const int32_t* widx;  // [U][T][W]
  const float* wgt;
  const int32_t* ridx;  // [U][T][R]
  const float* rgt;
  const float* alpha;   // [U][T]
  const float* beta;
  const void* v;        // [U][T][d_v]
  void* M;              // [U][N][d_v]
  float* o;             // [U][T][d_v]
  uint32_t* meta;       // [U][nchunk][words]
  MetaLayout ml;
  int U, T, W, R, d_v, nchunk, ncb;
  long long N;
};

__device__ __forceinline__ uint32_t chunk_hash(uint32_t s) { return (s * 2654435761u) >> 20; }  // 12 bits
__device__ __forceinline__ uint32_t filter_bit(uint32_t s) { return (s * 0x9E3779B1u) >> 18; }  // 14 bits

template <int LIST>
__global__ void __launch_bounds__(256) chunk_prep_kernel(ChunkArgs A) {
  constexpr int NOC = kC * LIST;
  constexpr int NO = NOC / 256;  // occurrences per thread, write and read each
  constexpr int SH = LIST == 8 ? 3 : LIST == 16 ? 4 : 5;
  // 48 KB of LDS: three workgroups per CU
  __shared__ short snx[NOC];       // next write occurrence [t][LIST] of the same slot, -1 at the end
  __shared__ uint32_t keys[kBuckets];
  __shared__ uint32_t head2[kBuckets / 2];  // first occurrence of each bucket's slot, 16 bits each (0xFFFF: none)
  // couplings: K[t][tau] at [t][tau] (tau < t), Q[t][tau] at [tau][t] (tau <= t)
  __shared__ float KQ[kC][kC + 1];
  __shared__ unsigned long long kmask[kC], qmask[kC];
  __shared__ float sal[kC], sbe[kC];
  __shared__ uint32_t filt[kFilterWords];  // a slot whose bit is clear is not written in the chunk
  __shared__ int wlcnt, tot[2];
  const int chunk = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int W = A.W, R = A.R, T = A.T;
  const int t0 = chunk * kC, L = min(kC, T - t0);
  const long long N = A.N;
  const size_t ut0 = (size_t)u * T + t0;
  uint32_t* blk = A.meta + ((size_t)u * A.nchunk + chunk) * A.ml.words;
  uint32_t* la = blk + A.ml.la;
  // this thread's occurrences i = tid + 256 k, all loads in flight at once
  int ws[NO], rs[NO];
  float wa[NO], ra[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int i = tid + 256 * k, t = i >> SH, j = i & (LIST - 1);
    const bool okw = t < L && j < W, okr = t < L && j < R;
    ws[k] = okw ? A.widx[(ut0 + t) * W + j] : -1;
    wa[k] = okw ? A.wgt[(ut0 + t) * W + j] : 0.f;
    rs[k] = okr ? A.ridx[(ut0 + t) * R + j] : -1;
    ra[k] = okr ? A.rgt[(ut0 + t) * R + j] : 0.f;
  }
  for (int i = tid; i < kBuckets; i += 256) keys[i] = kFree;
  for (int i = tid; i < kBuckets / 2; i += 256) head2[i] = 0xFFFFFFFFu;
  for (int i = tid; i < kFilterWords; i += 256) filt[i] = 0u;
  for (int i = tid; i < kC * (kC + 1); i += 256) (&KQ[0][0])[i] = 0.f;
  if (tid < kC) {
    kmask[tid] = 0ull;
    qmask[tid] = 0ull;
    sal[tid] = tid < L ? A.alpha[ut0 + tid] : 1.f;
    sbe[tid] = tid < L ? A.beta[ut0 + tid] : 0.f;
  }
  if (tid == 0) wlcnt = 0;
#pragma unroll
  for (int k = 0; k < NO; ++k)
    if (ws[k] < 0 || ws[k] >= N) ws[k] = -1;
  __syncthreads();
  // list heads: 16-bit entries, exchanged by compare-and-swap on their 32-bit word
  auto head_at = [&](int b) -> int {
    const int v = (int)((head2[b >> 1] >> ((b & 1) * 16)) & 0xFFFFu);
    return v == 0xFFFF ? -1 : v;
  };
  auto head_xchg = [&](int b, int v) -> int {
    uint32_t* w = &head2[b >> 1];
    const int sh = (b & 1) * 16;
    uint32_t old = *w;
    while (true) {
      const uint32_t nw = (old & ~(0xFFFFu << sh)) | ((uint32_t)v << sh);
      const uint32_t prev = atomicCAS(w, old, nw);
      if (prev == old) break;
      old = prev;
    }
    const int pv = (int)((old >> sh) & 0xFFFFu);
    return pv == 0xFFFF ? -1 : pv;
  };
  // the weight of write occurrence q (t LIST + j): from the input, for the rare slots with
  // several writers in the chunk
  auto wgt_of = [&](int q) -> float { return A.wgt[(ut0 + (q >> SH)) * W + (q & (LIST - 1))]; };
  auto find = [&](uint32_t s) -> int {  // bucket of a slot written in the chunk, or -1
    uint32_t b = chunk_hash(s);
    while (true) {
      const uint32_t k = keys[b];
      if (k == s) return (int)b;
      if (k == kFree) return -1;
      b = (b + 1) & (kBuckets - 1);
    }
  };
  auto insert = [&](uint32_t s) -> int {  // claim (or find) the slot's bucket
    uint32_t b = chunk_hash(s);
    while (true) {
      const uint32_t old = atomicCAS(&keys[b], kFree, s);
      if (old == kFree || old == s) return (int)b;
      b = (b + 1) & (kBuckets - 1);
    }
  };
  // Each stage issues this thread's occurrences together (one LDS round trip per stage):
  // claim the home bucket, then (rarely) probe on, then link into the slot's list.
  int bk[NO];
  uint32_t old[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    bk[k] = ws[k] >= 0 ? (int)chunk_hash((uint32_t)ws[k]) : -1;
    old[k] = ws[k] >= 0 ? atomicCAS(&keys[bk[k]], kFree, (uint32_t)ws[k]) : kFree;
  }
#pragma unroll
  for (int k = 0; k < NO; ++k)
    if (ws[k] >= 0 && old[k] != kFree && old[k] != (uint32_t)ws[k])
      bk[k] = insert((uint32_t)ws[k]);  // the home bucket holds another slot
  int nx[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) nx[k] = ws[k] >= 0 ? head_xchg(bk[k], tid + 256 * k) : -1;
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int i = tid + 256 * k;
    snx[i] = (short)nx[k];
    if (ws[k] >= 0) {
      const uint32_t fb = filter_bit((uint32_t)ws[k]);
      atomicOr(&filt[fb >> 5], 1u << (fb & 31));
    }
  }
  __syncthreads();
  // write occurrences: couplings to earlier writers, gathered decay, write-back terms
  int hd[NO];
  float st[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    hd[k] = ws[k] >= 0 ? head_at(bk[k]) : -1;
    st[k] = sal[(tid + 256 * k) >> SH];
  }
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int i = tid + 256 * k, t = i >> SH;
    float gwv = 0.f, wcv = 0.f, gev = 0.f;
    int wbv = -1;
    if (ws[k] >= 0 && hd[k] == i && nx[k] < 0) {  // the slot's only writer in the chunk
      gwv = st[k] * wa[k];
      wcv = wa[k];
      gev = st[k];
      wbv = 0;
    } else if (ws[k] >= 0) {
      const int b = bk[k];
      const float a = wa[k];
      float before = 1.f, after = 1.f, all = 1.f;
      int others = 0;
      for (int q = head_at(b); q >= 0; q = snx[q]) {
        const int tk = q >> SH;
        all *= sal[tk];
        if (tk < t) {
          before *= sal[tk];
          float between = 1.f;  // dec(n; tk, t)
          for (int l = head_at(b); l >= 0; l = snx[l]) {
            const int tl = l >> SH;
            if (tl > tk && tl < t) between *= sal[tl];
          }
          atomicAdd(&KQ[t][tk], sal[t] * a * between * wgt_of(q));
          atomicOr(&kmask[t], 1ull << tk);
          ++others;
        } else if (tk > t) {
          after *= sal[tk];
          others = -1000;  // not the last writer
        }
      }
      gwv = sal[t] * a * before;
      wcv = a * after;
      if (others >= 0) {  // the slot's last writer writes it back
        gev = all;
        const int start = others ? atomicAdd(&wlcnt, others) : 0;
        int e = start;
        for (int q = head_at(b); q >= 0; q = snx[q]) {
          const int tk = q >> SH;
          if (tk >= t) continue;  // the same writers that were counted
          float aft = 1.f;        // dec(n; tk, end)
          for (int l = head_at(b); l >= 0; l = snx[l])
            if ((l >> SH) > tk) aft *= sal[l >> SH];
          la[kLa0 + 2 * e] = (uint32_t)tk;
          la[kLa0 + 2 * e + 1] = __float_as_uint(wgt_of(q) * aft);
          ++e;
        }
        wbv = start << 8 | others;
      }
    }
    blk[A.ml.gw + i] = __float_as_uint(gwv);
    blk[A.ml.wc + i] = __float_as_uint(wcv);
    blk[A.ml.ge + i] = __float_as_uint(gev);
    blk[A.ml.wb + i] = (uint32_t)wbv;
  }
  // read occurrences: couplings to the chunk's writers up to and including the token
  uint32_t fw[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const uint32_t fb = filter_bit((uint32_t)rs[k]);
    fw[k] = (filt[fb >> 5] >> (fb & 31)) & 1u;
  }
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int i = tid + 256 * k, t = i >> SH;
    float grv = 0.f;
    const int s = rs[k];
    if (s >= 0 && s < N && fw[k] == 0u) {
      grv = ra[k];  // the slot is not written in the chunk
    } else if (s >= 0 && s < N) {
      const float w = ra[k];
      const int b = find((uint32_t)s);
      float upto = 1.f;
      if (b >= 0) {
        for (int q = head_at(b); q >= 0; q = snx[q]) {
          const int tk = q >> SH;
          if (tk > t) continue;
          upto *= sal[tk];
          float between = 1.f;  // dec(m; tk, t + 1)
          for (int l = head_at(b); l >= 0; l = snx[l]) {
            const int tl = l >> SH;
            if (tl > tk && tl <= t) between *= sal[tl];
          }
          atomicAdd(&KQ[tk][t], w * between * wgt_of(q));
          atomicOr(&qmask[t], 1ull << tk);
        }
      }
      grv = w * upto;
    }
    blk[A.ml.gr + i] = __float_as_uint(grv);
  }
  __syncthreads();
  // couplings out as row-sorted lists: wave 0 for K, wave 1 for Q (lane = row)
  const int wave = tid >> 6, lane = tid & 63;
  unsigned long long m0 = 0;
  int off = 0;
  if (wave < 2) {
    m0 = wave == 0 ? kmask[lane] : qmask[lane];
    const int cnt = __popcll(m0);
    off = cnt;  // inclusive scan over the 64 rows
    for (int s = 1; s < 64; s <<= 1) {
      const int x = __shfl_up(off, s, 64);
      if (lane >= s) off += x;
    }
    if (lane == 63) tot[wave] = off;
    off -= cnt;
    const unsigned long long rows = __ballot(cnt > 0);
    if (wave == 0) {
      // dependency level of each K row: 0 without entries, else one more than its deepest
      // entry's row; rows are final in ascending order (entries point to earlier rows)
      int lv = 0;
      for (int r = 0; r < kC; ++r) {
        const int l = __builtin_amdgcn_readlane(lv, r);
        if ((m0 >> r) & 1ull) lv = max(lv, l + 1);
      }
      int top = lv;
      for (int s = 32; s >= 1; s >>= 1) top = max(top, __shfl_xor(top, s, 64));
      unsigned long long lm[kLev];
#pragma unroll
      for (int l = 0; l < kLev; ++l) lm[l] = __ballot(lv == l + 1);
      if (lane == 0) {
        blk[A.ml.hdr + 3] = (uint32_t)rows;
        blk[A.ml.hdr + 4] = (uint32_t)(rows >> 32);
        la[kLevAt] = (uint32_t)min(top, kLev + 1);
#pragma unroll
        for (int l = 0; l < kLev; ++l) {
          la[132 + 2 * l] = (uint32_t)lm[l];
          la[133 + 2 * l] = (uint32_t)(lm[l] >> 32);
        }
      }
    }
  }
  __syncthreads();
  if (wave < 2) {
    const int wn = wlcnt, kn = tot[0], qn = tot[1];
    const int rp = wave == 0 ? 0 : 65, ep = kLa0 + 2 * wn + (wave == 0 ? 0 : 2 * kn);
    la[rp + lane] = (uint32_t)off;
    if (lane == 63) la[rp + 64] = (uint32_t)(wave == 0 ? kn : qn);
    unsigned long long m = m0;
    int e = off;
    while (m) {
      const int tk = __builtin_ctzll(m);
      m &= m - 1;
      const float c = wave == 0 ? sbe[lane] * KQ[lane][tk] : KQ[tk][lane];
      la[ep + 2 * e] = (uint32_t)tk;
      la[ep + 2 * e + 1] = __float_as_uint(c);
      ++e;
    }
    if (wave == 0 && lane == 0) {
      blk[A.ml.hdr] = (uint32_t)wn;
      blk[A.ml.hdr + 1] = (uint32_t)kn;
      blk[A.ml.hdr + 2] = (uint32_t)qn;
    }
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rs(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(uint32_t)bytes, 0x00020000);
}

// A row piece of CBD dwords: buffer load and store in one instruction.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int CBD>
__device__ __forceinline__ void piece_ld(rsrc_t rs, uint32_t off, uint32_t* w) {
  if constexpr (CBD == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
  } else if constexpr (CBD == 2) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    w[0] = x.x, w[1] = x.y;
  } else {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    w[0] = x.x, w[1] = x.y, w[2] = x.z, w[3] = x.w;
  }
}
template <int CBD>
__device__ __forceinline__ void piece_st(rsrc_t rs, uint32_t off, const uint32_t* w) {
  if constexpr (CBD == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, off, 0, 0);
  } else if constexpr (CBD == 2) {
    u32x2 x;
    x.x = w[0], x.y = w[1];
    __builtin_amdgcn_raw_buffer_store_b64(x, rs, off, 0, 0);
  } else {
    u32x4 x;
    x.x = w[0], x.y = w[1], x.z = w[2], x.w = w[3];
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, off, 0, 0);
  }
}

template <typename MemT>
struct RowWord;
template <>
struct RowWord<float> {
  static constexpr int kCols = 1;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = __uint_as_float(w); }
  __device__ static uint32_t pack(const float* x) { return __float_as_uint(x[0]); }
};
template <>
struct RowWord<uint16_t> {
  static constexpr int kCols = 2;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = bf16lo(w); x[1] = bf16hi(w); }
  __device__ static uint32_t pack(const float* x) { return pack_bf16x2(x[0], x[1]); }
};

// N consecutive words from a 4N-byte aligned address (N = 2, 4 or 8)
template <int N>
__device__ __forceinline__ void ld_words(const uint32_t* p, uint32_t* w) {
  if constexpr (N == 2) {
    const uint2 x = *(const uint2*)p;
    w[0] = x.x, w[1] = x.y;
  } else {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const uint4 x = ((const uint4*)p)[k];
      w[4 * k] = x.x, w[4 * k + 1] = x.y, w[4 * k + 2] = x.z, w[4 * k + 3] = x.w;
    }
  }
}

template <typename InT>
__device__ __forceinline__ float in_ld(const InT* p) {
  if constexpr (sizeof(InT) == 2) return bf16_to_f32(*p);
  else return *p;
}

#ifndef SDM_CHUNK_CFG
#define SDM_CHUNK_CFG 0  // lane map of the apply kernel: 0 picks by shape
#endif

// Phase 2. A workgroup owns a block of NQ * QD row dwords of one unit; the lanes of a token
// are (occurrence group g < G, quad q < NQ): lane (g, q) gathers dwords [q QD, q QD + QD) of
// the block for the token's occurrences [g OPL, g OPL + OPL), so the NQ lanes of one
// occurrence read NQ * QD contiguous dwords. P and O0 are summed over the G groups. With PRE
// the next chunk's slots are loaded while the current chunk runs (registers for latency).
template <typename MemT, typename InT, int QD, int NQ, int G, bool PRE, int LIST>
__global__ void __launch_bounds__(64 * NQ * G) chunk_apply_kernel(ChunkArgs A) {
  using RW = RowWord<MemT>;
  constexpr int LPT = NQ * G;            // lanes per token
  constexpr int NT = 64 * LPT;
  constexpr int OPL = LIST / G;          // occurrences per lane, write and read each
  constexpr int CPL = RW::kCols;
  constexpr int CBD = QD * NQ;           // row dwords per workgroup
  constexpr int NCOL = CBD * CPL;        // table columns per workgroup
  constexpr int QC = QD * CPL;           // columns of one lane's piece
  constexpr int CPLN = QC >= G ? QC / G : 1;  // columns of delta and o per lane
  constexpr int NLA = kLa0 + 2 * (kC * LIST + kKMax + kQMax);
  static_assert(NCOL <= 64 && OPL >= 2 && LPT <= 64, "lane map");
  __shared__ float D[kC][NCOL];          // delta of the chunk's tokens
  __shared__ uint32_t lst[NLA];          // the chunk's list area
  // blockIdx -> (unit, column block) with all column blocks of a unit in one L2 domain
  const int xcd = blockIdx.x % kXcd, y = blockIdx.x / kXcd;
  const int p = y % A.ncb, u = (y / A.ncb) * kXcd + xcd;
  if (u >= A.U) return;
  const int tid = threadIdx.x, t = tid / LPT, g = (tid % LPT) / NQ, q = tid % NQ;
  const int T = A.T, W = A.W, R = A.R, d_v = A.d_v;
  const int rowdw = d_v / CPL;  // a multiple of CBD
  const long long N = A.N;
  const rsrc_t rM = make_rs((const char*)A.M + (size_t)u * N * d_v * sizeof(MemT), (size_t)N * d_v * sizeof(MemT));
  const int qc0 = q * QC;                          // this lane's first column inside the block
  const int lc0 = qc0 + g * CPLN;                  // its first column of delta and o
  const bool cl = g * CPLN < QC;
  const InT* v = (const InT*)A.v + (size_t)u * T * d_v + p * NCOL + lc0;
  float* o = A.o + (size_t)u * T * d_v + p * NCOL + lc0;
  const int32_t* widx = A.widx + (size_t)u * T * W;
  const int32_t* ridx = A.ridx + (size_t)u * T * R;
  const float* beta = A.beta + (size_t)u * T;
  const uint32_t* meta = A.meta + (size_t)u * A.nchunk * A.ml.words;
  const MetaLayout ml = A.ml;
  const uint32_t pc = (uint32_t)(p * CBD + q * QD) * 4u;  // byte offset of the piece inside a row

  // this lane's slots of chunk c: occurrences j = g OPL + i (with the prefetch, 16-byte loads
  // when the lists fill LIST: each lane request then carries four slots; a token past T reads
  // token 0's and discards them. Without it the slots are needed at once and the narrower
  // loads keep the registers of the wide pieces below the spill point)
  const bool full = PRE && (OPL % 4 == 0) && W == LIST && R == LIST;
  auto fetch = [&](int c, int (&sw)[OPL], int (&sr)[OPL]) {
    const int tt = c * kC + t;
    const bool ok = tt < T;
    if (OPL % 4 == 0 && full) {
      const size_t base = ok ? (size_t)tt * LIST + g * OPL : 0;
#pragma unroll
      for (int k = 0; k < (OPL % 4 == 0 ? OPL / 4 : 0); ++k) {
        const int4 a = ((const int4*)(widx + base))[k], b = ((const int4*)(ridx + base))[k];
        sw[4 * k] = ok ? a.x : -1, sw[4 * k + 1] = ok ? a.y : -1;
        sw[4 * k + 2] = ok ? a.z : -1, sw[4 * k + 3] = ok ? a.w : -1;
        sr[4 * k] = ok ? b.x : -1, sr[4 * k + 1] = ok ? b.y : -1;
        sr[4 * k + 2] = ok ? b.z : -1, sr[4 * k + 3] = ok ? b.w : -1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < OPL; ++i) {
        const int j = g * OPL + i;
        sw[i] = ok && j < W ? widx[(size_t)tt * W + j] : -1;
        sr[i] = ok && j < R ? ridx[(size_t)tt * R + j] : -1;
      }
    }
  };
  int sw[OPL], sr[OPL];
  if constexpr (PRE) fetch(0, sw, sr);
  uint32_t h0 = meta[ml.hdr], h1 = meta[ml.hdr + 1], h2 = meta[ml.hdr + 2], h3 = meta[ml.hdr + 3],
           h4 = meta[ml.hdr + 4];

  for (int chunk = 0; chunk < A.nchunk; ++chunk) {
    const int t0 = chunk * kC;
    const bool tv = t0 + t < T;
    const uint32_t* mb = meta + (size_t)chunk * ml.words;
    const int wn = (int)h0, kn = (int)h1, qn = (int)h2;
    const unsigned long long krows = (unsigned long long)h3 | (unsigned long long)h4 << 32;
    const int nla = kLa0 + 2 * (wn + kn + qn);
    if constexpr (!PRE) fetch(chunk, sw, sr);
    // the list area: the first 2 NT words through registers, alongside the row traffic
    uint32_t lr0 = 0, lr1 = 0;
    if (tid < nla) lr0 = mb[ml.la + tid];
    if (tid + NT < nla) lr1 = mb[ml.la + tid + NT];
    // byte offsets of this lane's row pieces (kNoneByte: no row; loads read 0, stores drop)
    uint32_t wo[OPL], ro[OPL];
#pragma unroll
    for (int i = 0; i < OPL; ++i) {
      wo[i] = sw[i] >= 0 && sw[i] < N ? (uint32_t)sw[i] * (uint32_t)rowdw * 4u + pc : kNoneByte;
      ro[i] = sr[i] >= 0 && sr[i] < N ? (uint32_t)sr[i] * (uint32_t)rowdw * 4u + pc : kNoneByte;
    }
    uint32_t mw[OPL][QD], mr[OPL][QD];
#pragma unroll
    for (int i = 0; i < OPL; ++i) piece_ld<QD>(rM, wo[i], mw[i]);
#pragma unroll
    for (int i = 0; i < OPL; ++i) piece_ld<QD>(rM, ro[i], mr[i]);
    // gathered coefficients (zeros past the lists and past the chunk)
    const uint32_t* mt = mb + (size_t)t * LIST + g * OPL;
    float gw[OPL], gr[OPL];
    {
      uint32_t a[OPL], b[OPL];
      ld_words<OPL>(mt + ml.gw, a);
      ld_words<OPL>(mt + ml.gr, b);
#pragma unroll
      for (int i = 0; i < OPL; ++i) gw[i] = __uint_as_float(a[i]), gr[i] = __uint_as_float(b[i]);
    }
    float vv[CPLN], be = 0.f;
#pragma unroll
    for (int c = 0; c < CPLN; ++c) vv[c] = 0.f;
    if (tv && cl) {
#pragma unroll
      for (int c = 0; c < CPLN; ++c) vv[c] = in_ld<InT>(v + (size_t)(t0 + t) * d_v + c);
      be = beta[t0 + t];
    }
    // P and O0 from the chunk-start rows: partial sums over this lane's occurrences, then the groups
    float P[QC], O0[QC];
#pragma unroll
    for (int c = 0; c < QC; ++c) P[c] = O0[c] = 0.f;
#pragma unroll
    for (int i = 0; i < OPL; ++i) {
#pragma unroll
      for (int k = 0; k < QD; ++k) {
        float x[CPL], z[CPL];
        RW::unpack(mw[i][k], x);
        RW::unpack(mr[i][k], z);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          P[k * CPL + c] = fmaf(gw[i], x[c], P[k * CPL + c]);
          O0[k * CPL + c] = fmaf(gr[i], z[c], O0[k * CPL + c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < QC; ++c) {
#pragma unroll
      for (int s = NQ; s < LPT; s <<= 1) {
        P[c] += __shfl_xor(P[c], s, 64);
        O0[c] += __shfl_xor(O0[c], s, 64);
      }
    }
    // this lane's columns g CPLN + cc of its piece, picked by selects (no indexing by a lane value)
    float ol[CPLN];
#pragma unroll
    for (int cc = 0; cc < CPLN; ++cc) {
      float ps = 0.f, os = 0.f;
#pragma unroll
      for (int c = 0; c < QC; ++c)
        if (c == g * CPLN + cc) ps = P[c], os = O0[c];
      ol[cc] = os;
      if (cl) D[t][lc0 + cc] = be * (vv[cc] - ps);
    }
    // write-back coefficients, the next chunk's slots and header: in flight during the solve
    float wc[OPL], ge[OPL];
    int wb[OPL];
    {
      uint32_t a[OPL], b[OPL], c[OPL];
      ld_words<OPL>(mt + ml.wc, a);
      ld_words<OPL>(mt + ml.ge, b);
      ld_words<OPL>(mt + ml.wb, c);
#pragma unroll
      for (int i = 0; i < OPL; ++i) wc[i] = __uint_as_float(a[i]), ge[i] = __uint_as_float(b[i]), wb[i] = (int)c[i];
    }
    int nw_[OPL], nr_[OPL];
    if (chunk + 1 < A.nchunk) {
      if constexpr (PRE) fetch(chunk + 1, nw_, nr_);
      const uint32_t* hn = mb + ml.words + ml.hdr;
      h0 = hn[0], h1 = hn[1], h2 = hn[2], h3 = hn[3], h4 = hn[4];
    }
    lst[tid] = lr0;  // kLa0 > 0 words: always in range
    if (tid + NT < NLA) lst[tid + NT] = lr1;
    for (int i = tid + 2 * NT; i < nla; i += NT) lst[i] = mb[ml.la + i];
    __syncthreads();
    // forward solve over the K list: delta_t -= beta_t K[t][tau] delta_tau. Rows of one
    // dependency level need only rows of lower levels: each row's own lanes update it, one
    // barrier per level; past kLev levels a few lanes sweep the rows in order.
    if (kn > 0) {
      const uint32_t* ke = lst + kLa0 + 2 * wn;
      const int nlev = (int)lst[kLevAt];
      if (nlev <= kLev) {
        for (int l = 0; l < nlev; ++l) {
          const unsigned long long m = (unsigned long long)lst[132 + 2 * l] | (unsigned long long)lst[133 + 2 * l] << 32;
          if (((m >> t) & 1ull) && cl) {
            float acc[CPLN];
#pragma unroll
            for (int c = 0; c < CPLN; ++c) acc[c] = D[t][lc0 + c];
            for (int e = (int)lst[t]; e < (int)lst[t + 1]; ++e) {
              const float kv = __uint_as_float(ke[2 * e + 1]);
              const int tk = (int)ke[2 * e];
#pragma unroll
              for (int c = 0; c < CPLN; ++c) acc[c] = fmaf(-kv, D[tk][lc0 + c], acc[c]);
            }
#pragma unroll
            for (int c = 0; c < CPLN; ++c) D[t][lc0 + c] = acc[c];
          }
          __syncthreads();
        }
      } else {
        if (tid < NCOL) {
          unsigned long long rows = krows;
          while (rows) {
            const int r = __builtin_ctzll(rows);
            rows &= rows - 1;
            float acc = D[r][tid];
            for (int e = (int)lst[r]; e < (int)lst[r + 1]; ++e)
              acc = fmaf(-__uint_as_float(ke[2 * e + 1]), D[ke[2 * e]][tid], acc);
            D[r][tid] = acc;
          }
        }
        __syncthreads();
      }
    }
    // o = O0 + Q delta
    if (tv && cl) {
      const uint32_t* qe = lst + kLa0 + 2 * (wn + kn);
      for (int e = (int)lst[65 + t]; e < (int)lst[66 + t]; ++e) {
        const int tk = (int)qe[2 * e];
        const float qv = __uint_as_float(qe[2 * e + 1]);
#pragma unroll
        for (int c = 0; c < CPLN; ++c) ol[c] = fmaf(qv, D[tk][lc0 + c], ol[c]);
      }
      float* op = o + (size_t)(t0 + t) * d_v;
      if constexpr (CPLN % 4 == 0) {
#pragma unroll
        for (int c = 0; c < CPLN; c += 4) *(float4*)(op + c) = make_float4(ol[c], ol[c + 1], ol[c + 2], ol[c + 3]);
      } else if constexpr (CPLN == 2) {
        *(float2*)op = make_float2(ol[0], ol[1]);
      } else {
#pragma unroll
        for (int c = 0; c < CPLN; ++c) op[c] = ol[c];
      }
    }
    // each slot's last writer writes its row piece back once
    float dt[QC];
#pragma unroll
    for (int c = 0; c < QC; ++c) dt[c] = D[t][qc0 + c];
#pragma unroll
    for (int i = 0; i < OPL; ++i) {
      if (wb[i] < 0) continue;
      float yv[QC];
#pragma unroll
      for (int k = 0; k < QD; ++k) {
        float x[CPL];
        RW::unpack(mw[i][k], x);
#pragma unroll
        for (int c = 0; c < CPL; ++c) yv[k * CPL + c] = fmaf(ge[i], x[c], wc[i] * dt[k * CPL + c]);
      }
      const int e0 = wb[i] >> 8, e1 = e0 + (wb[i] & 255);
      for (int e = e0; e < e1; ++e) {
        const int tk = (int)lst[kLa0 + 2 * e];
        const float a = __uint_as_float(lst[kLa0 + 2 * e + 1]);
#pragma unroll
        for (int c = 0; c < QC; ++c) yv[c] = fmaf(a, D[tk][qc0 + c], yv[c]);
      }
      uint32_t pw[QD];
#pragma unroll
      for (int k = 0; k < QD; ++k) pw[k] = RW::pack(yv + k * CPL);
      piece_st<QD>(rM, wo[i], pw);
    }
    if constexpr (PRE) {
#pragma unroll
      for (int i = 0; i < OPL; ++i) sw[i] = nw_[i], sr[i] = nr_[i];
    }
    // the next chunk's gathers read these rows: stores complete, then the barrier
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

template <typename MemT, typename InT, int QD, int NQ, int G, bool PRE>
hipError_t launch_apply(ChunkArgs& A, int list, hipStream_t st) {
  constexpr int CPL = RowWord<MemT>::kCols;
  A.ncb = A.d_v / CPL / (QD * NQ);
  const int wgs = (A.U + kXcd - 1) / kXcd * kXcd * A.ncb;
  const dim3 gr((unsigned)wgs), b(64 * NQ * G);
  if (list == 8) hipLaunchKernelGGL((chunk_apply_kernel<MemT, InT, QD, NQ, G, PRE, 8>), gr, b, 0, st, A);
  else if (list == 16) hipLaunchKernelGGL((chunk_apply_kernel<MemT, InT, QD, NQ, G, PRE, 16>), gr, b, 0, st, A);
  else hipLaunchKernelGGL((chunk_apply_kernel<MemT, InT, QD, NQ, G, PRE, 32>), gr, b, 0, st, A);
  return hipGetLastError();
}

template <typename MemT, typename InT>
hipError_t launch_apply_cfg(ChunkArgs& A, int list, hipStream_t st) {
  constexpr int CPL = RowWord<MemT>::kCols;
  const int rowdw = A.d_v / CPL;  // a multiple of 4
  const long long ug = (A.U + kXcd - 1) / kXcd * kXcd;
  const int cus = device_cus();
  int cfg = SDM_CHUNK_CFG;
  if (cfg == 0) {
    // Units of one L2 domain stream their chunks' rows through it together. With one unit
    // per domain, narrow pieces keep every compute unit busy and the rows are reused from
    // L2; with more, each workgroup reads whole 64-byte sectors (16-dword pieces).
    if (A.U > kXcd && rowdw % 16 == 0 && ug * (rowdw / 16) >= cus) cfg = 1;
    else if (ug * (rowdw / 4) >= cus) cfg = 2;
    else cfg = ug * (rowdw / 2) >= cus ? 3 : 4;
  }
  switch (cfg) {
    case 1: return launch_apply<MemT, InT, 4, 4, 2, false>(A, list, st);  // 16 dwords, 512 lanes
    case 2: return launch_apply<MemT, InT, 4, 1, 4, true>(A, list, st);   // 4 dwords
    case 3: return launch_apply<MemT, InT, 2, 1, 4, true>(A, list, st);   // 2 dwords
    default: return launch_apply<MemT, InT, 1, 1, 4, true>(A, list, st);  // 1 dword
  }
}

}  // namespace

size_t chunked_workspace_bytes(const sdm_shape& S) {
  const size_t nch = ((size_t)S.T + kC - 1) / kC;
  return 256 + (size_t)S.B * S.H * nch * meta_layout(list_for(S)).words * 4;
}

bool chunked_supported(const sdm_shape& S) {
  // byte offsets of rows stay below the sentinel
  return S.W <= kMaxList && S.R <= kMaxList && (size_t)S.N * S.d_v * dtype_size(S.mem_dtype) < kNoneByte;
}

hipError_t launch_chunked(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                          const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                          void* ws, hipStream_t stream) {
  if (!chunked_supported(S)) return hipErrorInvalidValue;
  ChunkArgs A;
  A.widx = widx;
  A.wgt = wgt;
  A.ridx = ridx;
  A.rgt = rgt;
  A.alpha = alpha;
  A.beta = beta;
  A.v = v;
  A.M = M;
  A.o = o;
  A.U = S.B * S.H;
  A.T = S.T;
  A.W = S.W;
  A.R = S.R;
  A.d_v = S.d_v;
  A.N = S.N;
  A.nchunk = (S.T + kC - 1) / kC;
  A.ml = meta_layout(list_for(S));
  A.meta = (uint32_t*)((char*)ws + 256);
  A.ncb = 0;
  if (A.U == 0 || A.T == 0) return hipSuccess;
  const int list = A.ml.list;
  const dim3 pg((unsigned)A.nchunk, (unsigned)A.U);
  if (list == 8) hipLaunchKernelGGL(chunk_prep_kernel<8>, pg, dim3(256), 0, stream, A);
  else if (list == 16) hipLaunchKernelGGL(chunk_prep_kernel<16>, pg, dim3(256), 0, stream, A);
  else hipLaunchKernelGGL(chunk_prep_kernel<32>, pg, dim3(256), 0, stream, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return launch_apply_cfg<uint16_t, uint16_t>(A, list, stream);
  if (mb) return launch_apply_cfg<uint16_t, float>(A, list, stream);
  if (ib) return launch_apply_cfg<float, uint16_t>(A, list, stream);
  return launch_apply_cfg<float, float>(A, list, stream);
}

}  // namespace sdm
