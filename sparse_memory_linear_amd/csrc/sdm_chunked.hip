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
// chunk's write occurrences go into an LDS hash of per-slot linked lists; each write and read
// occurrence walks its slot's list for its couplings (accumulated densely in LDS, with a bit
// mask per row of the pairs that occur), its decay coefficient and its write-back terms. The
// product over a slot's writers between two tokens is a product over a set, so the list
// order does not matter. The couplings then leave as row-sorted lists.
//
// Phase 2 (chunk_apply_kernel, one workgroup per (unit, block of CBD row dwords), the chunks
// of a unit in order; lane = (token, dword)): each lane gathers its token's W + R row pieces
// at once and forms P and O0 in registers; delta starts as beta (V - P) in LDS, one wave
// sweeps the K list (if any), then o = O0 + Q delta and the last writer of each slot writes
// its row back once, rounded to the table dtype there. The next chunk's slot lists are
// prefetched into LDS while the current chunk runs.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kC = 64;                   // tokens per chunk
constexpr int kMaxList = 32;             // W, R <= 32 on this path
constexpr int kOcc = kC * kMaxList;
constexpr int kBuckets = 4096;           // LDS hash: at most 2048 distinct slots, at most half full
constexpr uint32_t kFree = 0xFFFFFFFFu;
constexpr int kKMax = kC * (kC - 1) / 2;  // distinct (t, tau < t) pairs
constexpr int kQMax = kC * (kC + 1) / 2;  // distinct (t, tau <= t) pairs
constexpr int kXcd = 8;                  // workgroups are dealt round-robin to this many L2 domains
constexpr uint32_t kNoneByte = 0x7FFFFFF0u;  // byte offset past every table (tables < 2^31 - 16 bytes)

// Per-(unit, chunk) block of Phase 1 results, in 4-byte words. Per-occurrence arrays are
// [kC][LIST] (LIST >= W, R; unused entries hold zeros and wb = -1).
struct MetaLayout {
  int list;
  size_t gw, wc, ge, wb, gr, hdr, kp, ke, qp, qe, wl, words;
};
__host__ __device__ inline size_t up4(size_t x) { return (x + 3) & ~(size_t)3; }
__host__ __device__ inline MetaLayout meta_layout(int list) {
  MetaLayout m;
  m.list = list;
  const size_t occ = (size_t)kC * list;
  m.gw = 0;               // alpha_t a_tj dec(n_tj; start, t)
  m.wc = m.gw + occ;      // a_tj dec(n_tj; t, end): the occurrence's own write-back coefficient
  m.ge = m.wc + occ;      // dec(n_tj; start, end) for the slot's last writer
  m.wb = m.ge + occ;      // -1, or for the slot's last writer (start << 8 | count) of its other writers in wl
  m.gr = m.wb + occ;      // u_tr dec(m_tr; start, t+1)
  m.hdr = m.gr + occ;     // [0] K entries, [1] Q entries, [2..3] 64-bit mask of rows with K entries
  m.kp = m.hdr + 4;       // [kC + 1] K row starts
  m.ke = up4(m.kp + kC + 1);   // [kKMax] (tau, beta_t K[t][tau]) sorted by t
  m.qp = m.ke + 2 * kKMax;     // [kC + 1] Q row starts
  m.qe = up4(m.qp + kC + 1);   // [kQMax] (tau, Q[t][tau]) sorted by t
  m.wl = m.qe + 2 * kQMax;     // [occ] (tau, a_tau dec(n; tau, end)): other writers of owned slots
  m.words = (m.wl + 2 * occ + 63) & ~(size_t)63;
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

__global__ void __launch_bounds__(256) chunk_prep_kernel(ChunkArgs A) {
  __shared__ int sn[kOcc];         // slot of each write occurrence, -1 for none
  __shared__ float sa[kOcc];       // its weight
  __shared__ short snx[kOcc];      // next occurrence of the same slot, -1 at the end
  __shared__ short sbk[kOcc];      // its hash bucket
  __shared__ uint32_t keys[kBuckets];
  __shared__ int head[kBuckets];
  // couplings: K[t][tau] at [t][tau] (tau < t), Q[t][tau] at [tau][t] (tau <= t)
  __shared__ float KQ[kC][kC + 1];
  __shared__ unsigned long long kmask[kC], qmask[kC];
  __shared__ float sal[kC], sbe[kC];
  __shared__ int wlcnt;
  const int chunk = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int W = A.W, R = A.R, T = A.T, LIST = A.ml.list;
  const int t0 = chunk * kC, L = min(kC, T - t0);
  const long long N = A.N;
  const size_t ut0 = (size_t)u * T + t0;
  uint32_t* blk = A.meta + ((size_t)u * A.nchunk + chunk) * A.ml.words;
  for (int i = tid; i < kBuckets; i += 256) {
    keys[i] = kFree;
    head[i] = -1;
  }
  for (int i = tid; i < kC * (kC + 1); i += 256) (&KQ[0][0])[i] = 0.f;
  if (tid < kC) {
    kmask[tid] = 0ull;
    qmask[tid] = 0ull;
    sal[tid] = tid < L ? A.alpha[ut0 + tid] : 1.f;
    sbe[tid] = tid < L ? A.beta[ut0 + tid] : 0.f;
  }
  if (tid == 0) wlcnt = 0;
  for (int i = tid; i < kC * W; i += 256) {
    const bool ok = i < L * W;
    const int s = ok ? A.widx[ut0 * W + i] : -1;
    sn[i] = s >= 0 && s < N ? s : -1;
    sa[i] = ok ? A.wgt[ut0 * W + i] : 0.f;
  }
  __syncthreads();
  auto find = [&](uint32_t s, bool insert) -> int {
    uint32_t b = chunk_hash(s);
    while (true) {
      const uint32_t k = keys[b];
      if (k == s) return (int)b;
      if (k == kFree) {
        if (!insert) return -1;
        const uint32_t old = atomicCAS(&keys[b], kFree, s);
        if (old == kFree || old == s) return (int)b;
      }
      b = (b + 1) & (kBuckets - 1);
    }
  };
  for (int i = tid; i < kC * W; i += 256) {
    if (sn[i] < 0) {
      snx[i] = -1;
      sbk[i] = -1;
      continue;
    }
    const int b = find((uint32_t)sn[i], true);
    sbk[i] = (short)b;
    snx[i] = (short)atomicExch(&head[b], i);
  }
  __syncthreads();
  // write occurrences: couplings to earlier writers, gathered decay, write-back terms
  for (int i = tid; i < kC * LIST; i += 256) {
    const int t = i / LIST, j = i % LIST, oi = t * W + j;
    float gwv = 0.f, wcv = 0.f, gev = 0.f;
    int wbv = -1;
    if (j < W && t < L && sn[oi] >= 0) {
      const int b = sbk[oi];
      float before = 1.f, after = 1.f, all = 1.f;
      int others = 0;
      for (int k = head[b]; k >= 0; k = snx[k]) {
        const int tk = k / W;
        all *= sal[tk];
        if (tk < t) {
          before *= sal[tk];
          float between = 1.f;  // dec(n; tk, t)
          for (int l = head[b]; l >= 0; l = snx[l]) {
            const int tl = l / W;
            if (tl > tk && tl < t) between *= sal[tl];
          }
          atomicAdd(&KQ[t][tk], sal[t] * sa[oi] * between * sa[k]);
          atomicOr(&kmask[t], 1ull << tk);
          ++others;
        } else if (tk > t) {
          after *= sal[tk];
          others = -1000;  // not the last writer
        }
      }
      gwv = sal[t] * sa[oi] * before;
      wcv = sa[oi] * after;
      if (others >= 0) {  // the slot's last writer writes it back
        gev = all;
        const int start = others ? atomicAdd(&wlcnt, others) : 0;
        int e = start;
        for (int k = head[b]; k >= 0; k = snx[k]) {
          const int tk = k / W;
          if (tk >= t) continue;  // the same writers that were counted
          float aft = 1.f;  // dec(n; tk, end)
          for (int l = head[b]; l >= 0; l = snx[l])
            if (l / W > tk) aft *= sal[l / W];
          blk[A.ml.wl + 2 * e] = (uint32_t)tk;
          blk[A.ml.wl + 2 * e + 1] = __float_as_uint(sa[k] * aft);
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
  for (int i = tid; i < kC * LIST; i += 256) {
    const int t = i / LIST, j = i % LIST;
    float grv = 0.f;
    if (j < R && t < L) {
      const int s = A.ridx[(ut0 + t) * R + j];
      const float w = A.rgt[(ut0 + t) * R + j];
      if (s >= 0 && s < N) {
        const int b = find((uint32_t)s, false);
        float upto = 1.f;
        if (b >= 0) {
          for (int k = head[b]; k >= 0; k = snx[k]) {
            const int tk = k / W;
            if (tk > t) continue;
            upto *= sal[tk];
            float between = 1.f;  // dec(m; tk, t + 1)
            for (int l = head[b]; l >= 0; l = snx[l]) {
              const int tl = l / W;
              if (tl > tk && tl <= t) between *= sal[tl];
            }
            atomicAdd(&KQ[tk][t], w * between * sa[k]);
            atomicOr(&qmask[t], 1ull << tk);
          }
        }
        grv = w * upto;
      }
    }
    blk[A.ml.gr + i] = __float_as_uint(grv);
  }
  __syncthreads();
  // couplings out as row-sorted lists: wave 0 for K, wave 1 for Q (lane = row)
  const int wave = tid >> 6, lane = tid & 63;
  if (wave < 2) {
    const unsigned long long m0 = wave == 0 ? kmask[lane] : qmask[lane];
    const int cnt = __popcll(m0);
    int off = cnt;  // inclusive scan over the 64 rows
    for (int s = 1; s < 64; s <<= 1) {
      const int x = __shfl_up(off, s, 64);
      if (lane >= s) off += x;
    }
    const int total = __shfl(off, 63, 64);
    off -= cnt;
    const size_t rp = wave == 0 ? A.ml.kp : A.ml.qp, ep = wave == 0 ? A.ml.ke : A.ml.qe;
    blk[rp + lane] = (uint32_t)off;
    if (lane == 63) blk[rp + 64] = (uint32_t)total;
    unsigned long long m = m0;
    int e = off;
    while (m) {
      const int tk = __builtin_ctzll(m);
      m &= m - 1;
      const float c = wave == 0 ? sbe[lane] * KQ[lane][tk] : KQ[tk][lane];
      blk[ep + 2 * e] = (uint32_t)tk;
      blk[ep + 2 * e + 1] = __float_as_uint(c);
      ++e;
    }
    const unsigned long long rows = __ballot(cnt > 0);
    if (lane == 0) {
      blk[A.ml.hdr + wave] = (uint32_t)total;
      if (wave == 0) {
        blk[A.ml.hdr + 2] = (uint32_t)rows;
        blk[A.ml.hdr + 3] = (uint32_t)(rows >> 32);
      }
    }
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rs(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(uint32_t)bytes, 0x00020000);
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

template <typename InT, int CPL>
__device__ __forceinline__ void load_v(const InT* p, float* x) {
  if constexpr (sizeof(InT) == 2) {
    if constexpr (CPL == 2) {
      const uint32_t w = *(const uint32_t*)p;
      x[0] = bf16lo(w);
      x[1] = bf16hi(w);
    } else {
      x[0] = bf16_to_f32(*p);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) x[c] = p[c];
  }
}

template <typename MemT, typename InT, int CBD, int LIST>
__global__ void __launch_bounds__(64 * CBD) chunk_apply_kernel(ChunkArgs A) {
  using RW = RowWord<MemT>;
  constexpr int CPL = RW::kCols;
  constexpr int NCOL = CBD * CPL;
  constexpr int NT = 64 * CBD;
  constexpr int PF = (2 * kC * LIST + NT - 1) / NT;  // prefetched slot indices per thread
  __shared__ float D[kC][NCOL + 1];                  // delta of the chunk's tokens
  __shared__ int sidx[2 * kC * LIST];                // the chunk's write and read slots, [kC][LIST] each
  // blockIdx -> (unit, column block) with all column blocks of a unit in one L2 domain
  const int xcd = blockIdx.x % kXcd, y = blockIdx.x / kXcd;
  const int p = y % A.ncb, u = (y / A.ncb) * kXcd + xcd;
  if (u >= A.U) return;
  const int tid = threadIdx.x, t = tid / CBD, d = tid % CBD;
  const int T = A.T, W = A.W, R = A.R, d_v = A.d_v;
  const int rowdw = d_v / CPL, dw = p * CBD + d;  // rowdw is a multiple of CBD
  const long long N = A.N;
  const rsrc_t rM = make_rs((const char*)A.M + (size_t)u * N * d_v * sizeof(MemT), (size_t)N * d_v * sizeof(MemT));
  const InT* v = (const InT*)A.v + (size_t)u * T * d_v + (size_t)dw * CPL;
  float* o = A.o + (size_t)u * T * d_v + (size_t)dw * CPL;
  const int32_t* widx = A.widx + (size_t)u * T * W;
  const int32_t* ridx = A.ridx + (size_t)u * T * R;
  const float* beta = A.beta + (size_t)u * T;
  const uint32_t* meta = A.meta + (size_t)u * A.nchunk * A.ml.words;
  const MetaLayout ml = A.ml;

  // slot lists of chunk c: entry e < kC*LIST is a write slot, the rest read slots; -1 past the list
  auto fetch_idx = [&](int c, int* pf) {
    const int t0 = c * kC, L = min(kC, T - t0);
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int e = tid + k * NT;
      const int rd = e >= kC * LIST, f = rd ? e - kC * LIST : e;
      const int tt = f / LIST, j = f % LIST, n = rd ? R : W;
      int s = -1;
      if (e < 2 * kC * LIST && tt < L && j < n) s = rd ? ridx[(size_t)(t0 + tt) * R + j] : widx[(size_t)(t0 + tt) * W + j];
      pf[k] = s;
    }
  };
  auto store_idx = [&](const int* pf) {
#pragma unroll
    for (int k = 0; k < PF; ++k)
      if (tid + k * NT < 2 * kC * LIST) sidx[tid + k * NT] = pf[k];
  };
  int pf[PF];
  fetch_idx(0, pf);
  store_idx(pf);
  __syncthreads();

  for (int chunk = 0; chunk < A.nchunk; ++chunk) {
    const int t0 = chunk * kC, L = min(kC, T - t0);
    const bool tv = t < L;
    const uint32_t* mb = meta + (size_t)chunk * ml.words;
    // byte offsets of this lane's row pieces (kNoneByte: no row; loads read 0, stores drop)
    uint32_t wo[LIST], ro[LIST];
#pragma unroll
    for (int j = 0; j < LIST; ++j) {
      const int n = sidx[t * LIST + j], m = sidx[kC * LIST + t * LIST + j];
      wo[j] = n >= 0 && n < N ? ((uint32_t)n * (uint32_t)rowdw + (uint32_t)dw) * 4u : kNoneByte;
      ro[j] = m >= 0 && m < N ? ((uint32_t)m * (uint32_t)rowdw + (uint32_t)dw) * 4u : kNoneByte;
    }
    if (chunk + 1 < A.nchunk) fetch_idx(chunk + 1, pf);
    uint32_t mw[LIST], mr[LIST];
#pragma unroll
    for (int j = 0; j < LIST; ++j) mw[j] = __builtin_amdgcn_raw_buffer_load_b32(rM, wo[j], 0, 0);
#pragma unroll
    for (int j = 0; j < LIST; ++j) mr[j] = __builtin_amdgcn_raw_buffer_load_b32(rM, ro[j], 0, 0);
    // per-occurrence coefficients of this token (zeros past the lists and past the chunk)
    float gw[LIST], gr[LIST], wc[LIST], ge[LIST];
    int wb[LIST];
    const uint4* q4 = (const uint4*)(mb + (size_t)t * LIST);
    const size_t occ4 = (size_t)kC * LIST / 4;
#pragma unroll
    for (int j4 = 0; j4 < LIST / 4; ++j4) {
      const uint4 a = q4[ml.gw / 4 + j4], b = q4[ml.gr / 4 + j4], c = q4[ml.wc / 4 + j4], e = q4[ml.ge / 4 + j4],
                  f = q4[ml.wb / 4 + j4];
      gw[4 * j4] = __uint_as_float(a.x), gw[4 * j4 + 1] = __uint_as_float(a.y);
      gw[4 * j4 + 2] = __uint_as_float(a.z), gw[4 * j4 + 3] = __uint_as_float(a.w);
      gr[4 * j4] = __uint_as_float(b.x), gr[4 * j4 + 1] = __uint_as_float(b.y);
      gr[4 * j4 + 2] = __uint_as_float(b.z), gr[4 * j4 + 3] = __uint_as_float(b.w);
      wc[4 * j4] = __uint_as_float(c.x), wc[4 * j4 + 1] = __uint_as_float(c.y);
      wc[4 * j4 + 2] = __uint_as_float(c.z), wc[4 * j4 + 3] = __uint_as_float(c.w);
      ge[4 * j4] = __uint_as_float(e.x), ge[4 * j4 + 1] = __uint_as_float(e.y);
      ge[4 * j4 + 2] = __uint_as_float(e.z), ge[4 * j4 + 3] = __uint_as_float(e.w);
      wb[4 * j4] = (int)f.x, wb[4 * j4 + 1] = (int)f.y, wb[4 * j4 + 2] = (int)f.z, wb[4 * j4 + 3] = (int)f.w;
    }
    (void)occ4;
    const int qs = (int)mb[ml.qp + t], qe = (int)mb[ml.qp + t + 1];
    const int kn = (int)mb[ml.hdr];
    float vv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) vv[c] = 0.f;
    float be = 0.f;
    if (tv) {
      load_v<InT, CPL>(v + (size_t)(t0 + t) * d_v, vv);
      be = beta[t0 + t];
    }
    // P and O0 from the chunk-start rows
    float P[CPL], O0[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) P[c] = O0[c] = 0.f;
#pragma unroll
    for (int j = 0; j < LIST; ++j) {
      float x[CPL], y[CPL];
      RW::unpack(mw[j], x);
      RW::unpack(mr[j], y);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        P[c] = fmaf(gw[j], x[c], P[c]);
        O0[c] = fmaf(gr[j], y[c], O0[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) D[t][d * CPL + c] = be * (vv[c] - P[c]);
    __syncthreads();
    // forward sweep over the K list: delta_t -= beta_t K[t][tau] delta_tau, rows in order
    if (kn > 0) {
      if (tid < NCOL) {
        unsigned long long rows = (unsigned long long)mb[ml.hdr + 2] | (unsigned long long)mb[ml.hdr + 3] << 32;
        while (rows) {
          const int r = __builtin_ctzll(rows);
          rows &= rows - 1;
          const int e0 = (int)mb[ml.kp + r], e1 = (int)mb[ml.kp + r + 1];
          float acc = D[r][tid];
          for (int e = e0; e < e1; ++e) acc = fmaf(-__uint_as_float(mb[ml.ke + 2 * e + 1]), D[mb[ml.ke + 2 * e]][tid], acc);
          D[r][tid] = acc;
        }
      }
      __syncthreads();
    }
    // o = O0 + Q delta
    float dt[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) dt[c] = D[t][d * CPL + c];
    if (tv) {
      for (int e = qs; e < qe; ++e) {
        const int tk = (int)mb[ml.qe + 2 * e];
        const float q = __uint_as_float(mb[ml.qe + 2 * e + 1]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) O0[c] = fmaf(q, D[tk][d * CPL + c], O0[c]);
      }
      if constexpr (CPL == 2) {
        *(float2*)(o + (size_t)(t0 + t) * d_v) = make_float2(O0[0], O0[1]);
      } else {
        o[(size_t)(t0 + t) * d_v] = O0[0];
      }
    }
    // each slot's last writer writes its row back once
#pragma unroll
    for (int j = 0; j < LIST; ++j) {
      if (wb[j] < 0) continue;
      float x[CPL], y[CPL];
      RW::unpack(mw[j], x);
#pragma unroll
      for (int c = 0; c < CPL; ++c) y[c] = fmaf(ge[j], x[c], wc[j] * dt[c]);
      const int e0 = wb[j] >> 8, e1 = e0 + (wb[j] & 255);
      for (int e = e0; e < e1; ++e) {
        const int tk = (int)mb[ml.wl + 2 * e];
        const float a = __uint_as_float(mb[ml.wl + 2 * e + 1]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) y[c] = fmaf(a, D[tk][d * CPL + c], y[c]);
      }
      __builtin_amdgcn_raw_buffer_store_b32(RW::pack(y), rM, wo[j], 0, 0);
    }
    // every lane has read this chunk's slot lists (before the first barrier): the next ones go in
    if (chunk + 1 < A.nchunk) store_idx(pf);
    // the next chunk's gathers read these rows: stores complete, then the barrier
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

template <typename MemT, typename InT, int CBD>
hipError_t launch_apply(const ChunkArgs& A, int list, hipStream_t st) {
  const int wgs = (A.U + kXcd - 1) / kXcd * kXcd * A.ncb;
  const dim3 g((unsigned)wgs), b(64 * CBD);
  if (list == 8) hipLaunchKernelGGL((chunk_apply_kernel<MemT, InT, CBD, 8>), g, b, 0, st, A);
  else if (list == 16) hipLaunchKernelGGL((chunk_apply_kernel<MemT, InT, CBD, 16>), g, b, 0, st, A);
  else hipLaunchKernelGGL((chunk_apply_kernel<MemT, InT, CBD, 32>), g, b, 0, st, A);
  return hipGetLastError();
}

template <typename MemT, typename InT>
hipError_t launch_apply_cbd(ChunkArgs& A, int list, hipStream_t st) {
  constexpr int CPL = RowWord<MemT>::kCols;
  const int rowdw = A.d_v / CPL;
  // widest column block that still gives every compute unit a workgroup
  const int cus = device_cus();
  const long long ug = (A.U + kXcd - 1) / kXcd * kXcd;
  if (ug * (rowdw / 4) >= cus) {
    A.ncb = rowdw / 4;
    return launch_apply<MemT, InT, 4>(A, list, st);
  }
  A.ncb = rowdw / 2;
  return launch_apply<MemT, InT, 2>(A, list, st);
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
  hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)A.nchunk, (unsigned)A.U), dim3(256), 0, stream, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int list = A.ml.list;
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return launch_apply_cbd<uint16_t, uint16_t>(A, list, stream);
  if (mb) return launch_apply_cbd<uint16_t, float>(A, list, stream);
  if (ib) return launch_apply_cbd<float, uint16_t>(A, list, stream);
  return launch_apply_cbd<float, float>(A, list, stream);
}

}  // namespace sdm
