// Dataflow execution of the sparse gated-delta recurrence, one workgroup per (unit, column
// block).
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Gated DeltaNet", §3 "Sparse memory
// updates" and "Sparse retrieval"; App. A.2: two tokens interact only through the slots
// they share): token t of a (batch, head) unit reads its W write slots, writes them back,
// and reads its R read slots after its write. Two facts make this parallel without changing
// the result:
//   * every column of the table evolves on its own given the slots and weights, so a unit's
//     rows are split into P column blocks handled by P independent workgroups;
//   * two tokens depend on each other only when they share a slot (a later token touching a
//     slot an earlier one wrote, or writing a slot an earlier one reads); tokens that share
//     no slot commute exactly.
// Inside a workgroup, waves claim tokens in order and run them as soon as their conflicting
// predecessors among the last kWin tokens have published their written rows in an LDS ring;
// rows written earlier than that come from the table in HBM. The result is bit-identical to
// processing the tokens one after another.
//
// deps_kernel precomputes, per token: a kWin-bit mask of conflicting earlier tokens, and per
// slot the most recent writer inside the window (distance, position) -- or none.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kWin = 32;            // explicit dependency / forwarding window (tokens)
constexpr int kRing = 2 * kWin;     // LDS ring of the written row blocks of recent tokens
constexpr int kDepBlk = 64;         // tokens per deps workgroup
constexpr int kHashBits = 14;       // deps hash table: 16384 entries, (kDepBlk + kWin) * (W + R) used
constexpr uint32_t kEmpty = 0xFFFFFFFFu;
constexpr int kWaves = 16;          // waves per workgroup of the recurrence
// Longest a wave waits (in units of s_sleep 2): about 3 s. When it runs out the workgroup
// gives up (abort flag), every wave exits, and the workspace error word records it: the
// result is then invalid, but the kernel always terminates.
constexpr long long kSpinBudget = 1ll << 26;

// ------------------------------------------------------------------ dependency pass
struct DepArgs {
  const int32_t* widx;  // [U][T][W]
  const int32_t* ridx;  // [U][T][R]
  uint32_t* mask;       // [U][T]: bit d-1 set -> token t-d conflicts with t (1 <= d <= kWin)
  int16_t* code;        // [U][T][W+R]: (d << 7) | j of the latest writer t-d at position j, or -1
  int T, W, R;
};

__device__ __forceinline__ uint32_t dep_hash(uint32_t slot) { return (slot * 2654435761u) >> (32 - kHashBits); }

// entry = slot << 14 | window offset << 7 | kind << 6 | position (kind 1 = read slot)
__global__ void __launch_bounds__(256) deps_kernel(DepArgs A) {
  __shared__ uint32_t table[1 << kHashBits];
  const int u = blockIdx.y;
  const int t0 = blockIdx.x * kDepBlk;
  const int wlo = t0 - kWin > 0 ? t0 - kWin : 0;
  const int whi = t0 + kDepBlk < A.T ? t0 + kDepBlk : A.T;
  const int ntok = whi - wlo;
  const int per = A.W + A.R;
  for (int i = threadIdx.x; i < (1 << kHashBits); i += 256) table[i] = kEmpty;
  __syncthreads();
  const int32_t* wi = A.widx + (size_t)u * A.T * A.W;
  const int32_t* ri = A.ridx + (size_t)u * A.T * A.R;
  for (int e = threadIdx.x; e < ntok * per; e += 256) {
    const int k = e / per, p = e % per;
    const int t = wlo + k;
    const bool rd = p >= A.W;
    const int j = rd ? p - A.W : p;
    const int32_t slot = rd ? ri[(size_t)t * A.R + j] : wi[(size_t)t * A.W + j];
    if (slot < 0) continue;
    const uint32_t ent = ((uint32_t)slot << 14) | ((uint32_t)k << 7) | (rd ? 64u : 0u) | (uint32_t)j;
    uint32_t h = dep_hash((uint32_t)slot);
    while (atomicCAS(&table[h], kEmpty, ent) != kEmpty) h = (h + 1) & ((1u << kHashBits) - 1);
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = t0 + wave; t < whi; t += 4) {
    const int kt = t - wlo;
    uint32_t m = 0;
    for (int p = lane; p < per; p += 64) {
      const bool rd = p >= A.W;
      const int32_t slot = rd ? ri[(size_t)t * A.R + (p - A.W)] : wi[(size_t)t * A.W + p];
      int best = -1, bestj = 0;
      if (slot >= 0) {
        uint32_t h = dep_hash((uint32_t)slot);
        while (true) {
          const uint32_t ent = table[h];
          if (ent == kEmpty) break;
          if ((ent >> 14) == (uint32_t)slot) {
            const int k = (ent >> 7) & 127;
            const bool erd = (ent >> 6) & 1u;
            const int d = kt - k;
            // conflicts: a write slot with any earlier slot use, a read slot with an earlier write
            if (d >= 1 && d <= kWin && (!rd || !erd)) m |= 1u << (d - 1);
            // latest writer: earlier token, or this token itself for a read slot
            if (!erd && d <= kWin && (d >= 1 || (rd && d == 0)) && k > best) {
              best = k;
              bestj = ent & 63;
            }
          }
          h = (h + 1) & ((1u << kHashBits) - 1);
        }
      }
      A.code[((size_t)u * A.T + t) * per + p] = best < 0 ? (int16_t)-1 : (int16_t)(((kt - best) << 7) | bestj);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m |= shfl_xor_u32(m, s);
    if (lane == 0) A.mask[(size_t)u * A.T + t] = m;
  }
}

// ------------------------------------------------------------------ recurrence
struct CsArgs {
  const int32_t* widx;
  const float* wgt;
  const int32_t* ridx;
  const float* rgt;
  const uint32_t* mask;
  const int16_t* code;
  const void* v;
  const float* alpha;
  const float* beta;
  void* M;
  float* o;
  unsigned long long* err;
  int U, T, W, R, d_v, P;  // P column blocks per unit
  long long N;
};

template <typename MemT>
struct Word;  // one 32-bit word of a row: 1 float32 or 2 bf16 columns
template <>
struct Word<float> {
  static constexpr int kCols = 1;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = __uint_as_float(w); }
  __device__ static uint32_t pack(const float* x) { return __float_as_uint(x[0]); }
};
template <>
struct Word<uint16_t> {
  static constexpr int kCols = 2;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = bf16lo(w); x[1] = bf16hi(w); }
  __device__ static uint32_t pack(const float* x) { return pack_bf16x2(x[0], x[1]); }
};

template <typename InT>
__device__ __forceinline__ float in_at(const InT* p, size_t i);
template <>
__device__ __forceinline__ float in_at<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float in_at<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ int lds_ld(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Workgroup = kWaves waves serving one (unit, column block). Lane = (row group g, word l):
// LPR lanes (one 32-bit word each) cover the block's part of a row, G = 64/LPR rows per
// instruction, NR row instructions per slot list.
template <typename MemT, typename InT, int LPR, int NR>
__global__ void __launch_bounds__(kWaves * 64) recurrence_kernel(CsArgs A) {
  using WT = Word<MemT>;
  constexpr int CPW = WT::kCols;  // columns per word
  constexpr int G = 64 / LPR;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int fwd_tok[kRing];   // token whose written rows sit in ring slot i
  __shared__ int done_tok[kRing];  // token whose table stores are complete
  __shared__ int claim, wm, abort_wg;

  const int W = A.W, R = A.R, T = A.T;
  const int lane = threadIdx.x & 63;
  const int g = lane / LPR, l = lane % LPR;
  // XCD-aware placement: all column blocks of a unit go to the same XCD (workgroups are
  // dealt to the 8 XCDs round-robin), so they share its L2 for rows and per-token inputs.
  const int xcd = blockIdx.x & 7, kb = blockIdx.x >> 3;
  const int u = xcd + 8 * (kb / A.P);
  const int cb = kb % A.P;
  if (u >= A.U) return;

  uint32_t* ring = (uint32_t*)smem;  // [kRing][W][LPR] words
  const int rowdw = A.d_v / CPW;      // words per table row
  uint32_t* Mu = (uint32_t*)A.M + (size_t)u * (size_t)A.N * rowdw + (size_t)cb * LPR + l;
  const int col0 = (cb * LPR + l) * CPW;  // first column of this lane
  const long long N = A.N;
  const int per = W + R;

  for (int i = threadIdx.x; i < kRing; i += blockDim.x) {
    fwd_tok[i] = -1;
    done_tok[i] = -1;
  }
  if (threadIdx.x == 0) {
    claim = 0;
    wm = 0;
    abort_wg = 0;
  }
  __syncthreads();

  while (true) {
    int t = 0;
    if (lane == 0) t = atomicAdd(&claim, 1);
    t = __shfl(t, 0, kWave);
    if (t >= T || lds_ld(&abort_wg)) break;
    const size_t ut = (size_t)u * T + t;
    // ---- per-token inputs
    int nj[NR], mr[NR], cw[NR], cr[NR];
    float aj[NR], ur[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = i * G + g;
      nj[i] = j < W ? A.widx[ut * W + j] : -1;
      aj[i] = j < W ? A.wgt[ut * W + j] : 0.f;
      cw[i] = j < W ? (int)A.code[ut * per + j] : -1;
      mr[i] = j < R ? A.ridx[ut * R + j] : -1;
      ur[i] = j < R ? A.rgt[ut * R + j] : 0.f;
      cr[i] = j < R ? (int)A.code[ut * per + W + j] : -1;
    }
    const float al = A.alpha[ut], be = A.beta[ut];
    float vv[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) vv[c] = in_at<InT>((const InT*)A.v, ut * A.d_v + col0 + c);
    const uint32_t pm = A.mask[ut];
    // ---- wait 1: every token up to t-kWin has finished (its ring slot may be reused and
    //      its table stores are visible), and the conflicting tokens of the window have
    //      published their written rows
    {
      long long budget = kSpinBudget;
      bool ok = true;
      while (lds_ld(&wm) < t - kWin + 1) {
        if (--budget <= 0 || lds_ld(&abort_wg)) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      const bool mine = lane < kWin && ((pm >> lane) & 1u);
      const int pt = t - 1 - lane;
      while (ok) {
        const bool wait = mine && lds_ld(&fwd_tok[pt & (kRing - 1)]) != pt;
        if (ballot(wait) == 0ull) break;
        if (--budget <= 0 || lds_ld(&abort_wg)) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (!ok) {
        if (lane == 0) {
          lds_st(&abort_wg, 1);
          atomicAdd(A.err, 1ull << 40);
        }
        break;
      }
    }
    // no ring or table read may move above the waits
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // ---- gather: rows written inside the window come from the ring, others from the table
    uint32_t wv[NR], rv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = i * G + g;
      uint32_t x = 0;
      if (j < W) {
        if (cw[i] >= 0) {
          const int d = cw[i] >> 7, jj = cw[i] & 127;
          x = ring[(((t - d) & (kRing - 1)) * W + jj) * LPR + l];
        } else if (nj[i] >= 0 && nj[i] < N) {
          x = Mu[(size_t)nj[i] * rowdw];
        }
      }
      wv[i] = x;
      uint32_t y = 0;
      if (j < R && cr[i] < 0 && mr[i] >= 0 && mr[i] < N) y = Mu[(size_t)mr[i] * rowdw];
      rv[i] = y;
    }
    // ---- decayed weighted read of the write slots
    float acc[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      float x[CPW];
      WT::unpack(wv[i], x);
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] = fmaf(aj[i], x[c], acc[c]);
    }
#pragma unroll
    for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] += shfl_xor_f32(acc[c], s);
    float dl[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) dl[c] = be * (vv[c] - al * acc[c]);
    // ---- gated delta write: new rows into this token's ring slot
    uint32_t* mine_ring = ring + (size_t)(t & (kRing - 1)) * W * LPR;
    uint32_t nwv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = i * G + g;
      float x[CPW], y[CPW];
      WT::unpack(wv[i], x);
#pragma unroll
      for (int c = 0; c < CPW; ++c) y[c] = fmaf(al, x[c], aj[i] * dl[c]);
      nwv[i] = WT::pack(y);
      if (j < W) mine_ring[j * LPR + l] = nwv[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) lds_st(&fwd_tok[t & (kRing - 1)], t);
    // ---- the table stores wait for the conflicting tokens' own stores (write after write)
    {
      long long budget = kSpinBudget;
      const bool mine = lane < kWin && ((pm >> lane) & 1u);
      const int pt = t - 1 - lane;
      bool ok = true;
      while (true) {
        const bool wait = mine && lds_ld(&done_tok[pt & (kRing - 1)]) != pt;
        if (ballot(wait) == 0ull) break;
        if (--budget <= 0 || lds_ld(&abort_wg)) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (!ok) {
        if (lane == 0) {
          lds_st(&abort_wg, 1);
          atomicAdd(A.err, 1ull << 40);
        }
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = i * G + g;
      if (j < W && nj[i] >= 0 && nj[i] < N) Mu[(size_t)nj[i] * rowdw] = nwv[i];
    }
    // ---- weighted read of the R slots after the write
    float ov[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) ov[c] = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      uint32_t x = rv[i];
      if (cr[i] >= 0) {
        const int d = cr[i] >> 7, jj = cr[i] & 127;
        x = ring[(((t - d) & (kRing - 1)) * W + jj) * LPR + l];
      }
      float y[CPW];
      WT::unpack(x, y);
#pragma unroll
      for (int c = 0; c < CPW; ++c) ov[c] = fmaf(ur[i], y[c], ov[c]);
    }
#pragma unroll
    for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
      for (int c = 0; c < CPW; ++c) ov[c] += shfl_xor_f32(ov[c], s);
    if (g == 0) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) A.o[ut * A.d_v + col0 + c] = ov[c];
    }
    // slot indices outside [0, N) were skipped; the first column block counts them
    if (cb == 0) {
      int bad = 0;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int j = i * G + g;
        bad += popc64(ballot(l == 0 && j < W && (nj[i] < 0 || nj[i] >= N)));
        bad += popc64(ballot(l == 0 && j < R && (mr[i] < 0 || mr[i] >= N)));
      }
      if (bad && lane == 0) atomicAdd(A.err, (unsigned long long)bad);
    }
    // ---- finished: table stores complete, then publish and advance the watermark
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) {
      lds_st(&done_tok[t & (kRing - 1)], t);
      int w = lds_ld(&wm);
      while (w < T && lds_ld(&done_tok[w & (kRing - 1)]) == w) {
        const int seen = atomicCAS(&wm, w, w + 1);
        w = seen == w ? w + 1 : seen;
      }
    }
  }
}

template <typename MemT, typename InT, int LPR>
hipError_t cs_launch_nr(const CsArgs& A, int nr, hipStream_t st) {
  const size_t lds = (size_t)kRing * A.W * LPR * 4;
  const int groups = (A.U + 7) / 8;
  dim3 grid(8 * groups * A.P);
  dim3 block(kWaves * 64);
  if (nr <= 1) hipLaunchKernelGGL((recurrence_kernel<MemT, InT, LPR, 1>), grid, block, lds, st, A);
  else if (nr <= 2) hipLaunchKernelGGL((recurrence_kernel<MemT, InT, LPR, 2>), grid, block, lds, st, A);
  else if (nr <= 4) hipLaunchKernelGGL((recurrence_kernel<MemT, InT, LPR, 4>), grid, block, lds, st, A);
  else hipLaunchKernelGGL((recurrence_kernel<MemT, InT, LPR, 8>), grid, block, lds, st, A);
  return hipGetLastError();
}

template <typename MemT, typename InT>
hipError_t cs_launch_lpr(const CsArgs& A, int lpr, hipStream_t st) {
  const int G = 64 / lpr;
  const int mx = A.W > A.R ? A.W : A.R;
  const int nr = (mx + G - 1) / G;
  switch (lpr) {
    case 2: return cs_launch_nr<MemT, InT, 2>(A, nr, st);
    case 4: return cs_launch_nr<MemT, InT, 4>(A, nr, st);
    case 8: return cs_launch_nr<MemT, InT, 8>(A, nr, st);
    case 16: return cs_launch_nr<MemT, InT, 16>(A, nr, st);
    default: return hipErrorInvalidValue;
  }
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  return cus;
}

}  // namespace

// Words per column block: split each row into P blocks of LPR 32-bit words (LPR in 2..16),
// aiming at about one workgroup per CU over all units.
int dataflow_lanes_per_row(const sdm_shape& S, int cus) {
  const int rowdw = S.d_v * (int)dtype_size(S.mem_dtype) / 4;
  const int U = S.B * S.H;
  int best = -1;
  for (int lpr = 16; lpr >= 2; lpr >>= 1) {
    if (rowdw % lpr) continue;
    const int G = 64 / lpr;
    const int mx = S.W > S.R ? S.W : S.R;
    if ((mx + G - 1) / G > 8) continue;
    if ((size_t)kRing * S.W * lpr * 4 > 64 * 1024) continue;
    best = lpr;
    if ((long long)U * (rowdw / lpr) >= cus) break;  // enough workgroups: keep blocks wide
  }
  return best;
}

bool dataflow_supported(const sdm_shape& S) {
  if (S.W + S.R > 128) return false;
  if (S.N > (1 << 18)) return false;  // deps table packs slots in 18 bits
  return dataflow_lanes_per_row(S, 256) > 0;
}

size_t dataflow_deps_bytes(const sdm_shape& S) {
  const size_t tok = (size_t)S.B * S.H * S.T;
  return tok * 4 + ((tok * (size_t)(S.W + S.R) * 2 + 255) & ~(size_t)255);
}

size_t dataflow_sched_words(const sdm_shape& S) {
  (void)S;
  return 0;
}

hipError_t launch_dataflow(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                           const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                           void* ws, const WsLayout& L, hipStream_t stream) {
  const int U = S.B * S.H;
  char* w = (char*)ws;
  const size_t tok = (size_t)U * S.T;
  int16_t* code = (int16_t*)(w + L.deps);
  uint32_t* mask = (uint32_t*)(w + L.deps + ((tok * (size_t)(S.W + S.R) * 2 + 255) & ~(size_t)255));
  DepArgs D;
  D.widx = widx;
  D.ridx = ridx;
  D.mask = mask;
  D.code = code;
  D.T = S.T;
  D.W = S.W;
  D.R = S.R;
  hipLaunchKernelGGL(deps_kernel, dim3((S.T + kDepBlk - 1) / kDepBlk, U), dim3(256), 0, stream, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int lpr = dataflow_lanes_per_row(S, device_cus());
  CsArgs A;
  A.widx = widx;
  A.wgt = wgt;
  A.ridx = ridx;
  A.rgt = rgt;
  A.mask = mask;
  A.code = code;
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  A.M = M;
  A.o = o;
  A.err = (unsigned long long*)(w + L.err);
  A.U = U;
  A.T = S.T;
  A.W = S.W;
  A.R = S.R;
  A.d_v = S.d_v;
  A.N = S.N;
  const int rowdw = S.d_v * (int)dtype_size(S.mem_dtype) / 4;
  A.P = rowdw / lpr;
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return cs_launch_lpr<uint16_t, uint16_t>(A, lpr, stream);
  if (mb && !ib) return cs_launch_lpr<uint16_t, float>(A, lpr, stream);
  if (!mb && ib) return cs_launch_lpr<float, uint16_t>(A, lpr, stream);
  return cs_launch_lpr<float, float>(A, lpr, stream);
}

}  // namespace sdm
