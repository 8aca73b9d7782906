// Dataflow execution of the sparse gated-delta recurrence.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Gated DeltaNet", §3 "Sparse memory
// updates" and "Sparse retrieval"; App. A.2: two tokens interact only through slots they
// share): token t of a (batch, head) unit reads its W write slots, writes them back, and
// reads its R read slots after its write. Two tokens of a unit depend on each other only
// when they share a slot: a later token that touches a slot an earlier token wrote (read
// after write), or a later token that writes a slot an earlier token reads (write after
// read). Tokens that share no slot commute exactly. So the token-heads are run as tasks by
// many waves at once; a task waits only for its earlier conflicting tokens, and the result
// is the same, bit for bit, as processing the tokens in order.
//
// Two kernels:
//   deps_kernel     -- for every token, the set of conflicting tokens among the 128 before
//                      it (a 128-bit mask), and for each read slot its position in the
//                      token's own write list (read-own-write forwarding);
//   dataflow_kernel -- persistent waves claim tasks per unit in token order, wait for their
//                      predecessors (done flags) and for every token more than 64..127
//                      positions back (complete 64-token blocks), then gather, update,
//                      scatter and read whole rows.
//
// Coherence: table rows are loaded and stored with device-scope cache policy (sc1), and
// the flags are device-scope atomics, so a task may run on any CU of any XCD. A task's row
// stores are complete (s_waitcnt vmcnt(0)) before its done flag is set.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kBlk = 64;        // tokens per completion block
constexpr int kWin = 128;       // explicit predecessor window (tokens)
constexpr int kHashBits = 15;   // deps hash table: 32768 entries (128 KB of LDS)
constexpr uint32_t kEmpty = 0xFFFFFFFFu;
// Longest a wave waits (in units of s_sleep 8, about 0.2 us): about 4 s. When it runs out
// the dependency wait is abandoned, the abort flag stops every other wait, the kernel
// drains, and the workspace error word records it (result invalid, never a hang).
constexpr long long kSpinBudget = 1ll << 24;

// ------------------------------------------------------------------ dependency pass
struct DepArgs {
  const int32_t* widx;  // [U][T][W]
  const int32_t* ridx;  // [U][T][R]
  uint64_t* mask;       // [U][T][2]
  int8_t* rmatch;       // [U][T][R]
  int T, W, R;
};

__device__ __forceinline__ uint32_t dep_hash(uint32_t slot) { return (slot * 2654435761u) >> (32 - kHashBits); }

// entry = slot << 9 | (window offset) << 1 | kind (1 = read slot, 0 = write slot)
__global__ void __launch_bounds__(256) deps_kernel(DepArgs A) {
  __shared__ uint32_t table[1 << kHashBits];
  const int u = blockIdx.y;
  const int t0 = blockIdx.x * kBlk;
  const int wlo = t0 - kWin > 0 ? t0 - kWin : 0;  // first token in the window
  const int whi = t0 + kBlk < A.T ? t0 + kBlk : A.T;
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
    const int32_t slot = rd ? ri[(size_t)t * A.R + (p - A.W)] : wi[(size_t)t * A.W + p];
    if (slot < 0) continue;
    const uint32_t ent = ((uint32_t)slot << 9) | ((uint32_t)k << 1) | (rd ? 1u : 0u);
    uint32_t h = dep_hash((uint32_t)slot);
    while (true) {
      uint32_t prev = atomicCAS(&table[h], kEmpty, ent);
      if (prev == kEmpty) break;
      h = (h + 1) & ((1u << kHashBits) - 1);
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = t0 + wave; t < whi; t += 4) {
    const int kt = t - wlo;
    uint64_t m0 = 0, m1 = 0;
    for (int p = lane; p < per; p += 64) {
      const bool rd = p >= A.W;
      const int32_t slot = rd ? ri[(size_t)t * A.R + (p - A.W)] : wi[(size_t)t * A.W + p];
      if (slot < 0) continue;
      uint32_t h = dep_hash((uint32_t)slot);
      while (true) {
        const uint32_t ent = table[h];
        if (ent == kEmpty) break;
        if ((ent >> 9) == (uint32_t)slot) {
          const int k = (ent >> 1) & 0xFF;
          const bool erd = ent & 1u;
          // earlier token; write slots conflict with anything, read slots with writes
          if (k < kt && (!rd || !erd)) {
            const int d = kt - k;  // distance >= 1
            if (d <= 64) m0 |= 1ull << (d - 1);
            else if (d <= kWin) m1 |= 1ull << (d - 65);
          }
        }
        h = (h + 1) & ((1u << kHashBits) - 1);
      }
      if (rd) {
        // position of this read slot in the token's own write list, or -1
        int pos = -1;
        for (int j = 0; j < A.W; ++j)
          if (wi[(size_t)t * A.W + j] == slot) pos = j;
        A.rmatch[((size_t)u * A.T + t) * A.R + (p - A.W)] = (int8_t)pos;
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      m0 |= shfl_xor_u64(m0, s);
      m1 |= shfl_xor_u64(m1, s);
    }
    if (lane == 0) {
      A.mask[((size_t)u * A.T + t) * 2 + 0] = m0;
      A.mask[((size_t)u * A.T + t) * 2 + 1] = m1;
    }
  }
}

// ------------------------------------------------------------------ dataflow recurrence
struct DfArgs {
  const int32_t* widx;
  const float* wgt;
  const int32_t* ridx;
  const float* rgt;
  const uint64_t* mask;
  const int8_t* rmatch;
  const void* v;
  const float* alpha;
  const float* beta;
  void* M;
  float* o;
  int* claim;       // [U] next token to claim
  int* done;        // [U][T] 1 when the token is finished
  int* blkcnt;      // [U][nblk] finished tokens per 64-token block
  int* blkwm;       // [U] number of leading complete blocks
  int* abort_flag;  // set when a wait exceeded its budget: every wave stops waiting and exits
  unsigned long long* err;
  int U, T, W, R, d_v, nblk;
  long long N;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename MemT>
struct RowT;
template <>
struct RowT<float> {
  static constexpr int kEl = 4;  // elements per 16 bytes
  __device__ static void unpack(const u32x4& w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
  __device__ static u32x4 pack(const float* x) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x[i]);
    return w;
  }
};
template <>
struct RowT<uint16_t> {
  static constexpr int kEl = 8;
  __device__ static void unpack(const u32x4& w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo(w[i]);
      x[2 * i + 1] = bf16hi(w[i]);
    }
  }
  __device__ static u32x4 pack(const float* x) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    return w;
  }
};

template <typename InT>
__device__ __forceinline__ float in_at(const InT* p, size_t i);
template <>
__device__ __forceinline__ float in_at<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float in_at<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ int ld_flag(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row access through a buffer resource with device-scope (sc1) cache policy.
constexpr int kSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

// Moves the unit's block watermark past every complete leading block; returns its value.
// Called by the task that completes a block and by tasks waiting on the watermark, so the
// watermark cannot stay behind a complete block.
__device__ int advance_watermark(const DfArgs& A, int u) {
  const int T = A.T;
  int wm = ld_flag(&A.blkwm[u]);
  while (wm < A.nblk) {
    const int bs = (wm + 1) * kBlk <= T ? kBlk : T - wm * kBlk;
    if (ld_flag(&A.blkcnt[(size_t)u * A.nblk + wm]) != bs) break;
    const int seen = atomicCAS(&A.blkwm[u], wm, wm + 1);
    wm = seen == wm ? wm + 1 : seen;
  }
  return wm;
}

// One wave per task. Lane = (row group g, 16-byte column chunk l): LPR lanes cover a row,
// G = 64 / LPR rows per instruction; NR = rows per lane for a list of up to NR*G slots.
template <typename MemT, typename InT, int LPR, int NR>
__global__ void __launch_bounds__(256) dataflow_kernel(DfArgs A) {
  using RT = RowT<MemT>;
  constexpr int EL = RT::kEl;
  constexpr int G = 64 / LPR;
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane / LPR, l = lane % LPR;
  const int W = A.W, R = A.R, T = A.T;
  const int rowbytes = LPR * 16;
  // per-wave LDS: this token's updated write rows, for reads of slots it just wrote
  u32x4* fwd = (u32x4*)(smem + (size_t)wave * W * rowbytes);
  const int gw = blockIdx.x * 4 + wave;
  const int nworkers = gridDim.x * 4;
  const long long N = A.N;
  const uint32_t unit_bytes = (uint32_t)((size_t)N * rowbytes);
  // workers are spread over the units; each worker serves one unit, claiming its tokens in order
  for (int u = gw % A.U; u < A.U; u += nworkers) {
    (void)0;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc((char*)A.M + (size_t)u * unit_bytes, unit_bytes);
    int known_blocks = 0;
    while (true) {
      int t = 0;
      if (lane == 0) t = ld_flag(A.abort_flag) ? T : atomicAdd(&A.claim[u], 1);
      t = __shfl(t, 0, kWave);
      if (t >= T) break;
      const size_t ut = (size_t)u * T + t;
      // --- task inputs (read-only; may be fetched before the wait)
      int nj[NR], mr[NR], fm[NR];
      float aj[NR], ur[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int j = i * G + g;
        nj[i] = j < W ? A.widx[ut * W + j] : -1;
        aj[i] = j < W ? A.wgt[ut * W + j] : 0.f;
        mr[i] = j < R ? A.ridx[ut * R + j] : -1;
        ur[i] = j < R ? A.rgt[ut * R + j] : 0.f;
        fm[i] = j < R ? (int)A.rmatch[ut * R + j] : -1;
      }
      const float al = A.alpha[ut], be = A.beta[ut];
      float vv[EL];
#pragma unroll
      for (int c = 0; c < EL; ++c) vv[c] = in_at<InT>((const InT*)A.v, ut * A.d_v + (size_t)l * EL + c);
      const uint64_t m0 = A.mask[ut * 2], m1 = A.mask[ut * 2 + 1];
      // --- wait: every token before the previous 64-token block is done, and every
      //     conflicting token among the last 128
      const int need_blocks = t / kBlk - 1;
      bool aborted = false;
      if (need_blocks > known_blocks) {
        int naps = 1;
        long long budget = kSpinBudget;
        while (true) {
          int wm = 0, ab = 0;
          if (lane == 0) {
            wm = advance_watermark(A, u);
            ab = ld_flag(A.abort_flag);
          }
          wm = __shfl(wm, 0, kWave);
          ab = __shfl(ab, 0, kWave);
          if (wm >= need_blocks) { known_blocks = wm; break; }
          if (ab || budget <= 0) { aborted = true; break; }
          for (int z = 0; z < naps; ++z) __builtin_amdgcn_s_sleep(8);
          budget -= naps;
          naps = naps < 16 ? naps * 2 : 16;
        }
      }
      if (!aborted) {
        // lane d waits for token t-1-d (mask word 0) and t-65-d (mask word 1)
        const bool p0 = (m0 >> lane) & 1ull, p1 = (m1 >> lane) & 1ull;
        long long budget = kSpinBudget;
        bool stop = false;
        while (!stop) {
          const bool w0 = p0 && ld_flag(&A.done[ut - 1 - lane]) == 0;
          const bool w1 = p1 && ld_flag(&A.done[ut - 65 - lane]) == 0;
          if (ballot(w0 || w1) == 0ull) break;
          if (budget <= 0 || __shfl(lane == 0 ? ld_flag(A.abort_flag) : 0, 0, kWave)) { aborted = true; break; }
          __builtin_amdgcn_s_sleep(8);
          budget -= 1;
        }
      }
      if (aborted) {
        if (lane == 0) {
          st_flag(A.abort_flag, 1);
          atomicAdd(A.err, 1ull << 40);
        }
        break;
      }
      __builtin_amdgcn_wave_barrier();
      __asm__ __volatile__("" ::: "memory");
      // --- gather write rows and read rows (device-coherent loads)
      u32x4 wrow[NR], rrow[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const bool okw = nj[i] >= 0 && nj[i] < N;
        const bool okr = mr[i] >= 0 && mr[i] < N;
        wrow[i] = okw ? __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)nj[i] * rowbytes + l * 16, 0, kSc1)
                      : u32x4{0, 0, 0, 0};
        rrow[i] = okr ? __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)mr[i] * rowbytes + l * 16, 0, kSc1)
                      : u32x4{0, 0, 0, 0};
      }
      // --- decayed weighted read of the write slots, reduced over row groups
      float acc[EL];
#pragma unroll
      for (int c = 0; c < EL; ++c) acc[c] = 0.f;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        float x[EL];
        RT::unpack(wrow[i], x);
#pragma unroll
        for (int c = 0; c < EL; ++c) acc[c] = fmaf(aj[i], x[c], acc[c]);
      }
#pragma unroll
      for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
        for (int c = 0; c < EL; ++c) acc[c] += shfl_xor_f32(acc[c], s);
      float dl[EL];
#pragma unroll
      for (int c = 0; c < EL; ++c) dl[c] = be * (vv[c] - al * acc[c]);
      // --- gated delta write of the W slots
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int j = i * G + g;
        if (j < W) {
          float x[EL], y[EL];
          RT::unpack(wrow[i], x);
#pragma unroll
          for (int c = 0; c < EL; ++c) y[c] = fmaf(al, x[c], aj[i] * dl[c]);
          const u32x4 nw = RT::pack(y);
          fwd[j * LPR + l] = nw;
          if (nj[i] >= 0 && nj[i] < N)
            __builtin_amdgcn_raw_buffer_store_b128(nw, rs, (uint32_t)nj[i] * rowbytes + l * 16, 0, kSc1);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // --- weighted read of the R slots after the write
      float ov[EL];
#pragma unroll
      for (int c = 0; c < EL; ++c) ov[c] = 0.f;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const u32x4 w = fm[i] >= 0 ? fwd[fm[i] * LPR + l] : rrow[i];
        float x[EL];
        RT::unpack(w, x);
#pragma unroll
        for (int c = 0; c < EL; ++c) ov[c] = fmaf(ur[i], x[c], ov[c]);
      }
#pragma unroll
      for (int s = LPR; s < 64; s <<= 1)
#pragma unroll
        for (int c = 0; c < EL; ++c) ov[c] += shfl_xor_f32(ov[c], s);
      if (g == 0) {
        float* op = A.o + ut * A.d_v + (size_t)l * EL;
#pragma unroll
        for (int c = 0; c < EL; ++c) op[c] = ov[c];
      }
      // slot indices outside [0, N) were skipped; count them once per task
      {
        int bad = 0;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const int j = i * G + g;
          const bool bw = l == 0 && j < W && (nj[i] < 0 || nj[i] >= N);
          const bool br = l == 0 && j < R && (mr[i] < 0 || mr[i] >= N);
          bad += popc64(ballot(bw)) + popc64(ballot(br));
        }
        if (bad && lane == 0) atomicAdd(A.err, (unsigned long long)bad);
      }
      // --- publish: stores complete, then the done flag and the block count
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) {
        st_flag(&A.done[ut], 1);
        const int b = t / kBlk;
        const int bsize = (b + 1) * kBlk <= T ? kBlk : T - b * kBlk;
        const int prev = atomicAdd(&A.blkcnt[(size_t)u * A.nblk + b], 1);
        if (prev + 1 == bsize) advance_watermark(A, u);  // this task completed block b
      }
    }
  }
}

template <typename MemT, typename InT, int LPR>
hipError_t df_launch_nr(const DfArgs& A, int nr, hipStream_t st, int cus) {
  const int rowbytes = LPR * 16;
  const size_t lds = (size_t)4 * A.W * rowbytes;
  auto go = [&](auto kern) -> hipError_t {
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    int grid = per_cu * cus;
    // no more workers than tasks, and per unit no more than the tokens that can be in flight
    long long cap = (long long)A.U * (A.T < kWin + kBlk ? A.T : kWin + kBlk);
    cap = (cap + 3) / 4;
    if (grid > cap) grid = (int)(cap < 1 ? 1 : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, A);
    return hipGetLastError();
  };
  if (nr <= 1) return go(dataflow_kernel<MemT, InT, LPR, 1>);
  if (nr <= 2) return go(dataflow_kernel<MemT, InT, LPR, 2>);
  if (nr <= 4) return go(dataflow_kernel<MemT, InT, LPR, 4>);
  return go(dataflow_kernel<MemT, InT, LPR, 8>);
}

template <typename MemT, typename InT>
hipError_t df_launch_lpr(const DfArgs& A, hipStream_t st, int cus) {
  const int rowbytes = A.d_v * (int)sizeof(MemT);
  const int lpr = rowbytes / 16;
  const int G = 64 / lpr;
  const int nr = (((A.W > A.R ? A.W : A.R) + G - 1) / G);
  switch (lpr) {
    case 1: return df_launch_nr<MemT, InT, 1>(A, nr, st, cus);
    case 2: return df_launch_nr<MemT, InT, 2>(A, nr, st, cus);
    case 4: return df_launch_nr<MemT, InT, 4>(A, nr, st, cus);
    case 8: return df_launch_nr<MemT, InT, 8>(A, nr, st, cus);
    case 16: return df_launch_nr<MemT, InT, 16>(A, nr, st, cus);
    case 32: return df_launch_nr<MemT, InT, 32>(A, nr, st, cus);
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

// Row layouts the dataflow kernel handles: rows of 16..512 bytes in a power of two with at
// most 8 rows of each slot list per lane.
bool dataflow_supported(const sdm_shape& S) {
  const int rowbytes = S.d_v * (int)dtype_size(S.mem_dtype);
  if (rowbytes < 16 || rowbytes > 512 || (rowbytes & (rowbytes - 1))) return false;
  const int G = 64 / (rowbytes / 16);
  const int mx = S.W > S.R ? S.W : S.R;
  if ((mx + G - 1) / G > 8) return false;
  if ((size_t)S.N * rowbytes > 0xFFFFFFFFull) return false;
  if ((size_t)4 * S.W * rowbytes > 64 * 1024) return false;
  if (S.W + S.R > 128) return false;  // dependency hash table load
  return true;
}

size_t dataflow_deps_bytes(const sdm_shape& S) {
  const size_t tok = (size_t)S.B * S.H * S.T;
  return tok * 16 + tok * (size_t)S.R;
}

size_t dataflow_sched_words(const sdm_shape& S) {
  const size_t U = (size_t)S.B * S.H;
  const size_t nblk = ((size_t)S.T + kBlk - 1) / kBlk;
  return U + U * S.T + U * nblk + U + 1;  // claim, done, blkcnt, blkwm, abort (int32 each)
}

hipError_t launch_dataflow(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                           const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                           void* ws, const WsLayout& L, hipStream_t stream) {
  const int U = S.B * S.H;
  char* w = (char*)ws;
  const size_t tok = (size_t)U * S.T;
  uint64_t* mask = (uint64_t*)(w + L.deps);
  int8_t* rmatch = (int8_t*)(w + L.deps + tok * 16);
  int* sched = (int*)(w + L.sched);
  const size_t words = dataflow_sched_words(S);
  hipError_t e = launch_zero(sched, (words * 4 + 7) / 8, stream);
  if (e != hipSuccess) return e;
  DepArgs D;
  D.widx = widx;
  D.ridx = ridx;
  D.mask = mask;
  D.rmatch = rmatch;
  D.T = S.T;
  D.W = S.W;
  D.R = S.R;
  hipLaunchKernelGGL(deps_kernel, dim3((S.T + kBlk - 1) / kBlk, U), dim3(256), 0, stream, D);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  DfArgs A;
  A.widx = widx;
  A.wgt = wgt;
  A.ridx = ridx;
  A.rgt = rgt;
  A.mask = mask;
  A.rmatch = rmatch;
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  A.M = M;
  A.o = o;
  A.nblk = (S.T + kBlk - 1) / kBlk;
  A.claim = sched;
  A.done = sched + U;
  A.blkcnt = A.done + (size_t)U * S.T;
  A.blkwm = A.blkcnt + (size_t)U * A.nblk;
  A.abort_flag = A.blkwm + U;
  A.err = (unsigned long long*)(w + L.err);
  A.U = U;
  A.T = S.T;
  A.W = S.W;
  A.R = S.R;
  A.d_v = S.d_v;
  A.N = S.N;
  const int cus = device_cus();
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return df_launch_lpr<uint16_t, uint16_t>(A, stream, cus);
  if (mb && !ib) return df_launch_lpr<uint16_t, float>(A, stream, cus);
  if (!mb && ib) return df_launch_lpr<float, uint16_t>(A, stream, cus);
  return df_launch_lpr<float, float>(A, stream, cus);
}

}  // namespace sdm
