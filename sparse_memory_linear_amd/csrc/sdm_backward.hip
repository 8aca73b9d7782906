// Memory-efficient backward of the sparse gated-delta recurrence (written-rows rule).
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, App. A.3 "Memory-Efficient
// Backward": the forward applies its sparse updates in place and the backward undoes them,
// so memory stays O(N d + T W d) instead of a table copy per chunk). The forward logs the
// pre-update values x_j of each token's W write rows; the backward walks the tokens in
// reverse with G, the gradient of the loss with respect to the current table:
//   read (after the write): du_r = <go_t, M[m_r]>;  G[m_r] += u_r go_t
//   write: s = sum_j a_j x_j, rho = alpha s, delta = beta (v - rho), dy_j = G[n_j]
//          d delta = sum_j a_j dy_j;  dv = beta d delta;  d rho = -beta d delta
//          da_j = <dy_j, delta> + alpha <d rho, x_j>
//          dalpha = sum_j <dy_j, x_j> + <d rho, s>;  dbeta = <d delta, v - rho>
//          G[n_j] = alpha dy_j + alpha a_j d rho
//   undo:  M[n_j] = x_j
//
// Every column of the table and of G evolves on its own, and two tokens interact only
// through a slot they share. A workgroup owns C columns of one unit; its K waves take the
// tokens in reverse, wave w the tokens T-1-w, T-1-w-K, ... A token starts once every later
// token that shares a slot with it has finished (at most K-1 of them can still be running;
// the preparation pass lists them per token as a bit mask) and every token K or more later
// has finished; a wave publishes a finished token in an LDS ring once its stores are
// complete. Inside a wave, NG row groups of C = 64 / NG lanes hold the same C columns and
// split the token's rows (up to 8 write and 8 read rows per group); only the sums over rows
// (s and d delta) cross between groups.
//
// Each token issues all of its row loads at once. The read-write coupling inside a token (a
// read slot that is also written: its G update must land before the write consumes G) is
// resolved by tables from the preparation pass instead of through memory: wadd_j, the sum
// of u_r over the reads of slot n_j, is folded into dy_j, and only reads of slots the token
// does not write store G (the first of equal read slots, carrying their summed weight).
// Slot lists and tables are fetched two own tokens ahead; the sums over columns (weight,
// alpha and beta gradients) go through LDS and shuffles and are added across column blocks
// with atomics into outputs zeroed first.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kMaxSel = 64;        // W, R <= 64
constexpr int kXcd = 8;            // workgroups are dealt round-robin to this many L2 domains
constexpr uint32_t kNone = 0x1FFFFFFCu;  // element index of a row that touches nothing: its
                                         // byte offset (x 2 or 4) lies past every table
constexpr int kMaxWaves = 16;      // waves per workgroup (K)
constexpr int kFinRing = 128;      // finished-token ring (> 4 K: a token waits on at most
                                   // 2K - 1 later tokens, none older than 2K is running)
constexpr int kPrepBlk = 16;       // tokens per preparation workgroup
// Longest a wave waits for another (in units of s_sleep 1, ~27 ns): about 3.6 s. When it
// runs out the workgroup gives up, every wave exits, and the error word counts it.
constexpr long long kSpinBudget = 1ll << 27;

// Row traffic goes through buffer instructions on per-unit resources: a 32-bit byte offset
// per row (one register) instead of a 64-bit address. Loads return the raw bits (bf16 in
// the low half), so that no use of a load has to wait before the token's other loads are
// issued; cvt() turns them into a float.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rs(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(uint32_t)bytes, 0x00020000);
}
template <typename T>
__device__ __forceinline__ uint32_t bld(rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(T) == 2) return __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
}
template <typename T>
__device__ __forceinline__ void bst(rsrc_t rs, uint32_t off, float x) {
  if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pack_bf16x2(x, 0.f), rs, off, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, off, 0, 0);
}
template <typename T>
__device__ __forceinline__ float cvt(uint32_t r) {
  if constexpr (sizeof(T) == 2) return __uint_as_float(r << 16);
  else return __uint_as_float(r);
}
// CW consecutive values of T (CW = 1 or 2) as raw words: a bf16 pair in one word, float32
// values one word each; loaded and stored in one buffer instruction.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <typename T, int CW>
struct Wide {
  static constexpr int kN = CW == 1 || sizeof(T) == 2 ? 1 : 2;
  __device__ static void ld(rsrc_t rs, uint32_t off, uint32_t* w) {
    if constexpr (CW == 1) {
      w[0] = bld<T>(rs, off);
    } else if constexpr (sizeof(T) == 2) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
    } else {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
      w[0] = x.x, w[1] = x.y;
    }
  }
  __device__ static float val(const uint32_t* w, int k) {
    if constexpr (CW == 1) return cvt<T>(w[0]);
    else if constexpr (sizeof(T) == 2) return k == 0 ? __uint_as_float(w[0] << 16) : __uint_as_float(w[0] & 0xFFFF0000u);
    else return __uint_as_float(w[k]);
  }
  __device__ static void st_raw(rsrc_t rs, uint32_t off, const uint32_t* w) {
    if constexpr (CW == 1 || sizeof(T) == 2) {
      if constexpr (CW == 1 && sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w[0], rs, off, 0, 0);
      else __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, off, 0, 0);
    } else {
      u32x2 x;
      x.x = w[0], x.y = w[1];
      __builtin_amdgcn_raw_buffer_store_b64(x, rs, off, 0, 0);
    }
  }
};
template <int CW>
__device__ __forceinline__ void st_f32w(rsrc_t rs, uint32_t off, const float* v) {
  if constexpr (CW == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), rs, off, 0, 0);
  } else {
    u32x2 x;
    x.x = __float_as_uint(v[0]), x.y = __float_as_uint(v[1]);
    __builtin_amdgcn_raw_buffer_store_b64(x, rs, off, 0, 0);
  }
}

__device__ __forceinline__ int lds_ld(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ------------------------------------------------------------------ preparation pass
// Per token: dep, bit i set if token t+1+i (i < win) shares a slot with it; rst, bit r set
// if read r stores G; wadd[j] and rc[r] (the coupling tables). An LDS hash of every slot of
// the block's tokens and the win tokens after them (key: slot; info: token offset, kind,
// position) answers each (token, position) by one probe sequence.
struct PrepArgs {
  const int32_t* widx;  // [U][T][W]
  const int32_t* ridx;  // [U][T][R]
  const float* rgt;     // [U][T][R]
  uint32_t* dep;        // [U][T]
  unsigned long long* rst;  // [U][T]
  float* wadd;          // [U][T][W]
  float* rc;            // [U][T][R]
  int T, W, R, win, bits;
  long long N;
};

__device__ __forceinline__ uint32_t prep_hash(uint32_t slot, int bits) { return (slot * 2654435761u) >> (32 - bits); }

__global__ void __launch_bounds__(256) bwd_prep_kernel(PrepArgs A) {
  extern __shared__ uint32_t psm[];
  const int bits = A.bits;
  const uint32_t hmask = (1u << bits) - 1;
  uint32_t* keys = psm;                                    // 2^bits slots (kEmptyKey: free)
  uint16_t* info = (uint16_t*)(psm + (1 << bits));         // offset << 7 | kind << 6 | position
  uint32_t* depm = (uint32_t*)(info + (1 << bits));        // [kPrepBlk]
  uint32_t* rstm = depm + kPrepBlk;                        // [2 kPrepBlk]
  constexpr uint32_t kEmptyKey = 0xFFFFFFFFu;
  const int u = blockIdx.y, t0 = blockIdx.x * kPrepBlk, T = A.T, W = A.W, R = A.R, per = W + R;
  const int t_end = min(t0 + kPrepBlk, T), h_end = min(t_end + A.win, T);
  for (int i = threadIdx.x; i < (1 << bits); i += 256) keys[i] = kEmptyKey;
  for (int i = threadIdx.x; i < 3 * kPrepBlk; i += 256) depm[i] = 0u;
  __syncthreads();
  const int32_t* wi = A.widx + (size_t)u * T * W;
  const int32_t* ri = A.ridx + (size_t)u * T * R;
  const float* rg = A.rgt + (size_t)u * T * R;
  for (int e = threadIdx.x; e < (h_end - t0) * per; e += 256) {
    const int k = e / per, p = e - k * per;
    const bool rd = p >= W;
    const int q = rd ? p - W : p;
    const int32_t slot = rd ? ri[(size_t)(t0 + k) * R + q] : wi[(size_t)(t0 + k) * W + q];
    if (slot < 0 || slot >= A.N) continue;
    uint32_t h = prep_hash((uint32_t)slot, bits);
    while (atomicCAS(&keys[h], kEmptyKey, (uint32_t)slot) != kEmptyKey) h = (h + 1) & hmask;
    info[h] = (uint16_t)((k << 7) | ((int)rd << 6) | q);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < (t_end - t0) * per; e += 256) {
    const int k = e / per, p = e - k * per, t = t0 + k;
    const bool rd = p >= W;
    const int q = rd ? p - W : p;
    const int32_t slot = rd ? ri[(size_t)t * R + q] : wi[(size_t)t * W + q];
    float acc = 0.f;
    bool dup = false, inw = false;
    uint32_t dm = 0;
    const bool valid = slot >= 0 && slot < A.N;
    if (valid) {
      uint32_t h = prep_hash((uint32_t)slot, bits);
      while (true) {
        const uint32_t key = keys[h];
        if (key == kEmptyKey) break;
        if (key == (uint32_t)slot) {
          const int inf = info[h], d = (inf >> 7) - k, kind = (inf >> 6) & 1, qq = inf & 63;
          if (d >= 1 && d <= A.win) dm |= 1u << (d - 1);
          if (d == 0 && kind == 1) {  // a read of the same slot in this token
            acc += rg[(size_t)t * R + qq];
            dup = dup || (rd && qq < q);
          }
          if (d == 0 && kind == 0 && rd) inw = true;
        }
        h = (h + 1) & hmask;
      }
    }
    if (dm) atomicOr(&depm[k], dm);
    const size_t ut = (size_t)u * T + t;
    if (!rd) {
      A.wadd[ut * W + q] = acc;
    } else {
      const bool st = valid && !dup && !inw;
      A.rc[ut * R + q] = st ? acc : 0.f;
      if (st) atomicOr(&rstm[2 * k + (q >> 5)], 1u << (q & 31));
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < t_end - t0; k += 256) {
    const size_t ut = (size_t)u * T + t0 + k;
    A.dep[ut] = depm[k];
    A.rst[ut] = (unsigned long long)rstm[2 * k] | ((unsigned long long)rstm[2 * k + 1] << 32);
  }
}

// ------------------------------------------------------------------ reverse walk
struct BwdArgs {
  const int32_t* widx;  // [U][T][W]
  const float* wgt;
  const int32_t* ridx;  // [U][T][R]
  const void* v;        // [U][T][d_v] in dtype
  const float* alpha;   // [U][T]
  const float* beta;
  void* M;              // [U][N][d_v] mem dtype: table after the forward in, M0 out
  const void* xlog;     // [U][T][W][d_v] mem dtype
  const float* go;      // [U][T][d_v]
  float* G;             // [U][N][d_v]: gradient of the final table in, of M0 out
  float* dv;            // [U][T][d_v]
  float* dalpha;        // [U][T] (zeroed)
  float* dbeta;         // [U][T] (zeroed)
  float* dwgt;          // [U][T][W] (zeroed)
  float* drgt;          // [U][T][R] (zeroed)
  const uint32_t* dep;  // preparation pass outputs
  const unsigned long long* rst;
  const float* wadd;
  const float* rc;
  unsigned long long* err;
  int U, T, W, R, d_v, P, K;
  long long N;
};

// Slot lists of one token and its coupling tables.
template <int LIST>
struct alignas(16) TokMeta {
  int n[LIST], m[LIST];
  float a[LIST], wadd[LIST], rc[LIST];
  float al, be;
  uint32_t dep, rlo, rhi;
};
static_assert(sizeof(TokMeta<8>) % 16 == 0 && sizeof(TokMeta<64>) % 16 == 0, "LDS layout keeps 16-byte rows");

template <int NG, int MH>
constexpr size_t wave_lds_bytes() {
  constexpr int C = 64 / NG, LIST = MH * NG;
  return (3 * sizeof(TokMeta<LIST>) + (size_t)2 * LIST * (C + 1) * 4 + 15) / 16 * 16;
}
constexpr size_t kCtrlBytes = (kFinRing + 16) * 4;

// NG row groups of C = 64 / NG lanes: each group holds the same C * CW columns (CW per lane)
// and takes up to MH write rows and MH read rows of every token.
template <typename MemT, typename InT, int NG, int MH, int CW>
__global__ void __launch_bounds__(CW == 1 ? kMaxWaves * 64 : 512) backward_kernel(BwdArgs A) {
  constexpr int C = 64 / NG;
  constexpr int LIST = MH * NG;  // longest slot list handled; group h holds rows h*MH + i
  using Meta = TokMeta<LIST>;
  extern __shared__ __align__(16) unsigned char smem[];
  int* fin = (int*)smem;       // [kFinRing]: token that finished in each ring position
  int* ctrl = fin + kFinRing;  // [0]: give-up flag
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, K = A.K;
  Meta* meta = (Meta*)(smem + kCtrlBytes + wave * wave_lds_bytes<NG, MH>());
  // per-column partials of one token: write rows [0, LIST), read rows [LIST, 2 LIST)
  float(*part)[C + 1] = (float(*)[C + 1])((unsigned char*)(meta + 3));
  for (int i = threadIdx.x; i < kFinRing; i += blockDim.x) fin[i] = -1;
  if (threadIdx.x < 16) ctrl[threadIdx.x] = 0;
  __syncthreads();
  const int h = lane / C, cl = lane % C, hb = h * MH;
  // blockIdx -> (unit, column block) with all column blocks of a unit in one L2 domain
  const int xcd = blockIdx.x % kXcd, y = blockIdx.x / kXcd;
  const int p = y % A.P, u = (y / A.P) * kXcd + xcd;
  if (u >= A.U) return;
  const int c = (p * C + cl) * CW;  // this lane's first column (d_v is a multiple of CW)
  const bool act = c < A.d_v;
  const uint32_t cc = act ? c : 0;  // inactive lanes load column 0 and discard it
  const int T = A.T, W = A.W, R = A.R, d_v = A.d_v;
  const long long N = A.N;
  constexpr uint32_t ms = sizeof(MemT), is = sizeof(InT);
  const rsrc_t rM = make_rs((const char*)A.M + (size_t)u * N * d_v * ms, (size_t)N * d_v * ms);
  const rsrc_t rG = make_rs(A.G + (size_t)u * N * d_v, (size_t)N * d_v * 4);
  const rsrc_t rX = make_rs((const char*)A.xlog + (size_t)u * T * W * d_v * ms, (size_t)T * W * d_v * ms);
  const rsrc_t rV = make_rs((const char*)A.v + (size_t)u * T * d_v * is, (size_t)T * d_v * is);
  const rsrc_t rO = make_rs(A.go + (size_t)u * T * d_v, (size_t)T * d_v * 4);
  const rsrc_t rD = make_rs(A.dv + (size_t)u * T * d_v, (size_t)T * d_v * 4);
  const uint32_t rowG = (uint32_t)d_v * 4, rowM = (uint32_t)d_v * ms;
  const size_t ut = (size_t)u * T;
  const rsrc_t rDW = make_rs(A.dwgt + ut * W, (size_t)T * W * 4);  // this unit's weight gradients
  const rsrc_t rDR = make_rs(A.drgt + ut * R, (size_t)T * R * 4);
  auto group_sum = [](float x) {
#pragma unroll
    for (int m = C; m < 64; m *= 2) x = add_xor_f32(x, m);
    return x;
  };
  auto column_sum = [](float x) {
#pragma unroll
    for (int m = 1; m < C; m *= 2) x = add_xor_f32(x, m);
    return x;
  };
  auto sync = [] {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  };

  // slot lists and tables of a token, lane-distributed, from global memory to LDS; list
  // positions past W or R get slot -1 (no row)
  int qn, qm;
  float qa, qwd, qrc, qal, qbe;
  uint32_t qdep;
  unsigned long long qrst;
  auto fetch = [&](int tt) {
    const size_t bw = (ut + tt) * W, br = (ut + tt) * R;
    const bool lw = lane < W, lr = lane < R;
    qn = lw ? A.widx[bw + lane] : -1;
    qa = lw ? A.wgt[bw + lane] : 0.f;
    qwd = lw ? A.wadd[bw + lane] : 0.f;
    qm = lr ? A.ridx[br + lane] : -1;
    qrc = lr ? A.rc[br + lane] : 0.f;
    qal = A.alpha[ut + tt];
    qbe = A.beta[ut + tt];
    qdep = A.dep[ut + tt];
    qrst = A.rst[ut + tt];
  };
  auto put = [&](Meta& mt) {
    if (lane < LIST) {
      mt.n[lane] = qn;
      mt.a[lane] = qa;
      mt.wadd[lane] = qwd;
      mt.m[lane] = qm;
      mt.rc[lane] = qrc;
    }
    if (lane == 0) {
      mt.al = qal;
      mt.be = qbe;
      mt.dep = qdep;
      mt.rlo = (uint32_t)qrst;
      mt.rhi = (uint32_t)(qrst >> 32);
    }
  };
  // this group's rows of a token as element indices slot * d_v + c into the unit's table;
  // kNone for no such row, a slot outside [0, N) or an inactive column. N * d_v < kNone
  // (tables stay below 2^31 - 16 bytes per unit), so kNone times the element size lies past
  // the end of the table's resource: a load of it returns zero and a store of it is dropped.
  const uint32_t N32 = (uint32_t)N;
  uint32_t rn[MH], rm[MH];
  auto rows_of = [&](const Meta& mt) {
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      const uint32_t n = (uint32_t)mt.n[hb + i], m = (uint32_t)mt.m[hb + i];  // hb + i < LIST
      rn[i] = act && n < N32 ? n * (uint32_t)d_v + (uint32_t)c : kNone;
      rm[i] = act && m < N32 ? m * (uint32_t)d_v + (uint32_t)c : kNone;
    }
  };
  // sums over this wave's columns of one token's row partials, added into the outputs: lane
  // j sums write row j and read row j (W, R <= 64), each into its own output resource
  auto reduce = [&](int tt) {
    if (lane < W) {
      float sum = 0.f;
#pragma unroll 8
      for (int q = 0; q < C; ++q) sum += part[lane][q];
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(sum, rDW, ((uint32_t)tt * W + lane) * 4, 0, 0);
    }
    if (lane < R) {
      float sum = 0.f;
#pragma unroll 8
      for (int q = 0; q < C; ++q) sum += part[LIST + lane][q];
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(sum, rDR, ((uint32_t)tt * R + lane) * 4, 0, 0);
    }
  };
  auto give_up = [&] {
    if (lane == 0) {
      lds_st(&ctrl[0], 1);
      atomicAdd(A.err, 1ull);
    }
  };

  int t = T - 1 - wave;
  if (t < 0) return;
  fetch(t);
  put(meta[0]);
  sync();
  rows_of(meta[0]);
  fetch(t >= K ? t - K : 0);
  if (t >= K) put(meta[1]);
  sync();

  int b0 = 0;  // buffer of token t; t - K uses (b0 + 1) % 3, t - 2K (b0 + 2) % 3
  long long budget = kSpinBudget;
  int prev = -1;  // this wave's previous token, whose column sums are still due
  for (; t >= 0; t -= K) {
    Meta& mt = meta[b0];
    Meta& m1 = meta[b0 == 2 ? 0 : b0 + 1];
    Meta& m2 = meta[b0 == 0 ? 2 : b0 - 1];
    // 1. the lists two own tokens ahead (independent of everything running)
    fetch(t >= 2 * K ? t - 2 * K : 0);
    // 2. wait for the later tokens this one depends on: those sharing a slot among the next
    //    K - 1, and every token from t + K on
    {
      const uint32_t dm = mt.dep;
      const int tau = t + 1 + lane;
      const bool need = lane < 2 * K - 1 && tau < T && (lane >= K - 1 || ((dm >> lane) & 1u));
      bool gave_up = false;
      while (true) {
        const bool pending = need && lds_ld(&fin[tau & (kFinRing - 1)]) != tau;
        if (ballot(pending) == 0ull) break;
        if (--budget <= 0) {
          give_up();
          gave_up = true;
          break;
        }
        if (lds_ld(&ctrl[0])) {
          gave_up = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (gave_up) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    // 3. every row load of token t at once (a row past W reads a neighbouring log row, or
    //    zeros past the end of the log, and is discarded)
    using WM = Wide<MemT, CW>;
    using WF = Wide<float, CW>;
    using WI = Wide<InT, CW>;
    uint32_t xr[MH][WM::kN], mrr[MH][WM::kN], gy[MH][WF::kN], gr[MH][WF::kN];
    const uint32_t xo = ((uint32_t)t * W + hb) * rowM + cc * ms;
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      WM::ld(rX, xo + i * rowM, xr[i]);
      WF::ld(rG, rn[i] * 4, gy[i]);
      WM::ld(rM, rm[i] * ms, mrr[i]);
      WF::ld(rG, rm[i] * 4, gr[i]);
    }
    uint32_t graw[WF::kN], vraw[WI::kN];
    WF::ld(rO, (uint32_t)t * rowG + cc * 4, graw);
    WI::ld(rV, ((uint32_t)t * d_v + cc) * is, vraw);
    // 4. while they are in flight: the previous token's column sums
    const unsigned long long rstm = ((unsigned long long)mt.rlo | ((unsigned long long)mt.rhi << 32)) >> hb;
    const float al = mt.al, be = mt.be;
    if (prev >= 0) reduce(prev);
    // the lists two own tokens ahead go to LDS (their loads were issued before this token's
    // row loads, so waiting for them does not wait for the rows)
    if (t >= 2 * K) put(m2);
    sync();
    // 5. token t (rows without a slot loaded zeros: dy = 0 there since wadd = 0)
    float g[CW], vc[CW];
#pragma unroll
    for (int k = 0; k < CW; ++k) {
      g[k] = act ? WF::val(graw, k) : 0.f;
      vc[k] = act ? WI::val(vraw, k) : 0.f;
    }
    float aj[MH], wd[MH];
    if constexpr (MH % 4 == 0) {
#pragma unroll
      for (int i = 0; i < MH; i += 4) {
        *(float4*)&aj[i] = *(const float4*)&mt.a[hb + i];
        *(float4*)&wd[i] = *(const float4*)&mt.wadd[hb + i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < MH; ++i) {
        aj[i] = mt.a[hb + i];
        wd[i] = mt.wadd[hb + i];
      }
    }
    float s[CW], dd[CW];
    float x[MH][CW], dy[MH][CW];
#pragma unroll
    for (int k = 0; k < CW; ++k) s[k] = dd[k] = 0.f;
#pragma unroll
    for (int i = 0; i < MH; ++i) {
#pragma unroll
      for (int k = 0; k < CW; ++k) {
        x[i][k] = rn[i] != kNone ? WM::val(xr[i], k) : 0.f;
        dy[i][k] = WF::val(gy[i], k) + wd[i] * g[k];
        s[k] = fmaf(aj[i], x[i][k], s[k]);
        dd[k] = fmaf(aj[i], dy[i][k], dd[k]);
      }
    }
    float resid[CW], delta[CW], drho[CW], pal[CW];
#pragma unroll
    for (int k = 0; k < CW; ++k) {
      s[k] = group_sum(s[k]);
      dd[k] = group_sum(dd[k]);
      resid[k] = vc[k] - al * s[k];
      delta[k] = be * resid[k];
      drho[k] = -be * dd[k];
      pal[k] = 0.f;
    }
    // row partials summed over this lane's columns
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      float pw = 0.f, pr = 0.f;
#pragma unroll
      for (int k = 0; k < CW; ++k) {
        pw += dy[i][k] * delta[k] + al * drho[k] * x[i][k];
        pal[k] = fmaf(dy[i][k], x[i][k], pal[k]);
        pr += g[k] * WM::val(mrr[i], k);
      }
      part[hb + i][cl] = pw;
      part[LIST + hb + i][cl] = pr;
    }
    // dalpha and dbeta: sums over rows (groups) and over this wave's columns
    float lal = 0.f, lbe = 0.f;
#pragma unroll
    for (int k = 0; k < CW; ++k) {
      lal += group_sum(pal[k]) + drho[k] * s[k];
      lbe += dd[k] * resid[k];
    }
    const float sal = column_sum(act ? lal : 0.f);
    const float sbe = column_sum(act ? lbe : 0.f);
    if (lane == 0) {
      atomicAdd(A.dalpha + ut + t, sal);
      atomicAdd(A.dbeta + ut + t, sbe);
    }
    // stores of token t (dropped for rows without a slot): G and the undone rows of M; G of
    // the reads that store it
    float rcv[MH];
    if constexpr (MH % 4 == 0) {
#pragma unroll
      for (int i = 0; i < MH; i += 4) *(float4*)&rcv[i] = *(const float4*)&mt.rc[hb + i];
    } else {
#pragma unroll
      for (int i = 0; i < MH; ++i) rcv[i] = mt.rc[hb + i];
    }
#pragma unroll
    for (int i = 0; i < MH; ++i) {
      float gv[CW], rv[CW];
#pragma unroll
      for (int k = 0; k < CW; ++k) {
        gv[k] = al * (dy[i][k] + aj[i] * drho[k]);
        rv[k] = WF::val(gr[i], k) + rcv[i] * g[k];
      }
      st_f32w<CW>(rG, rn[i] * 4, gv);
      WM::st_raw(rM, rn[i] * ms, xr[i]);  // the undone row is the logged row, bit for bit
      const uint32_t rs = (rstm >> i) & 1ull ? rm[i] : kNone;
      st_f32w<CW>(rG, rs * 4, rv);
    }
    if (h == 0 && act) {
      float dvv[CW];
#pragma unroll
      for (int k = 0; k < CW; ++k) dvv[k] = be * dd[k];
      st_f32w<CW>(rD, (uint32_t)t * rowG + c * 4, dvv);
    }
    // 6. publish token t once its stores are complete
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) lds_st(&fin[t & (kFinRing - 1)], t);
    sync();
    if (t >= K) rows_of(m1);
    prev = t;
    b0 = b0 == 2 ? 0 : b0 + 1;
  }
  reduce(prev);
}

// ------------------------------------------------------------------ addressing backward
// Gradients of the selected slots' softmax weights (PL §4 "SDM Configuration") with respect
// to the addressed rows x and the sub-keys (PL §2 "Product Key Memory": slot n = i*s + j
// scores x[:h].C1[i] + x[h:].C2[j]), the selection held fixed:
//   dscore_k = w_k (dw_k - sum_l w_l dw_l)
//   dx[half] = sum_k dscore_k C_half[i_half(k)];   dC_half = D^T X_half
// with D [tokens][s] holding each token's score gradients at its sub-keys of that half. A
// workgroup owns one head, one half, one slice of 64 sub-key columns and a chunk of that
// head's tokens. In steps of 32 tokens its 16 waves take two tokens each: the score
// gradients (one wave reduction), dx by gathering the selected sub-key rows eight at a
// time, and the token's row of D (one LDS atomic per selected slot, so equal sub-keys of
// one token add up) and of X. Then each wave adds D[:, its 32 sub-keys]^T X to its 32x64
// block of the sub-key gradient on the float32 MFMA (v_mfma_f32_32x32x2f32, K = 32 tokens
// in steps of 2; any split of K works as long as both operands use the same one), and the
// block is added to the output once at the end.
constexpr int kAbChunk = 4096;   // tokens per workgroup
constexpr int kAbWaves = 16;
constexpr int kAbStep = 32;      // tokens per MFMA step (two per wave)

typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct AddrBwdArgs {
  const void* x;        // [B][H][T][d_k]
  const void* sub;      // [H][2][s][hd]
  const int32_t* idx;   // [B][H][T][n_sel]
  const float* w;
  const float* dw;
  float* dx;            // [B][H][T][d_k]
  float* dsub;          // [H][2][s][hd], added to
  int B, H, T, d_k, hd, s, n_sel, nslice;
  long long N;
};

template <typename InT>
__global__ void __launch_bounds__(kAbWaves * 64) addr_backward_kernel(AddrBwdArgs A) {
  extern __shared__ float sm[];
  const int s = A.s, n_sel = A.n_sel, T = A.T, H = A.H, d_k = A.d_k;
  float* Dm = sm;                      // [kAbStep][s]: score gradients by sub-key
  float* Xm = sm + kAbStep * s;        // [kAbStep][64]: this slice of x's half
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.z, hf = blockIdx.y / A.nslice, slice = blockIdx.y % A.nslice;
  const int c = slice * 64 + lane;  // column within the half
  const bool act = c < A.hd;
  const int cc = act ? c : 0;       // inactive lanes read column 0, add zeros, store nothing
  for (int i = threadIdx.x; i < kAbStep * s; i += blockDim.x) Dm[i] = 0.f;
  const InT* C = (const InT*)A.sub + ((size_t)h * 2 + hf) * s * A.hd;
  const long long Th = (long long)A.B * T;
  const long long t0 = (long long)blockIdx.x * kAbChunk;
  const long long t1 = t0 + kAbChunk < Th ? t0 + kAbChunk : Th;
  auto ld = [](const InT* p, size_t i) -> float {
    if constexpr (sizeof(InT) == 2) return bf16_to_f32(p[i]);
    else return p[i];
  };
  const int r0 = wave * 32;  // this wave's block of sub-keys
  f32x16_t acc0 = {}, acc1 = {};
  // a token's inputs (weights, their gradients, slots, this lane's x column), loaded one step
  // ahead so that a step waits only for its sub-key row gathers
  struct TokIn {
    float wl, dwl, xv;
    int il;
  };
  auto load_tok = [&](long long cs, int q, TokIn& r) {
    const long long tt = cs + wave * 2 + q;
    const bool live = tt < t1;
    const long long b = tt / T, t = tt - b * T;
    const size_t row = live ? ((size_t)b * H + h) * T + t : 0;
    const bool lk = live && lane < n_sel;
    r.wl = lk ? A.w[row * n_sel + lane] : 0.f;
    r.dwl = lk ? A.dw[row * n_sel + lane] : 0.f;
    r.il = lk ? A.idx[row * n_sel + lane] : -1;
    r.xv = live && act ? ld((const InT*)A.x, row * d_k + hf * A.hd + c) : 0.f;
  };
  TokIn nx[2];
  load_tok(t0, 0, nx[0]);
  load_tok(t0, 1, nx[1]);
  __syncthreads();
  for (long long c0 = t0; c0 < t1; c0 += kAbStep) {
    TokIn cur[2] = {nx[0], nx[1]};
    if (c0 + kAbStep < t1) {
      load_tok(c0 + kAbStep, 0, nx[0]);
      load_tok(c0 + kAbStep, 1, nx[1]);
    }
    int mine[2];  // D entry this lane wrote for each of its tokens (-1: none)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tl = wave * 2 + q;
      const long long tt = c0 + tl;
      const bool live = tt < t1;
      const long long b = tt / T, t = tt - b * T;
      const size_t row = live ? ((size_t)b * H + h) * T + t : 0;  // token row of x, idx, w, dx
      const float wl = cur[q].wl, dwl = cur[q].dwl;
      const int il = cur[q].il;
      const float S = wave_sum_f32(wl * dwl);
      const float dsc = wl * (dwl - S);
      // this half's sub-key of each selected slot; -1 for a slot outside [0, N)
      const int ii = il >= 0 && il < A.N ? (hf == 0 ? il / s : il % s) : -1;
      float dxv = 0.f;
      // sixteen selected slots at a time, every load unguarded (a slot outside [0, N) reads
      // row 0 with coefficient 0), so that sixteen row loads are in flight together
      for (int k0 = 0; k0 < n_sel; k0 += 16) {
        int rk[16];
        float dk[16], cv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int k = min(k0 + u, 63);
          const int ik = k0 + u < n_sel ? __builtin_amdgcn_readlane(ii, k) : -1;
          const float d = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(dsc), k));
          rk[u] = ik >= 0 ? ik : 0;
          dk[u] = ik >= 0 ? d : 0.f;
          cv[u] = ld(C, (size_t)rk[u] * A.hd + cc);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) dxv = fmaf(dk[u], cv[u], dxv);
      }
      if (live && act) A.dx[row * d_k + hf * A.hd + c] = dxv;
      Xm[tl * 64 + lane] = cur[q].xv;
      mine[q] = ii;
      if (ii >= 0) atomicAdd(&Dm[tl * s + ii], dsc);
    }
    __syncthreads();
    if (r0 < s) {
      const int rr = r0 + (lane & 31);
#pragma unroll 4
      for (int k0 = 0; k0 < kAbStep; k0 += 2) {
        const int kk = k0 + (lane >> 5);
        const float a = rr < s ? Dm[kk * s + rr] : 0.f;
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Xm[kk * 64 + (lane & 31)], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Xm[kk * 64 + 32 + (lane & 31)], acc1, 0, 0, 0);
      }
    }
    __syncthreads();
    // clear this wave's entries of D for the next step (rows of its own tokens)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (mine[q] >= 0) Dm[(wave * 2 + q) * s + mine[q]] = 0.f;
  }
  // D[row][col]: lane holds col = lane % 32, rows 8*(e/4) + 4*(lane/32) + e%4
  if (r0 < s) {
    float* out = A.dsub + ((size_t)h * 2 + hf) * s * A.hd;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = r0 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const int c0 = slice * 64 + (lane & 31), c1 = c0 + 32;
      if (r < s && c0 < A.hd && acc0[e] != 0.f) atomicAdd(&out[(size_t)r * A.hd + c0], acc0[e]);
      if (r < s && c1 < A.hd && acc1[e] != 0.f) atomicAdd(&out[(size_t)r * A.hd + c1], acc1[e]);
    }
  }
}

__global__ void __launch_bounds__(256) zero_f32_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t zero_f32(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// Workspace of the backward: the error word first (offset 0, as every workspace of the
// library), then the preparation pass outputs.
struct BwdWs {
  size_t err, dep, rst, wadd, rc, total;
};
size_t bws_align(size_t x) { return (x + 255) & ~(size_t)255; }
BwdWs bwd_layout(const sdm_shape& S) {
  const size_t tok = (size_t)S.B * S.H * (size_t)S.T;
  BwdWs L;
  size_t o = 0;
  L.err = o;
  o = bws_align(o + 8);
  L.dep = o;
  o = bws_align(o + tok * 4);
  L.rst = o;
  o = bws_align(o + tok * 8);
  L.wadd = o;
  o = bws_align(o + tok * S.W * 4);
  L.rc = o;
  o = bws_align(o + tok * S.R * 4);
  L.total = o;
  return L;
}

template <typename MemT, typename InT, int NG, int MH, int CW>
hipError_t launch_cfg(BwdArgs A, const PrepArgs& Pa0, long long wgs, hipStream_t st) {
  A.P = (A.d_v + CW * 64 / NG - 1) / (CW * 64 / NG);
  // K waves per workgroup: 8, or 16 when fewer than two workgroups per CU would run (8 with
  // two columns per lane, whose row registers need the larger per-wave register file)
  A.K = CW == 2 || wgs >= 2ll * device_cus() ? 8 : kMaxWaves;
  PrepArgs Pa = Pa0;
  Pa.win = A.K - 1;
  const int entries = (kPrepBlk + Pa.win) * (A.W + A.R);
  Pa.bits = 6;
  while ((1 << Pa.bits) < 2 * entries) ++Pa.bits;
  const size_t plds = ((size_t)4 << Pa.bits) + ((size_t)2 << Pa.bits) + 3 * kPrepBlk * 4;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((A.T + kPrepBlk - 1) / kPrepBlk), (unsigned)A.U), dim3(256),
                     plds, st, Pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = kCtrlBytes + (size_t)A.K * wave_lds_bytes<NG, MH>();
  hipLaunchKernelGGL((backward_kernel<MemT, InT, NG, MH, CW>), dim3((unsigned)wgs), dim3(64 * A.K), lds, st, A);
  return hipGetLastError();
}

#ifndef SDM_BWD_CW
#define SDM_BWD_CW 0  // columns per lane of the reverse walk: 0 picks by shape
#endif

// Column blocks of C = 64 / NG columns, each row group taking MH in {2, 4, 8} rows of each
// kind (NG * MH >= max(W, R)): the widest block whose grid still gives every CU a
// workgroup, else the narrowest (units with few heads fill the chip with narrow blocks).
template <typename MemT, typename InT>
hipError_t launch_bwd(const BwdArgs& A, const PrepArgs& Pa, hipStream_t st) {
  const int list = A.W > A.R ? A.W : A.R;
  const int cus = device_cus();
  int pick = -1;
  long long pick_wgs = 0;
  for (int lg = 0; lg <= 4; ++lg) {  // NG = 1, 2, 4, 8, 16
    const int NG = 1 << lg, C = 64 / NG;
    if ((list + NG - 1) / NG > 8) continue;
    pick = lg;
    pick_wgs = (long long)((A.U + kXcd - 1) / kXcd) * kXcd * ((A.d_v + C - 1) / C);
    if (pick_wgs >= cus) break;
  }
  if (pick < 0) return hipErrorInvalidValue;
  const int NG = 1 << pick, mh = (list + NG - 1) / NG;
  const int MH = mh <= 2 ? 2 : mh <= 4 ? 4 : 8;
  // Two columns per lane when the wider blocks still give every CU a workgroup: a wave then
  // moves 64-byte pieces of bf16 rows, whole sectors, instead of halves that the unit's
  // other column blocks fetch again at other times.
  {
    const int C = 64 / NG;
    const long long wgs2 = (long long)((A.U + kXcd - 1) / kXcd) * kXcd * ((A.d_v + 2 * C - 1) / (2 * C));
    int cw = A.d_v % (2 * C) == 0 && wgs2 >= cus ? 2 : 1;
    if (SDM_BWD_CW) cw = SDM_BWD_CW;
    if (cw == 2) {
      if (NG == 2 && MH == 4) return launch_cfg<MemT, InT, 2, 4, 2>(A, Pa, wgs2, st);
      if (NG == 2 && MH == 8) return launch_cfg<MemT, InT, 2, 8, 2>(A, Pa, wgs2, st);
      if (NG == 4 && MH == 4) return launch_cfg<MemT, InT, 4, 4, 2>(A, Pa, wgs2, st);
      if (NG == 4 && MH == 8) return launch_cfg<MemT, InT, 4, 8, 2>(A, Pa, wgs2, st);
    }
  }
  if (NG == 1 && MH == 2) return launch_cfg<MemT, InT, 1, 2, 1>(A, Pa, pick_wgs, st);
  if (NG == 1 && MH == 4) return launch_cfg<MemT, InT, 1, 4, 1>(A, Pa, pick_wgs, st);
  if (NG == 1 && MH == 8) return launch_cfg<MemT, InT, 1, 8, 1>(A, Pa, pick_wgs, st);
  if (NG == 2 && MH == 2) return launch_cfg<MemT, InT, 2, 2, 1>(A, Pa, pick_wgs, st);
  if (NG == 2 && MH == 4) return launch_cfg<MemT, InT, 2, 4, 1>(A, Pa, pick_wgs, st);
  if (NG == 2 && MH == 8) return launch_cfg<MemT, InT, 2, 8, 1>(A, Pa, pick_wgs, st);
  if (NG == 4 && MH == 2) return launch_cfg<MemT, InT, 4, 2, 1>(A, Pa, pick_wgs, st);
  if (NG == 4 && MH == 4) return launch_cfg<MemT, InT, 4, 4, 1>(A, Pa, pick_wgs, st);
  if (NG == 4 && MH == 8) return launch_cfg<MemT, InT, 4, 8, 1>(A, Pa, pick_wgs, st);
  if (NG == 8 && MH == 2) return launch_cfg<MemT, InT, 8, 2, 1>(A, Pa, pick_wgs, st);
  if (NG == 8 && MH == 4) return launch_cfg<MemT, InT, 8, 4, 1>(A, Pa, pick_wgs, st);
  if (NG == 8 && MH == 8) return launch_cfg<MemT, InT, 8, 8, 1>(A, Pa, pick_wgs, st);
  if (NG == 16 && MH == 2) return launch_cfg<MemT, InT, 16, 2, 1>(A, Pa, pick_wgs, st);
  if (NG == 16 && MH == 4) return launch_cfg<MemT, InT, 16, 4, 1>(A, Pa, pick_wgs, st);
  return hipErrorInvalidValue;
}

}  // namespace

size_t backward_workspace_bytes(const sdm_shape& S) { return bwd_layout(S).total; }

hipError_t launch_backward(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                           const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                           const void* xlog, const float* go, float* G, float* dv, float* dalpha, float* dbeta,
                           float* dwgt, float* drgt, void* ws, hipStream_t stream) {
  if (S.W > kMaxSel || S.R > kMaxSel) return hipErrorInvalidValue;
  const int U = S.B * S.H;
  const size_t tok = (size_t)U * S.T;
  const BwdWs L = bwd_layout(S);
  char* w = (char*)ws;
  hipError_t e = zero_f32((float*)(w + L.err), 2, stream);
  if (e != hipSuccess) return e;
  e = zero_f32(dalpha, tok, stream);
  if (e != hipSuccess) return e;
  e = zero_f32(dbeta, tok, stream);
  if (e != hipSuccess) return e;
  e = zero_f32(dwgt, tok * S.W, stream);
  if (e != hipSuccess) return e;
  e = zero_f32(drgt, tok * S.R, stream);
  if (e != hipSuccess) return e;
  if (tok == 0) return hipSuccess;
  PrepArgs Pa;
  Pa.widx = widx;
  Pa.ridx = ridx;
  Pa.rgt = rgt;
  Pa.dep = (uint32_t*)(w + L.dep);
  Pa.rst = (unsigned long long*)(w + L.rst);
  Pa.wadd = (float*)(w + L.wadd);
  Pa.rc = (float*)(w + L.rc);
  Pa.T = S.T;
  Pa.W = S.W;
  Pa.R = S.R;
  Pa.N = S.N;
  BwdArgs A;
  A.widx = widx;
  A.wgt = wgt;
  A.ridx = ridx;
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  A.M = M;
  A.xlog = xlog;
  A.go = go;
  A.G = G;
  A.dv = dv;
  A.dalpha = dalpha;
  A.dbeta = dbeta;
  A.dwgt = dwgt;
  A.drgt = drgt;
  A.dep = Pa.dep;
  A.rst = Pa.rst;
  A.wadd = Pa.wadd;
  A.rc = Pa.rc;
  A.err = (unsigned long long*)(w + L.err);
  A.U = U;
  A.T = S.T;
  A.W = S.W;
  A.R = S.R;
  A.d_v = S.d_v;
  A.N = S.N;
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return launch_bwd<uint16_t, uint16_t>(A, Pa, stream);
  if (mb && !ib) return launch_bwd<uint16_t, float>(A, Pa, stream);
  if (!mb && ib) return launch_bwd<float, uint16_t>(A, Pa, stream);
  return launch_bwd<float, float>(A, Pa, stream);
}

hipError_t launch_address_backward(const sdm_shape& S, const void* x, const void* subkeys, int n_sel,
                                   const int32_t* idx, const float* w, const float* dw, float* dx, float* dsub,
                                   hipStream_t stream) {
  AddrBwdArgs A;
  A.x = x;
  A.sub = subkeys;
  A.idx = idx;
  A.w = w;
  A.dw = dw;
  A.dx = dx;
  A.dsub = dsub;
  A.B = S.B;
  A.H = S.H;
  A.T = S.T;
  A.d_k = S.d_k;
  A.hd = S.d_k / 2;
  A.s = (int)isqrt64(S.N);
  A.n_sel = n_sel;
  A.nslice = (A.hd + 63) / 64;
  A.N = S.N;
  const long long Th = (long long)S.B * S.T;
  if (Th == 0) return hipSuccess;
  const dim3 grid((unsigned)((Th + kAbChunk - 1) / kAbChunk), (unsigned)(2 * A.nslice), (unsigned)S.H);
  const size_t lds = ((size_t)kAbStep * A.s + (size_t)kAbStep * 64) * 4;
  if (S.in_dtype == SDM_BF16)
    hipLaunchKernelGGL(addr_backward_kernel<uint16_t>, grid, dim3(kAbWaves * 64), lds, stream, A);
  else
    hipLaunchKernelGGL(addr_backward_kernel<float>, grid, dim3(kAbWaves * 64), lds, stream, A);
  return hipGetLastError();
}

}  // namespace sdm
