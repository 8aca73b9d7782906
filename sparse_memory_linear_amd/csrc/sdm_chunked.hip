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
// Phase 1 (chunk_prep_kernel, one workgroup per (unit, chunk), every chunk in parallel): the
// chunk's write occurrences go into an LDS hash of per-slot linked lists; each write and
// read occurrence walks its slot's list for its interactions, its decay coefficient and its
// write-back coefficient (the product over a slot's writers between two tokens is a product
// over a set, so the list order does not matter), and X = (I + diag(beta) K)^-1 diag(beta)
// comes from one forward substitution per column. Phase 2 (chunk_apply_kernel, one
// workgroup per (unit, block of 4 columns), the chunks of a unit in order): gather the
// chunk's rows into LDS, form P and O0, delta = X (V - P), o = O0 + Q delta, and the last
// writer of each slot writes its row back once (rounded to the table dtype there).

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kC = 64;           // tokens per chunk
constexpr int kMaxList = 32;     // W, R <= 32 on this path
constexpr int kOcc = kC * kMaxList;
constexpr int kBuckets = 4096;   // LDS hash: at most 2048 distinct slots, at most half full
constexpr uint32_t kFree = 0xFFFFFFFFu;
constexpr int kCB = 4;           // columns per Phase 2 workgroup

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
  // Phase 1 outputs, per (unit, chunk)
  float* X;             // [kC][kC]: (I + diag(beta) K)^-1 diag(beta)
  float* Q;             // [kC][kC]
  float* gw;            // [kC][W]: alpha_t a_tj dec(n_tj; start, t)
  float* gr;            // [kC][R]: u_tr dec(m_tr; start, t+1)
  float* ew;            // [kC][W]: a_tj dec(n_tj; t, end)
  float* ge;            // [kC][W]: dec(n_tj; start, end) for the slot's last writer
  int* nxt;             // [kC][W]: next writer of the same slot in the chunk's list, -1 at the end
  int* own;             // [kC][W]: for the slot's last writer, the head of its list; else -1
  int U, T, W, R, d_v, nchunk;
  long long N;
};

__device__ __forceinline__ uint32_t chunk_hash(uint32_t s) { return (s * 2654435761u) >> 20; }  // 12 bits

__global__ void __launch_bounds__(256) chunk_prep_kernel(ChunkArgs A) {
  __shared__ int sn[kOcc];
  __shared__ float sa[kOcc];
  __shared__ int snx[kOcc];
  __shared__ float sal[kC], sbe[kC];
  __shared__ uint32_t keys[kBuckets];
  __shared__ int head[kBuckets];
  __shared__ float K[kC][kC + 1];
  __shared__ float Qs[kC][kC + 1];
  const int chunk = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int W = A.W, R = A.R, T = A.T;
  const int t0 = chunk * kC, L = min(kC, T - t0);
  const long long N = A.N;
  const size_t ut0 = (size_t)u * T + t0;
  for (int i = tid; i < kBuckets; i += 256) {
    keys[i] = kFree;
    head[i] = -1;
  }
  for (int i = tid; i < kC * (kC + 1); i += 256) {
    (&K[0][0])[i] = 0.f;
    (&Qs[0][0])[i] = 0.f;
  }
  for (int i = tid; i < L * W; i += 256) {
    sn[i] = A.widx[ut0 * W + i];
    sa[i] = A.wgt[ut0 * W + i];
  }
  for (int i = tid; i < L; i += 256) {
    sal[i] = A.alpha[ut0 + i];
    sbe[i] = A.beta[ut0 + i];
  }
  __syncthreads();
  // the chunk's write occurrences into per-slot lists (slots outside [0, N) touch nothing)
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
  for (int i = tid; i < L * W; i += 256) {
    const int s = sn[i];
    if (s < 0 || s >= N) {
      snx[i] = -1;
      continue;
    }
    const int b = find((uint32_t)s, true);
    snx[i] = atomicExch(&head[b], i);
  }
  __syncthreads();
  // write occurrences: interactions with earlier writers, gathered decay, write-back terms
  const size_t cb = ((size_t)u * A.nchunk + chunk);  // this chunk's block of the outputs
  for (int i = tid; i < kC * W; i += 256) {
    const int t = i / W;
    float gwv = 0.f, ewv = 0.f, gev = 0.f;
    int ownv = -1;
    if (t < L && sn[i] >= 0 && sn[i] < N) {
      const int b = find((uint32_t)sn[i], false);
      float before = 1.f, after = 1.f, all = 1.f;
      bool last = true;
      for (int k = head[b]; k >= 0; k = snx[k]) {
        const int tk = k / W;
        all *= sal[tk];
        if (tk < t) {
          before *= sal[tk];
          // dec(n; tk, t): writers strictly between tk and t
          float between = 1.f;
          for (int l = head[b]; l >= 0; l = snx[l]) {
            const int tl = l / W;
            if (tl > tk && tl < t) between *= sal[tl];
          }
          atomicAdd(&K[t][tk], sal[t] * sa[i] * between * sa[k]);
        } else if (tk > t) {
          after *= sal[tk];
          last = false;
        }
      }
      gwv = sal[t] * sa[i] * before;
      ewv = sa[i] * after;
      if (last) {
        ownv = head[b];
        gev = all;
      }
    }
    A.gw[cb * kC * W + i] = gwv;
    A.ew[cb * kC * W + i] = ewv;
    A.ge[cb * kC * W + i] = gev;
    A.nxt[cb * kC * W + i] = i < L * W ? snx[i] : -1;
    A.own[cb * kC * W + i] = ownv;
  }
  // read occurrences: couplings to the chunk's writers up to and including the token
  for (int i = tid; i < kC * R; i += 256) {
    const int t = i / R;
    float grv = 0.f;
    if (t < L) {
      const int s = A.ridx[ut0 * R + i];
      const float w = A.rgt[ut0 * R + i];
      if (s >= 0 && s < N) {
        const int b = find((uint32_t)s, false);
        float upto = 1.f;
        if (b >= 0) {
          for (int k = head[b]; k >= 0; k = snx[k]) {
            const int tk = k / W;
            if (tk > t) continue;
            upto *= sal[tk];
            float between = 1.f;
            for (int l = head[b]; l >= 0; l = snx[l]) {
              const int tl = l / W;
              if (tl > tk && tl <= t) between *= sal[tl];
            }
            atomicAdd(&Qs[t][tk], w * between * sa[k]);
          }
        }
        grv = w * upto;
      }
    }
    A.gr[cb * kC * R + i] = grv;
  }
  __syncthreads();
  // X = (I + diag(beta) K)^-1 diag(beta): column c by forward substitution
  float* X = A.X + cb * kC * kC;
  float* Qo = A.Q + cb * kC * kC;
  if (tid < kC) {
    const int c = tid;
    float x[kC];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float acc = i == c ? 1.f : 0.f;
      if (i > c && i < L) {
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < kC; ++k)
          if (k >= c && k < i) sum = fmaf(K[i][k], x[k], sum);
        acc = -sbe[i] * sum;
      }
      x[i] = i >= c && i < L ? acc : 0.f;
    }
    const float bc = c < L ? sbe[c] : 0.f;
#pragma unroll
    for (int i = 0; i < kC; ++i) X[i * kC + c] = x[i] * bc;
  }
  for (int i = tid; i < kC * kC; i += 256) Qo[i] = Qs[i / kC][i % kC];
}

template <typename MemT>
__device__ __forceinline__ float mem_ld(const MemT* p, size_t i) {
  if constexpr (sizeof(MemT) == 2) return bf16_to_f32(p[i]);
  else return p[i];
}
template <typename MemT>
__device__ __forceinline__ void mem_st(MemT* p, size_t i, float x) {
  if constexpr (sizeof(MemT) == 2) p[i] = (uint16_t)pack_bf16x2(x, 0.f);
  else p[i] = x;
}

template <typename MemT, typename InT>
__global__ void __launch_bounds__(256) chunk_apply_kernel(ChunkArgs A) {
  __shared__ float Mw[kOcc][kCB];   // gathered write rows
  __shared__ float Mr[kOcc][kCB];   // gathered read rows
  __shared__ float P[kC][kCB], Dl[kC][kCB], O0[kC][kCB];
  const int u = blockIdx.y, c0 = blockIdx.x * kCB, tid = threadIdx.x;
  const int W = A.W, R = A.R, T = A.T, d_v = A.d_v;
  const long long N = A.N;
  MemT* M = (MemT*)A.M + (size_t)u * N * d_v;
  const InT* v = (const InT*)A.v + (size_t)u * T * d_v;
  float* o = A.o + (size_t)u * T * d_v;
  for (int chunk = 0; chunk < A.nchunk; ++chunk) {
    const int t0 = chunk * kC, L = min(kC, T - t0);
    const size_t ut0 = (size_t)u * T + t0;
    const size_t cb = ((size_t)u * A.nchunk + chunk);
    const float* gw = A.gw + cb * kC * W;
    const float* gr = A.gr + cb * kC * R;
    // 1. gather the chunk's rows (this block's columns)
    for (int i = tid; i < L * W * kCB; i += 256) {
      const int occ = i / kCB, c = i % kCB;
      const int s = A.widx[ut0 * W + occ];
      const bool ok = s >= 0 && s < N && c0 + c < d_v;
      Mw[occ][c] = ok ? mem_ld(M, (size_t)s * d_v + c0 + c) : 0.f;
    }
    for (int i = tid; i < L * R * kCB; i += 256) {
      const int occ = i / kCB, c = i % kCB;
      const int s = A.ridx[ut0 * R + occ];
      const bool ok = s >= 0 && s < N && c0 + c < d_v;
      Mr[occ][c] = ok ? mem_ld(M, (size_t)s * d_v + c0 + c) : 0.f;
    }
    __syncthreads();
    // 2. P and O0 (thread per token and column)
    const int t = tid / kCB, c = tid % kCB;
    if (t < L) {
      float p = 0.f, q = 0.f;
      for (int j = 0; j < W; ++j) p = fmaf(gw[t * W + j], Mw[t * W + j][c], p);
      for (int r = 0; r < R; ++r) q = fmaf(gr[t * R + r], Mr[t * R + r][c], q);
      const float vv = c0 + c < d_v ? (sizeof(InT) == 2 ? bf16_to_f32(((const uint16_t*)v)[(size_t)(t0 + t) * d_v + c0 + c])
                                                        : ((const float*)v)[(size_t)(t0 + t) * d_v + c0 + c])
                                    : 0.f;
      P[t][c] = vv - p;  // V - P
      O0[t][c] = q;
    }
    __syncthreads();
    // 3. delta = X (V - P)
    const float* X = A.X + cb * kC * kC;
    if (t < L) {
      float d = 0.f;
      for (int k = 0; k <= t; ++k) d = fmaf(X[t * kC + k], P[k][c], d);
      Dl[t][c] = d;
    }
    __syncthreads();
    // 4. o = O0 + Q delta
    const float* Q = A.Q + cb * kC * kC;
    if (t < L && c0 + c < d_v) {
      float y = O0[t][c];
      for (int k = 0; k <= t; ++k) y = fmaf(Q[t * kC + k], Dl[k][c], y);
      o[(size_t)(t0 + t) * d_v + c0 + c] = y;
    }
    // 5. each slot's last writer writes its row back once
    const float* ew = A.ew + cb * kC * W;
    const float* ge = A.ge + cb * kC * W;
    const int* nxt = A.nxt + cb * kC * W;
    const int* own = A.own + cb * kC * W;
    for (int i = tid; i < L * W * kCB; i += 256) {
      const int occ = i / kCB, cc = i % kCB;
      const int hd = own[occ];
      if (hd < 0 || c0 + cc >= d_v) continue;
      float row = ge[occ] * Mw[occ][cc];
      for (int k = hd; k >= 0; k = nxt[k]) row = fmaf(ew[k], Dl[k / W][cc], row);
      const int s = A.widx[ut0 * W + occ];
      mem_st(M, (size_t)s * d_v + c0 + cc, row);
    }
    // the next chunk's gathers read these rows: stores complete, then the barrier
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

}  // namespace

size_t chunked_workspace_bytes(const sdm_shape& S) {
  const size_t nch = ((size_t)S.T + kC - 1) / kC;
  const size_t per = (size_t)kC * kC * 4 * 2 + (size_t)kC * S.W * 4 * 5 + (size_t)kC * S.R * 4;
  return 256 + (size_t)S.B * S.H * nch * per;
}

bool chunked_supported(const sdm_shape& S) { return S.W <= kMaxList && S.R <= kMaxList; }

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
  const size_t nblk = (size_t)A.U * A.nchunk;
  char* w = (char*)ws + 256;
  A.X = (float*)w;
  w += nblk * kC * kC * 4;
  A.Q = (float*)w;
  w += nblk * kC * kC * 4;
  A.gw = (float*)w;
  w += nblk * kC * S.W * 4;
  A.ew = (float*)w;
  w += nblk * kC * S.W * 4;
  A.ge = (float*)w;
  w += nblk * kC * S.W * 4;
  A.nxt = (int*)w;
  w += nblk * kC * S.W * 4;
  A.own = (int*)w;
  w += nblk * kC * S.W * 4;
  A.gr = (float*)w;
  if (A.U == 0 || A.T == 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)A.nchunk, (unsigned)A.U), dim3(256), 0, stream, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((S.d_v + kCB - 1) / kCB), (unsigned)A.U);
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) hipLaunchKernelGGL((chunk_apply_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, stream, A);
  else if (mb) hipLaunchKernelGGL((chunk_apply_kernel<uint16_t, float>), grid, dim3(256), 0, stream, A);
  else if (ib) hipLaunchKernelGGL((chunk_apply_kernel<float, uint16_t>), grid, dim3(256), 0, stream, A);
  else hipLaunchKernelGGL((chunk_apply_kernel<float, float>), grid, dim3(256), 0, stream, A);
  return hipGetLastError();
}

}  // namespace sdm
