// Whole-table decay, applied lazily: the variant of the recurrence in which alpha_t decays
// every row of the table, not only the written ones.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Gated DeltaNet": the decay gate
// alpha_t scales the whole state; §3 "Sparse memory updates" and "Connection to GDN"): with
// the whole table decayed every token, the value of row n before token t is its last
// written value times exp(L_{t-1} - lam_n), where L_t is the running sum of log alpha over
// the tokens so far and lam_n its value when row n was last written. So no untouched row is
// ever read or written: the state carries lam [U][N] and the running L [U] beside the
// table, and every token-slot access of a call gets one factor
//   write slot of token t:  exp(L_{t-1} - lam)   (value before the token's decay)
//   read slot of token t:   exp(L_t - lam)       (value after it; 1 for a row t writes)
// that the pipeline applies to the gathered row (write slots) or to the read weight.
//
// The factors depend only on which tokens write which slots, known before the recurrence
// runs: decay_pass_kernel walks the tokens of a unit in chunks of at most `win` tokens.
// Within the window the dependency pass already names each access's latest writer; an
// access with none there sees no write since the chunk began, so the per-slot record of
// the latest writer as of the chunk start decides it. Each workgroup keeps that record for
// one range of slots in LDS.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kPassThreads = 1024;
constexpr int kPassChunk = 32;                 // tokens per chunk; at most the smallest window
constexpr int kPassSlotsMax = 32768;           // slots of one workgroup's LDS record (128 KB)
constexpr uint32_t kCoded = 0x80000000u;       // packed slot word of the dependency pass
constexpr uint32_t kInvalid = 0x40000000u;
constexpr uint32_t kSlotMask = 0x3FFFFu;

// log alpha, floored so that a zero gate gives a finite, fully decaying cumulative sum
__device__ __forceinline__ double log_gate(float a) { return fmax(log((double)a), -1000.0); }
__device__ __forceinline__ float decay_factor(double to, double from) { return expf((float)(to - from)); }

// L[u][0] = lrun[u]; L[u][t + 1] = L[u][t] + log alpha[u][t]; then lrun[u] = L[u][T].
__global__ void __launch_bounds__(kScanThreads) log_decay_scan_kernel(const float* alpha, double* L, double* lrun,
                                                                      int T) {
  __shared__ double part[kScanThreads];
  const int u = blockIdx.x, tid = threadIdx.x;
  const float* a = alpha + (size_t)u * T;
  double* Lu = L + (size_t)u * (T + 1);
  const int per = (T + kScanThreads - 1) / kScanThreads;
  const int lo = tid * per, hi = min(T, lo + per);
  double s = 0.0;
  for (int t = lo; t < hi; ++t) s += log_gate(a[t]);
  part[tid] = s;
  __syncthreads();
  // inclusive scan of the per-thread sums (Hillis-Steele over LDS)
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const double add = tid >= off ? part[tid - off] : 0.0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const double base = lrun[u];
  double run = base + (tid > 0 ? part[tid - 1] : 0.0);
  if (tid == 0) Lu[0] = base;
  for (int t = lo; t < hi; ++t) {
    run += log_gate(a[t]);
    Lu[t + 1] = run;
  }
  __syncthreads();
  if (tid == 0) lrun[u] = base + part[kScanThreads - 1];
}

struct PassArgs {
  const uint32_t* pk;  // [U][T][E] packed slot words (write slots, then read slots)
  const double* L;     // [U][T + 1]
  double* lam;         // [U][N] in/out
  float* fac;          // [U][T][E] out
  int T, W, E, P, span;
  long long N;
};

// One workgroup per (unit, slot range of `span` slots): factors of the accesses to its
// slots, then the cumulative log-decay at each of its slots' last write.
__global__ void __launch_bounds__(kPassThreads) decay_pass_kernel(PassArgs A) {
  extern __shared__ int last_tok[];  // [span]: latest writer so far in this call, -1 = none
  const int u = blockIdx.x / A.P, p = blockIdx.x % A.P, tid = threadIdx.x;
  const int T = A.T, W = A.W, E = A.E, span = A.span;
  const long long n0 = (long long)p * span;
  for (int i = tid; i < span; i += kPassThreads) last_tok[i] = -1;
  __syncthreads();
  const uint32_t* pk = A.pk + (size_t)u * T * E;
  const double* L = A.L + (size_t)u * (T + 1);
  double* lam = A.lam + (size_t)u * A.N;
  float* fac = A.fac + (size_t)u * T * E;
  for (int c0 = 0; c0 < T; c0 += kPassChunk) {
    const int c1 = min(T, c0 + kPassChunk);
    // factors of the chunk's accesses to this range, from the record as of the chunk start
    for (int i = c0 * E + tid; i < c1 * E; i += kPassThreads) {
      const int t = i / E, e = i - t * E;
      const uint32_t w = pk[i];
      if ((w & (kCoded | kInvalid)) == kInvalid) {
        if (p == 0) fac[i] = 1.f;  // slot outside [0, N): no weight, any finite factor
        continue;
      }
      const long long n = w & kSlotMask;
      if (n < n0 || n >= n0 + span) continue;
      const double to = e >= W ? L[t + 1] : L[t];
      float f;
      if (w & kCoded) {
        const int d = (w >> 24) & 127;
        f = d == 0 ? 1.f : decay_factor(to, L[t - d + 1]);
      } else {
        const int lt = last_tok[n - n0];
        f = decay_factor(to, lt >= 0 ? L[lt + 1] : lam[n]);
      }
      fac[i] = f;
    }
    __syncthreads();
    // the chunk's writes to this range
    for (int i = c0 * W + tid; i < c1 * W; i += kPassThreads) {
      const int t = i / W, j = i - t * W;
      const uint32_t w = pk[(size_t)t * E + j];
      if ((w & (kCoded | kInvalid)) == kInvalid) continue;
      const long long n = w & kSlotMask;
      if (n >= n0 && n < n0 + span) atomicMax(&last_tok[n - n0], t);
    }
    __syncthreads();
  }
  for (int i = tid; i < span; i += kPassThreads) {
    const long long n = n0 + i;
    if (n < A.N && last_tok[i] >= 0) lam[n] = L[last_tok[i] + 1];
  }
}

// out[u][n][c] = M[u][n][c] * exp(lrun[u] - lam[u][n]), float32
template <typename MemT>
__global__ void __launch_bounds__(256) materialize_kernel(const MemT* M, const double* lam, const double* lrun,
                                                          float* out, long long N, int d_v, long long rows) {
  const long long row = (long long)blockIdx.x * (256 / 32) + threadIdx.x / 32;
  if (row >= rows) return;
  const long long u = row / N;
  const float f = decay_factor(lrun[u], lam[row]);
  for (int c = threadIdx.x % 32; c < d_v; c += 32) {
    float x;
    if constexpr (sizeof(MemT) == 2) x = bf16_to_f32(M[row * d_v + c]);
    else x = M[row * d_v + c];
    out[row * d_v + c] = x * f;
  }
}

}  // namespace

hipError_t launch_log_decay_scan(const sdm_shape& S, const float* alpha, double* L, double* lrun,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(log_decay_scan_kernel, dim3(S.B * S.H), dim3(kScanThreads), 0, stream, alpha, L, lrun, S.T);
  return hipGetLastError();
}

int decay_pass_ranges(const sdm_shape& S) { return (int)((S.N + kPassSlotsMax - 1) / kPassSlotsMax); }

hipError_t launch_decay_pass(const sdm_shape& S, const uint32_t* pk, const double* L, double* lam, float* fac,
                             int win, hipStream_t stream) {
  if (win < kPassChunk) return hipErrorInvalidValue;
  PassArgs A;
  A.pk = pk;
  A.L = L;
  A.lam = lam;
  A.fac = fac;
  A.T = S.T;
  A.W = S.W;
  A.E = S.W + S.R;
  A.P = decay_pass_ranges(S);
  A.span = (int)((S.N + A.P - 1) / A.P);
  A.N = S.N;
  hipLaunchKernelGGL(decay_pass_kernel, dim3(S.B * S.H * A.P), dim3(kPassThreads), (size_t)A.span * 4, stream, A);
  return hipGetLastError();
}

hipError_t launch_materialize(const sdm_shape& S, const void* M, const double* lam, const double* lrun, float* out,
                              hipStream_t stream) {
  const long long rows = (long long)S.B * S.H * S.N;
  const dim3 grid((unsigned)((rows + 7) / 8));
  if (S.mem_dtype == SDM_BF16)
    hipLaunchKernelGGL(materialize_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)M, lam, lrun, out,
                       (long long)S.N, S.d_v, rows);
  else
    hipLaunchKernelGGL(materialize_kernel<float>, grid, dim3(256), 0, stream, (const float*)M, lam, lrun, out,
                       (long long)S.N, S.d_v, rows);
  return hipGetLastError();
}

}  // namespace sdm
