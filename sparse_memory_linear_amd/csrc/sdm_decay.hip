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
// runs. Within the window the dependency pass already names each access's latest writer;
// for the other accesses decay_order_kernel walks the tokens of a unit in chunks of at
// most `win` tokens, keeping per slot range (in LDS) the latest writer so far: an access
// with no writer inside the window sees no write since its chunk began, so the record as
// of the chunk start is its latest writer. When a unit's slot ranges alone would leave
// most compute units idle, its tokens are cut into segments walked in parallel:
// decay_seglast_kernel first records each segment's latest writer of every slot, and a
// segment's walk starts from the latest of those records over the segments before it.
// decay_factor_kernel then forms every factor in parallel, and decay_lam_kernel moves lam
// forward for the slots the call wrote.

#include <algorithm>

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kScanThreads = 256;
constexpr int kPassThreads = 1024;
constexpr int kPerThread = 8;                  // accesses per thread and chunk (chunk * (W + R) <= 8192)
constexpr int kPassSlotsMax = 32768;           // slots of one workgroup's LDS record (128 KB)
constexpr uint32_t kCoded = 0x80000000u;       // packed slot word of the dependency pass
constexpr uint32_t kInvalid = 0x40000000u;
constexpr uint32_t kSlotMask = 0x3FFFFu;

// log alpha, floored so that a zero gate gives a finite, fully decaying cumulative sum
__device__ __forceinline__ double log_gate(float a) { return fmax(log((double)a), -1000.0); }
__device__ __forceinline__ float decay_factor(double to, double from) { return expf((float)(to - from)); }

// L[u][0] = lrun[u]; L[u][t + 1] = L[u][t] + log alpha[u][t]; then lrun[u] = L[u][T].
// Three steps, so that a long sequence is scanned by many workgroups: each block of
// kScanBlock tokens sums its log gates into L at its end boundary e_b = min((b+1)*kScanBlock,
// T); one thread per unit turns those sums into running totals (from lrun) in place; each
// block then scans its own tokens from the total at its start and writes every entry but its
// end boundary, which already holds the running total.
constexpr int kScanPer = 8;                         // tokens per thread
constexpr int kScanBlock = kScanThreads * kScanPer;  // tokens per block

__device__ __forceinline__ double block_sum_f64(double v, double* part) {
  const int tid = threadIdx.x;
  part[tid] = v;
  __syncthreads();
  for (int off = kScanThreads / 2; off > 0; off >>= 1) {
    if (tid < off) part[tid] += part[tid + off];
    __syncthreads();
  }
  return part[0];
}

__global__ void __launch_bounds__(kScanThreads) log_decay_sums_kernel(const float* alpha, double* L, int T) {
  __shared__ double part[kScanThreads];
  const int u = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
  const float* a = alpha + (size_t)u * T;
  const int lo = b * kScanBlock + tid * kScanPer, hi = min(T, lo + kScanPer);
  double s = 0.0;
  for (int t = lo; t < hi; ++t) s += log_gate(a[t]);
  const double tot = block_sum_f64(s, part);
  if (tid == 0) L[(size_t)u * (T + 1) + min((b + 1) * kScanBlock, T)] = tot;
}

__global__ void log_decay_totals_kernel(double* L, double* lrun, int T, int U) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= U) return;
  double* Lu = L + (size_t)u * (T + 1);
  double run = lrun[u];
  Lu[0] = run;
  for (int e = kScanBlock; e - kScanBlock < T; e += kScanBlock) {
    const int eb = min(e, T);
    run += Lu[eb];
    Lu[eb] = run;
  }
  lrun[u] = run;
}

__global__ void __launch_bounds__(kScanThreads) log_decay_scan_kernel(const float* alpha, double* L, int T) {
  __shared__ double part[kScanThreads];
  const int u = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
  const float* a = alpha + (size_t)u * T;
  double* Lu = L + (size_t)u * (T + 1);
  const int lo = b * kScanBlock + tid * kScanPer, hi = min(T, lo + kScanPer);
  const int eb = min((b + 1) * kScanBlock, T);
  double s = 0.0;
  for (int t = lo; t < hi; ++t) s += log_gate(a[t]);
  // inclusive scan of the per-thread sums (Hillis-Steele over LDS)
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const double add = tid >= off ? part[tid - off] : 0.0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  double run = Lu[b * kScanBlock] + (tid > 0 ? part[tid - 1] : 0.0);
  for (int t = lo; t < hi; ++t) {
    run += log_gate(a[t]);
    if (t + 1 != eb) Lu[t + 1] = run;
  }
}

struct PassArgs {
  const uint32_t* pk;  // [U][T][E] packed slot words (write slots, then read slots)
  const double* L;     // [U][T + 1]
  double* lam;         // [U][N] in/out
  float* fac;          // [U][T][E] out (first holds each outside-window access's latest writer)
  int* lastw;          // [U][N] latest writer of each slot in this call, -1 = none
  int* segl;           // [U][nseg - 1][N] latest writer of each slot within each segment but the last
  int U, T, W, E, P, span, chunk;
  int nseg, seglen;    // token segments per unit (seglen a multiple of chunk)
  long long N;
};

// Latest writer of every slot of one range within one token segment (all but a unit's last
// segment): the largest token of the segment that writes the slot, -1 if none does.
__global__ void __launch_bounds__(kPassThreads) decay_seglast_kernel(PassArgs A) {
  extern __shared__ int last_tok[];  // [span]
  const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int per_unit = A.P * (A.nseg - 1);
  const int u = xcd + 8 * (k / per_unit), p = k % per_unit % A.P, seg = k % per_unit / A.P, tid = threadIdx.x;
  if (u >= A.U) return;
  const int E = A.E, W = A.W, span = A.span;
  const long long n0 = (long long)p * span;
  for (int i = tid; i < span; i += kPassThreads) last_tok[i] = -1;
  __syncthreads();
  const int t_lo = min(A.T, seg * A.seglen), t_hi = min(A.T, t_lo + A.seglen);
  const uint32_t* pk = A.pk + ((size_t)u * A.T + t_lo) * E;
  const int nw = (t_hi - t_lo) * E;
  for (int q0 = 0; q0 < nw; q0 += kPerThread * kPassThreads) {
    uint32_t w[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int q = q0 + tid + r * kPassThreads;
      w[r] = q < nw ? pk[q] : kInvalid;
    }
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int q = q0 + tid + r * kPassThreads;
      if ((w[r] & (kCoded | kInvalid)) == kInvalid || q % E >= W) continue;
      const long long n = w[r] & kSlotMask;
      if (n >= n0 && n < n0 + span) atomicMax(&last_tok[n - n0], t_lo + q / E);
    }
  }
  __syncthreads();
  int* out = A.segl + ((size_t)u * (A.nseg - 1) + seg) * A.N;
  for (int i = tid; i < span; i += kPassThreads)
    if (n0 + i < A.N) out[n0 + i] = last_tok[i];
}

// Order pass: one workgroup per (unit, range of `span` slots, token segment), tokens in
// chunks of at most `win`. The record starts as the latest writer over the earlier
// segments. An access with no writer inside the window sees no write since its chunk
// began, so the record of the latest writer as of the chunk start (LDS) is its latest
// writer; it is left, as an int, in the access's factor word. Then the chunk's writes
// update the record. The next chunk's slot words are loaded while a chunk is processed;
// the loop touches nothing but LDS and registers otherwise. All workgroups of a unit run
// on one XCD.
__global__ void __launch_bounds__(kPassThreads) decay_order_kernel(PassArgs A) {
  extern __shared__ int last_tok[];  // [span]
  const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int per_unit = A.P * A.nseg;
  const int u = xcd + 8 * (k / per_unit), p = k % per_unit % A.P, seg = k % per_unit / A.P, tid = threadIdx.x;
  if (u >= A.U) return;
  const int W = A.W, E = A.E, span = A.span, C = A.chunk;
  const int t_lo = min(A.T, seg * A.seglen), T = min(A.T, t_lo + A.seglen);  // this segment: [t_lo, T)
  const long long n0 = (long long)p * span;
  const int* prev = A.segl + (size_t)u * (A.nseg - 1) * A.N + n0;
  for (int i = tid; i < span; i += kPassThreads) {
    int lt = -1;
    for (int sg = 0; sg < seg; ++sg)
      if (n0 + i < A.N) lt = max(lt, prev[(size_t)sg * A.N + i]);
    last_tok[i] = lt;
  }
  const uint32_t* pk = A.pk + (size_t)u * A.T * E;
  int* lt_out = (int*)(A.fac + (size_t)u * A.T * E);
  const int per = C * E;  // accesses per chunk, at most kPerThread * kPassThreads
  uint32_t cur[kPerThread], nxt[kPerThread];
  auto load = [&](int c0, uint32_t (&w)[kPerThread]) {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int q = tid + r * kPassThreads;
      const long long i = (long long)c0 * E + q;
      w[r] = (q < per && i < (long long)T * E) ? pk[i] : kInvalid;
    }
  };
  load(t_lo, cur);
  __syncthreads();
  for (int c0 = t_lo; c0 < T; c0 += C) {
    load(c0 + C, nxt);
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const uint32_t w = cur[r];
      if (w & (kCoded | kInvalid)) continue;  // inside the window, or outside [0, N)
      const long long n = w & kSlotMask;
      if (n < n0 || n >= n0 + span) continue;
      lt_out[(size_t)c0 * E + tid + r * kPassThreads] = last_tok[n - n0];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int q = tid + r * kPassThreads;
      const uint32_t w = cur[r];
      if ((w & (kCoded | kInvalid)) == kInvalid || q % E >= W) continue;
      const long long n = w & kSlotMask;
      if (n >= n0 && n < n0 + span) atomicMax(&last_tok[n - n0], c0 + q / E);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) cur[r] = nxt[r];
  }
  if (seg != A.nseg - 1) return;  // the last segment's record is the call's latest writer
  int* lastw = A.lastw + (size_t)u * A.N;
  for (int i = tid; i < span; i += kPassThreads)
    if (n0 + i < A.N) lastw[n0 + i] = last_tok[i];
}

// Factor of every access (one thread each), from the window's writer or the order pass's.
__global__ void __launch_bounds__(256) decay_factor_kernel(PassArgs A) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per_unit = (long long)A.T * A.E;
  if (i >= per_unit * A.U) return;
  const int u = (int)(i / per_unit);
  const long long iu = i - (long long)u * per_unit;
  const int t = (int)(iu / A.E), e = (int)(iu - (long long)t * A.E);
  const uint32_t w = A.pk[i];
  const double* L = A.L + (size_t)u * (A.T + 1);
  float f = 1.f;  // also for a slot outside [0, N): it carries no weight
  if ((w & (kCoded | kInvalid)) != kInvalid) {
    const double to = e >= A.W ? L[t + 1] : L[t];
    if (w & kCoded) {
      const int d = (w >> 24) & 127;
      if (d > 0) f = decay_factor(to, L[t - d + 1]);
    } else {
      const int lt = __float_as_int(A.fac[i]);
      f = decay_factor(to, lt >= 0 ? L[lt + 1] : A.lam[(size_t)u * A.N + (w & kSlotMask)]);
    }
  }
  A.fac[i] = f;
}

// lam of every slot written in this call: the cumulative log-decay after its latest writer.
__global__ void __launch_bounds__(256) decay_lam_kernel(PassArgs A) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)A.U * A.N) return;
  const int lt = A.lastw[i];
  if (lt >= 0) A.lam[i] = A.L[(size_t)(i / A.N) * (A.T + 1) + lt + 1];
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
  const int U = S.B * S.H, nb = (S.T + kScanBlock - 1) / kScanBlock;
  hipError_t e;
  if (nb > 0) {
    hipLaunchKernelGGL(log_decay_sums_kernel, dim3(nb, U), dim3(kScanThreads), 0, stream, alpha, L, S.T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(log_decay_totals_kernel, dim3((U + 63) / 64), dim3(64), 0, stream, L, lrun, S.T, U);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nb > 0) {
    hipLaunchKernelGGL(log_decay_scan_kernel, dim3(nb, U), dim3(kScanThreads), 0, stream, alpha, L, S.T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

int decay_pass_ranges(const sdm_shape& S) { return (int)((S.N + kPassSlotsMax - 1) / kPassSlotsMax); }

// Token segments per unit for the order pass: enough (at most 4) for the workgroups to cover
// the 256 compute units, each segment at least 2048 tokens long (shorter walks do not repay
// the extra pass).
int decay_segments(const sdm_shape& S) {
  const long long wgs = (long long)S.B * S.H * decay_pass_ranges(S);
  int nseg = wgs >= 256 ? 1 : (int)std::min<long long>(4, 256 / wgs);
  while (nseg > 1 && S.T < 2048LL * nseg) --nseg;
  return nseg;
}

hipError_t launch_decay_pass(const sdm_shape& S, const uint32_t* pk, const double* L, double* lam, float* fac,
                             int* lastw, int* segl, int win, hipStream_t stream) {
  PassArgs A;
  A.pk = pk;
  A.L = L;
  A.lam = lam;
  A.fac = fac;
  A.lastw = lastw;
  A.U = S.B * S.H;
  A.T = S.T;
  A.W = S.W;
  A.E = S.W + S.R;
  A.P = decay_pass_ranges(S);
  A.span = (int)((S.N + A.P - 1) / A.P);
  A.N = S.N;
  // the longest chunk inside the window whose accesses fit the threads' registers
  A.chunk = std::min(win, kPerThread * kPassThreads / A.E);
  if (A.chunk < 1) return hipErrorInvalidValue;
  A.segl = segl;
  A.nseg = decay_segments(S);
  A.seglen = (S.T + A.nseg - 1) / A.nseg;
  A.seglen = (A.seglen + A.chunk - 1) / A.chunk * A.chunk;
  const int groups = (A.U + 7) / 8;
  hipError_t e;
  if (A.nseg > 1) {
    hipLaunchKernelGGL(decay_seglast_kernel, dim3(8 * groups * A.P * (A.nseg - 1)), dim3(kPassThreads),
                       (size_t)A.span * 4, stream, A);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decay_order_kernel, dim3(8 * groups * A.P * A.nseg), dim3(kPassThreads), (size_t)A.span * 4,
                     stream, A);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long acc = (long long)A.U * A.T * A.E;
  hipLaunchKernelGGL(decay_factor_kernel, dim3((unsigned)((acc + 255) / 256)), dim3(256), 0, stream, A);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long slots = (long long)A.U * S.N;
  hipLaunchKernelGGL(decay_lam_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, stream, A);
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
