// Memory-table kernels: M0 copy-on-init and the sequential sparse gated-delta recurrence.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1): §3 "Learned initial state" -- each
// sequence's table starts as a copy of M0; §2 "Gated DeltaNet" and §3 "Sparse memory
// updates" -- a token reads the weighted sum of its W write slots, decays it by alpha,
// forms the residual against v scaled by beta, and writes alpha*old + weight*residual
// back to those W slots only; §3 "Sparse retrieval" -- the token's output is the weighted
// sum of its R read slots, read after its write.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

// ---------------------------------------------------------------- M0 copy-on-init
// Each thread moves 16-byte chunks: one read of M0[h], B writes (one per sequence).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// chunks = H * N * rowbytes / 16 (one head-major copy of M0); M holds B such copies. The
// kernel moves chunks [c0, c1).
__global__ void __launch_bounds__(256) init_kernel(const u32x4* __restrict__ M0, u32x4* __restrict__ M, int B,
                                                   size_t chunks, size_t c0, size_t c1) {
  for (size_t i = c0 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < c1; i += (size_t)gridDim.x * blockDim.x) {
    u32x4 v = __builtin_nontemporal_load(&M0[i]);
    for (int b = 0; b < B; ++b) __builtin_nontemporal_store(v, &M[(size_t)b * chunks + i]);
  }
}

// ---------------------------------------------------------------- recurrence (sequential)
// One wave per (unit, block of up to 64 row dwords). Lane owns one 32-bit word of every row
// (two bf16 columns or one float32 column). Tokens are processed in order; every load of a
// row is issued after the same lane's earlier stores to it, so program order alone makes
// each token see the writes of all earlier tokens.
template <typename MemT>
struct MemTraits;
template <>
struct MemTraits<float> {
  static constexpr int kCols = 1;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = __uint_as_float(w); }
  __device__ static uint32_t pack(const float* x) { return __float_as_uint(x[0]); }
};
template <>
struct MemTraits<uint16_t> {  // bf16
  static constexpr int kCols = 2;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = bf16lo(w); x[1] = bf16hi(w); }
  __device__ static uint32_t pack(const float* x) { return pack_bf16x2(x[0], x[1]); }
};

template <typename InT>
__device__ __forceinline__ float in_val(const InT* p, size_t i);
template <>
__device__ __forceinline__ float in_val<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float in_val<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

struct RecArgs {
  const int32_t* widx;
  const float* wgt;
  const int32_t* ridx;
  const float* rgt;
  const void* v;
  const float* alpha;
  const float* beta;
  void* M;
  float* o;
  uint32_t* xlog;  // optional [U][T][W][d_v] log of the pre-update written rows
  unsigned long long* err;
  int U, T, W, R, d_v;
  long long N;
};

template <typename MemT, typename InT>
__global__ void __launch_bounds__(64) recurrent_seq_kernel(RecArgs A) {
  using MT = MemTraits<MemT>;
  constexpr int CPL = MT::kCols;
  const int u = blockIdx.y;
  const int lane = threadIdx.x;
  const int rowdw = A.d_v / CPL;
  const int dw = blockIdx.x * 64 + lane;
  const bool active = dw < rowdw;
  const int dwc = active ? dw : 0;
  uint32_t* Mu = (uint32_t*)A.M + (size_t)u * (size_t)A.N * rowdw;
  const InT* v = (const InT*)A.v;
  const long long N = A.N;
  for (int t = 0; t < A.T; ++t) {
    const size_t ut = (size_t)u * A.T + t;
    const float al = A.alpha[ut], be = A.beta[ut];
    const int32_t* wi = A.widx + ut * A.W;
    const float* ww = A.wgt + ut * A.W;
    const int32_t* ri = A.ridx + ut * A.R;
    const float* rw = A.rgt + ut * A.R;
    // decayed weighted read of the write slots
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    for (int j = 0; j < A.W; ++j) {
      const int n = wi[j];
      if (n < 0 || n >= N) continue;
      float x[CPL];
      MT::unpack(Mu[(size_t)n * rowdw + dwc], x);
      const float a = ww[j];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(a, x[c], acc[c]);
    }
    float delta[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float vv = in_val<InT>(v, ut * A.d_v + (size_t)dwc * CPL + c);
      delta[c] = be * (vv - al * acc[c]);
    }
    // gated delta write of the W slots (old values re-read; they are unchanged)
    for (int j = 0; j < A.W; ++j) {
      const int n = wi[j];
      uint32_t* lg = A.xlog ? A.xlog + (ut * A.W + j) * rowdw + dwc : nullptr;
      if (n < 0 || n >= N) {
        if (lane == 0 && blockIdx.x == 0) atomicAdd(A.err, 1ull);
        if (lg && active) *lg = 0u;  // no row: the log holds zeros
        continue;
      }
      uint32_t* p = &Mu[(size_t)n * rowdw + dwc];
      float x[CPL], y[CPL];
      const uint32_t old = *p;
      if (lg && active) *lg = old;  // the row as this token reads it, before its write
      MT::unpack(old, x);
      const float a = ww[j];
#pragma unroll
      for (int c = 0; c < CPL; ++c) y[c] = fmaf(al, x[c], a * delta[c]);
      if (active) *p = MT::pack(y);
    }
    // weighted read of the R slots, after the write
    float o[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = 0.f;
    for (int r = 0; r < A.R; ++r) {
      const int m = ri[r];
      if (m < 0 || m >= N) {
        if (lane == 0 && blockIdx.x == 0) atomicAdd(A.err, 1ull);
        continue;
      }
      float x[CPL];
      MT::unpack(Mu[(size_t)m * rowdw + dwc], x);
      const float w = rw[r];
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] = fmaf(w, x[c], o[c]);
    }
    if (active) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) A.o[ut * A.d_v + (size_t)dw * CPL + c] = o[c];
    }
  }
}

template <typename MemT, typename InT>
hipError_t launch_seq(const RecArgs& A, hipStream_t st) {
  constexpr int CPL = MemTraits<MemT>::kCols;
  const int rowdw = A.d_v / CPL;
  dim3 grid((rowdw + 63) / 64, A.U);
  hipLaunchKernelGGL((recurrent_seq_kernel<MemT, InT>), grid, dim3(64), 0, st, A);
  return hipGetLastError();
}

__global__ void zero_kernel(unsigned long long* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0ull;
}

}  // namespace

// Clears n 8-byte words with a kernel (not a memset node, so the call can be captured).
hipError_t launch_zero(void* p, size_t n_words, hipStream_t stream) {
  if (n_words == 0) return hipSuccess;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (unsigned long long*)p, n_words);
  return hipGetLastError();
}

hipError_t launch_init_part(const sdm_shape& S, const void* M0, void* M, size_t c0, size_t c1, hipStream_t stream) {
  const size_t rowbytes = (size_t)S.d_v * dtype_size(S.mem_dtype);
  const size_t chunks = (size_t)S.H * (size_t)S.N * rowbytes / 16;
  if (c1 > chunks) c1 = chunks;
  if (c1 <= c0 || S.B == 0) return hipSuccess;
  size_t blocks = (c1 - c0 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(init_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)M0, (u32x4*)M, S.B,
                     chunks, c0, c1);
  return hipGetLastError();
}

hipError_t launch_init(const sdm_shape& S, const void* M0, void* M, hipStream_t stream) {
  return launch_init_part(S, M0, M, 0, ~(size_t)0, stream);
}

hipError_t launch_recurrent(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                            const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                            void* ws, const WsLayout& L, const DecayState* dk, hipStream_t stream, void* xlog) {
  RecArgs A;
  A.widx = widx;
  A.wgt = wgt;
  A.ridx = ridx;
  A.rgt = rgt;
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  A.M = M;
  A.o = o;
  A.xlog = (uint32_t*)xlog;
  A.err = (unsigned long long*)((char*)ws + L.err);
  A.U = S.B * S.H;
  A.T = S.T;
  A.W = S.W;
  A.R = S.R;
  A.d_v = S.d_v;
  A.N = S.N;
  if (A.U == 0 || A.T == 0) return hipSuccess;
  if (dataflow_supported(S, dk != nullptr))
    return launch_dataflow(S, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, L, dk, xlog, stream);
  if (dk) return hipErrorInvalidValue;  // the whole-table decay runs on the pipeline only
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return launch_seq<uint16_t, uint16_t>(A, stream);
  if (mb && !ib) return launch_seq<uint16_t, float>(A, stream);
  if (!mb && ib) return launch_seq<float, uint16_t>(A, stream);
  return launch_seq<float, float>(A, stream);
}

}  // namespace sdm
