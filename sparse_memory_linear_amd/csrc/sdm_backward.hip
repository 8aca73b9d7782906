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
// Every column of the table and of G evolves on its own, so a wave owns 64 columns of one
// unit and walks all its tokens: each lane touches only its own column of every row, and
// needs no synchronisation with other lanes or waves for the table. The scalar gradients
// (sums over columns) are reduced in the wave through LDS and added across the column
// blocks with atomics into outputs zeroed first.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kCols = 64;      // columns per wave
constexpr int kMaxSel = 64;    // W, R <= 64

template <typename T>
__device__ __forceinline__ float ld_val(const T* p, size_t i) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(p[i]);
  else return p[i];
}
template <typename T>
__device__ __forceinline__ void st_val(T* p, size_t i, float x) {
  if constexpr (sizeof(T) == 2) p[i] = (uint16_t)pack_bf16x2(x, 0.f);
  else p[i] = x;
}

struct BwdArgs {
  const int32_t* widx;  // [U][T][W]
  const float* wgt;
  const int32_t* ridx;  // [U][T][R]
  const float* rgt;
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
  int T, W, R, d_v, P;
  long long N;
};

template <typename MemT, typename InT>
__global__ void __launch_bounds__(64) backward_kernel(BwdArgs A) {
  __shared__ int sn[kMaxSel], sm[kMaxSel];
  __shared__ float sa[kMaxSel], su[kMaxSel];
  __shared__ float part[2 * kMaxSel + 2][kCols + 1];  // per-lane partial sums, padded rows
  const int lane = threadIdx.x;
  const int u = blockIdx.x / A.P, p = blockIdx.x % A.P;
  const int c = p * kCols + lane;
  const bool act = c < A.d_v;
  const int T = A.T, W = A.W, R = A.R, d_v = A.d_v;
  MemT* M = (MemT*)A.M + (size_t)u * A.N * d_v;
  float* G = A.G + (size_t)u * A.N * d_v;
  const MemT* xlog = (const MemT*)A.xlog + (size_t)u * T * W * d_v;
  const InT* v = (const InT*)A.v + (size_t)u * T * d_v;
  const size_t ut = (size_t)u * T;
  float x[kMaxSel], dy[kMaxSel];
  for (int t = T - 1; t >= 0; --t) {
    if (lane < W) {
      sn[lane] = A.widx[(ut + t) * W + lane];
      sa[lane] = A.wgt[(ut + t) * W + lane];
    }
    if (lane < R) {
      sm[lane] = A.ridx[(ut + t) * R + lane];
      su[lane] = A.rgt[(ut + t) * R + lane];
    }
    __syncthreads();
    const float al = A.alpha[ut + t], be = A.beta[ut + t];
    const float g = act ? A.go[(ut + t) * d_v + c] : 0.f;
    const float vc = act ? ld_val((const InT*)v, (size_t)t * d_v + c) : 0.f;
    // read after the write (slots outside [0, N) carry no weight and are skipped)
    for (int r = 0; r < R; ++r) {
      const bool ok = sm[r] >= 0 && sm[r] < A.N;
      const size_t e = ok ? (size_t)sm[r] * d_v + c : 0;
      float pr = 0.f;
      if (act && ok) {
        pr = g * ld_val((const MemT*)M, e);
        G[e] += su[r] * g;
      }
      part[W + r][lane] = pr;
    }
    // write: x_j from the log, dy_j the gradient of the written values
    float s = 0.f, dd = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxSel; ++j) {
      if (j < W) {
        const bool ok = act && sn[j] >= 0 && sn[j] < A.N;
        x[j] = ok ? ld_val(xlog, ((size_t)t * W + j) * d_v + c) : 0.f;
        dy[j] = ok ? G[(size_t)sn[j] * d_v + c] : 0.f;
        s = fmaf(sa[j], x[j], s);
        dd = fmaf(sa[j], dy[j], dd);
      }
    }
    const float resid = vc - al * s, delta = be * resid, drho = -be * dd;
    float pal = drho * s;
#pragma unroll
    for (int j = 0; j < kMaxSel; ++j) {
      if (j < W) {
        part[j][lane] = dy[j] * delta + al * drho * x[j];
        pal = fmaf(dy[j], x[j], pal);
        if (act && sn[j] >= 0 && sn[j] < A.N) {
          const size_t e = (size_t)sn[j] * d_v + c;
          G[e] = al * dy[j] + al * sa[j] * drho;
          st_val(M, e, x[j]);
        }
      }
    }
    part[W + R][lane] = pal;
    part[W + R + 1][lane] = dd * resid;
    if (act) A.dv[(ut + t) * d_v + c] = be * dd;
    __syncthreads();
    // sums over this wave's columns: lane i adds row i, then one atomic per block
    for (int i = lane; i < W + R + 2; i += kCols) {
      float sum = 0.f;
      for (int k = 0; k < kCols; ++k) sum += part[i][k];
      float* dst = i < W ? A.dwgt + (ut + t) * W + i
                         : i < W + R ? A.drgt + (ut + t) * R + (i - W)
                                     : i == W + R ? A.dalpha + ut + t : A.dbeta + ut + t;
      atomicAdd(dst, sum);
    }
    __syncthreads();
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

template <typename MemT, typename InT>
hipError_t launch_bwd(const BwdArgs& A, int U, hipStream_t st) {
  hipLaunchKernelGGL((backward_kernel<MemT, InT>), dim3(U * A.P), dim3(64), 0, st, A);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                           const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                           const void* xlog, const float* go, float* G, float* dv, float* dalpha, float* dbeta,
                           float* dwgt, float* drgt, hipStream_t stream) {
  if (S.W > kMaxSel || S.R > kMaxSel) return hipErrorInvalidValue;
  const int U = S.B * S.H;
  const size_t tok = (size_t)U * S.T;
  hipError_t e = zero_f32(dalpha, tok, stream);
  if (e != hipSuccess) return e;
  e = zero_f32(dbeta, tok, stream);
  if (e != hipSuccess) return e;
  e = zero_f32(dwgt, tok * S.W, stream);
  if (e != hipSuccess) return e;
  e = zero_f32(drgt, tok * S.R, stream);
  if (e != hipSuccess) return e;
  BwdArgs A;
  A.widx = widx;
  A.wgt = wgt;
  A.ridx = ridx;
  A.rgt = rgt;
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
  A.T = S.T;
  A.W = S.W;
  A.R = S.R;
  A.d_v = S.d_v;
  A.P = (S.d_v + kCols - 1) / kCols;
  A.N = S.N;
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return launch_bwd<uint16_t, uint16_t>(A, U, stream);
  if (mb && !ib) return launch_bwd<uint16_t, float>(A, U, stream);
  if (!mb && ib) return launch_bwd<float, uint16_t>(A, U, stream);
  return launch_bwd<float, float>(A, U, stream);
}

}  // namespace sdm
