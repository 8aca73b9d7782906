// The steps on either side of the recurrence: gates from their pre-activations, and the
// output of each token (RMS normalisation, elementwise gate, mixing of the heads).
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, App. B "Gate dynamics": forget gate
// exp(g), input gate sigma(b); §4 "SDM Configuration": forget gate and time-step bias as in
// Gated DeltaNet; §3 "Sparse retrieval": the read is RMS-normalised, elementwise gated and
// projected into the layer output):
//   alpha = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])),  beta = sigmoid(b)
//   x[t, h, :] = o[t, h, :] / rms(o[t, h, :]) * w * silu(z[t, h, :])      (bf16)
//   y[t, :]    = Wo . concat_h x[t, h, :]                                 (MFMA, float32)

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

// ------------------------------------------------------------------ gates
__global__ void __launch_bounds__(256) gates_kernel(const float* a, const float* b, const float* A_log,
                                                    const float* dt_bias, float* alpha, float* beta, int H, int T,
                                                    long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int h = (int)((i / T) % H);
  const float x = a[i] + dt_bias[h];
  const float sp = x > 20.f ? x : log1pf(expf(x));  // softplus
  alpha[i] = expf(-expf(A_log[h]) * sp);
  beta[i] = 1.f / (1.f + expf(-b[i]));
}

// ------------------------------------------------------------------ normalisation and gate
// One wave per token-head: o [B,H,T,d_v] f32 -> x [B,T,H,d_v] bf16 (token-major, the layout
// the head mixing reads); z [B,T,H,d_v] in_dtype.
template <bool ZBF16>
__global__ void __launch_bounds__(256) output_gate_kernel(const float* o, const void* z, const float* w, float eps,
                                                          uint16_t* x, int H, int T, int d_v, long long units) {
  const long long th = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, h, t)
  const int lane = threadIdx.x & 63;
  if (th >= units) return;
  const int t = (int)(th % T);
  const long long bh = th / T;
  const int h = (int)(bh % H);
  const long long b = bh / H;
  const float* orow = o + th * d_v;
  const long long tok = (b * T + t) * H + h;  // row of x and z
  float ss = 0.f;
  for (int c = lane; c < d_v; c += 64) ss = fmaf(orow[c], orow[c], ss);
  const float r = rsqrtf(wave_sum_f32(ss) / (float)d_v + eps);
  for (int c = lane; c < d_v; c += 64) {
    const float zz = ZBF16 ? bf16_to_f32(((const uint16_t*)z)[tok * d_v + c]) : ((const float*)z)[tok * d_v + c];
    const float y = orow[c] * r * w[c] * (zz / (1.f + expf(-zz)));
    x[tok * d_v + c] = (uint16_t)pack_bf16x2(y, 0.f);
  }
}

// ------------------------------------------------------------------ head mixing
// y[M, N] = x[M, K] . Wo[N, K]^T, bf16 operands, float32 accumulation on MFMA
// (v_mfma_f32_32x32x16_bf16). Workgroup tile 128 x 128 (four waves, 64 x 64 each); K in
// steps of 64 staged through LDS, the next step's global loads in flight while the current
// one is multiplied. Each lane takes 8 consecutive k of its row of x and of Wo for one MFMA:
// the same split of k for both operands, so the products pair up whatever the instruction's
// internal order of k. Rows of the LDS tiles are padded to 72 bf16 (144 bytes) so that the
// 16-byte fragment reads stay aligned.
constexpr int kMixTile = 128;
constexpr int kMixK = 64;
constexpr int kMixPad = 72;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) head_mix_kernel(const uint16_t* X, const uint16_t* Wo, float* Y, long long M,
                                                       int K, int N) {
  __shared__ __align__(16) uint16_t As[kMixTile * kMixPad];
  __shared__ __align__(16) uint16_t Bs[kMixTile * kMixPad];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long long m0 = (long long)blockIdx.x * kMixTile;
  const int n0 = blockIdx.y * kMixTile;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  float16_t acc[2][2] = {};
  // staging: 128 rows x 64 k of each operand = 1024 pieces of 8 bf16, four per thread
  uint4 ra[4], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = tid + r * 256, row = q >> 3, kk = (q & 7) * 8;
      const bool kin = k0 + kk < K;  // K is a multiple of 32: the last step may be half full
      ra[r] = kin && m0 + row < M ? *(const uint4*)(X + (m0 + row) * (long long)K + k0 + kk) : make_uint4(0u, 0u, 0u, 0u);
      rb[r] = kin && n0 + row < N ? *(const uint4*)(Wo + (long long)(n0 + row) * K + k0 + kk) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  load(0);
  for (int k0 = 0; k0 < K; k0 += kMixK) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = tid + r * 256, row = q >> 3, kk = (q & 7) * 8;
      *(uint4*)(As + row * kMixPad + kk) = ra[r];
      *(uint4*)(Bs + row * kMixPad + kk) = rb[r];
    }
    __syncthreads();
    if (k0 + kMixK < K) load(k0 + kMixK);
#pragma unroll
    for (int ks = 0; ks < kMixK; ks += 16) {
      bf16x8_t af[2], bf[2];
      const int kq = ks + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(As + (wm + i * 32 + (lane & 31)) * kMixPad + kq));
        bf[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(Bs + (wn + i * 32 + (lane & 31)) * kMixPad + kq));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // D[row][col]: lane holds col = lane % 32, rows 8*(e/4) + 4*(lane/32) + e%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const long long row = m0 + wm + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row < M) Y[row * N + col] = acc[i][j][e];
      }
    }
}

}  // namespace

hipError_t launch_gates(const sdm_shape& S, const float* a, const float* b, const float* A_log, const float* dt_bias,
                        float* alpha, float* beta, hipStream_t stream) {
  const long long n = (long long)S.B * S.H * S.T;
  hipLaunchKernelGGL(gates_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, b, A_log, dt_bias,
                     alpha, beta, S.H, S.T, n);
  return hipGetLastError();
}

hipError_t launch_output_gate(const sdm_shape& S, const float* o, const void* z, const float* w, float eps,
                              uint16_t* x, hipStream_t stream) {
  const long long units = (long long)S.B * S.H * S.T;
  const dim3 grid((unsigned)((units + 3) / 4));
  if (S.in_dtype == SDM_BF16)
    hipLaunchKernelGGL(output_gate_kernel<true>, grid, dim3(256), 0, stream, o, z, w, eps, x, S.H, S.T, S.d_v, units);
  else
    hipLaunchKernelGGL(output_gate_kernel<false>, grid, dim3(256), 0, stream, o, z, w, eps, x, S.H, S.T, S.d_v, units);
  return hipGetLastError();
}

hipError_t launch_head_mix(const uint16_t* x, const uint16_t* Wo, float* y, long long M, int K, int N,
                           hipStream_t stream) {
  const dim3 grid((unsigned)((M + kMixTile - 1) / kMixTile), (unsigned)((N + kMixTile - 1) / kMixTile));
  hipLaunchKernelGGL(head_mix_kernel, grid, dim3(256), 0, stream, x, Wo, y, M, K, N);
  return hipGetLastError();
}

}  // namespace sdm
