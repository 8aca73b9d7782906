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

// Same output for d_v in {32, 64, 128, 256}: DV / 8 lanes per token-head, 8 values each
// (two 16-byte loads of o, one or two of z, one 16-byte store of x), 64 / (DV / 8)
// token-heads per wave; the sum of squares is a reduction over the token-head's lanes.
template <bool ZBF16, int DV>
__global__ void __launch_bounds__(256) output_gate_vec_kernel(const float* o, const void* z, const float* w,
                                                              float eps, uint16_t* x, int H, int T, long long units) {
  constexpr int L = DV / 8;
  const long long th = ((long long)blockIdx.x * 256 + threadIdx.x) / L;  // (b, h, t)
  const int cp = (threadIdx.x % L) * 8;
  const bool live = th < units;  // every lane takes part in the reduction
  const long long thc = live ? th : units - 1;
  const int t = (int)(thc % T);
  const long long bh = thc / T;
  const int h = (int)(bh % H);
  const long long b = bh / H;
  const float* orow = o + thc * DV + cp;
  const float4 o0 = *(const float4*)orow, o1 = *(const float4*)(orow + 4);
  const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
  const long long zo = ((b * T + t) * H + h) * DV + cp;  // row of x and z
  float zv[8];
  if (ZBF16) {
    const uint4 zq = *(const uint4*)((const uint16_t*)z + zo);
    const uint32_t zw[4] = {zq.x, zq.y, zq.z, zq.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) zv[c] = (c & 1) ? bf16hi(zw[c >> 1]) : bf16lo(zw[c >> 1]);
  } else {
    const float4 z0 = *(const float4*)((const float*)z + zo), z1 = *(const float4*)((const float*)z + zo + 4);
    zv[0] = z0.x; zv[1] = z0.y; zv[2] = z0.z; zv[3] = z0.w;
    zv[4] = z1.x; zv[5] = z1.y; zv[6] = z1.z; zv[7] = z1.w;
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) ss = fmaf(ov[c], ov[c], ss);
#pragma unroll
  for (int m = 1; m < L; m <<= 1) ss = add_xor_f32(ss, m);
  const float r = rsqrtf(ss / (float)DV + eps);
  uint32_t xw[4];
#pragma unroll
  for (int c = 0; c < 8; c += 2) {
    const float y0 = ov[c] * r * w[cp + c] * (zv[c] / (1.f + expf(-zv[c])));
    const float y1 = ov[c + 1] * r * w[cp + c + 1] * (zv[c + 1] / (1.f + expf(-zv[c + 1])));
    xw[c >> 1] = pack_bf16x2(y0, y1);
  }
  if (live) *(uint4*)(x + zo) = make_uint4(xw[0], xw[1], xw[2], xw[3]);
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

// ------------------------------------------------------------------ gate fused into mixing
// y[m, n] = sum_h sum_c x[m, h, c] Wo[n, h d_v + c] with x = the bf16 output of the
// normalisation and gate above, never written to memory. One workgroup (8 waves) owns RM
// rows (tokens) and every column of y:
//   1. x for its rows and all K = H d_v columns goes into LDS: each head's row piece of d_v
//      values is loaded by DV / 8 lanes (8 values each), whose sum of squares is a reduction
//      over those lanes; o is read once, in float32, straight from the recurrence's output.
//   2. each wave takes groups of 64 output columns in turn and multiplies the resident x by
//      those 64 rows of Wo: x fragments come from LDS, Wo fragments straight from memory into
//      registers (no wave shares them, so staging them through LDS would buy nothing), loaded
//      four K steps ahead of the MFMAs. No barrier in this part.
// The gate of every token-head is thus evaluated once, whatever d_model is.
constexpr int kProjThreads = 512;
constexpr int kProjAhead = 4;  // K steps of 16 whose Wo fragments are in flight

struct OutProjArgs {
  const float* o;     // [B,H,T,DV] f32
  const void* z;      // [B,T,H,DV] bf16 or f32
  const float* w;     // [DV]
  const uint16_t* Wo; // [N, H*DV] bf16
  float* y;           // [B*T, N] f32
  float eps;
  int H, T, N;
  long long M;        // B*T
};

size_t output_project_lds(int rm, int K) { return (size_t)rm * (K + 8) * 2; }

template <bool ZBF16, int DV, int RM>
__global__ void __launch_bounds__(kProjThreads) output_project_kernel(OutProjArgs A) {
  extern __shared__ __align__(16) uint16_t As[];  // [RM][K + 8]
  constexpr int L = DV / 8;                       // lanes per row piece, 8 columns each
  constexpr int RP = kProjThreads / L;            // row pieces per pass
  constexpr int NP = (RM + RP - 1) / RP;          // passes per head
  const int H = A.H, T = A.T, K = A.H * DV, PA = K + 8;
  const long long m0 = (long long)blockIdx.x * RM;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // ---- 1. gated x of the RM rows into LDS
  {
    const int cp = (tid % L) * 8, rr = tid / L;
    int ob[NP], zb[NP];  // o row base b*H*T + t, z row base (b*T + t)*H; -1 past M or past RM
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int row = rr + RP * i;
      const long long m = m0 + row;
      if (row < RM && m < A.M) {
        const int b = (int)(m / T), t = (int)(m % T);
        ob[i] = b * H * T + t;
        zb[i] = (b * T + t) * H;
      } else {
        ob[i] = -1;
        zb[i] = 0;
      }
    }
    float wv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) wv[c] = A.w[cp + c];
    float4 oa[NP][2];
    uint4 za[NP][ZBF16 ? 1 : 2];
    auto load = [&](int h) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (ob[i] >= 0) {
          const float* orow = A.o + (size_t)(ob[i] + h * T) * DV + cp;
          oa[i][0] = *(const float4*)orow;
          oa[i][1] = *(const float4*)(orow + 4);
          const size_t zo = (size_t)(zb[i] + h) * DV + cp;
          if (ZBF16) {
            za[i][0] = *(const uint4*)((const uint16_t*)A.z + zo);
          } else {
            za[i][0] = *(const uint4*)((const float*)A.z + zo);
            za[i][ZBF16 ? 0 : 1] = *(const uint4*)((const float*)A.z + zo + 4);  // (index 1 when float32)
          }
        } else {
          oa[i][0] = oa[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    };
    load(0);
    for (int h = 0; h < H; ++h) {
      float ov[NP][8];
      uint32_t zw[NP][ZBF16 ? 4 : 8];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        ov[i][0] = oa[i][0].x; ov[i][1] = oa[i][0].y; ov[i][2] = oa[i][0].z; ov[i][3] = oa[i][0].w;
        ov[i][4] = oa[i][1].x; ov[i][5] = oa[i][1].y; ov[i][6] = oa[i][1].z; ov[i][7] = oa[i][1].w;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(za[i]);
#pragma unroll
        for (int q = 0; q < (ZBF16 ? 4 : 8); ++q) zw[i][q] = src[q];
      }
      if (h + 1 < H) load(h + 1);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) ss = fmaf(ov[i][c], ov[i][c], ss);
#pragma unroll
        for (int m = 1; m < L; m <<= 1) ss = add_xor_f32(ss, m);
        const float r = rsqrtf(ss / (float)DV + A.eps);
        uint32_t xw[4];
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
          float zz[2];
#pragma unroll
          for (int e = 0; e < 2; ++e)
            zz[e] = ZBF16 ? (((c + e) & 1) ? bf16hi(zw[i][(c + e) >> 1]) : bf16lo(zw[i][(c + e) >> 1]))
                          : __uint_as_float(zw[i][c + e]);
          const float y0 = ov[i][c] * r * wv[c] * (zz[0] / (1.f + expf(-zz[0])));
          const float y1 = ov[i][c + 1] * r * wv[c + 1] * (zz[1] / (1.f + expf(-zz[1])));
          xw[c >> 1] = pack_bf16x2(y0, y1);
        }
        const int row = rr + RP * i;
        if (row < RM)
          *(uint4*)(As + row * PA + h * DV + cp) =
              ob[i] >= 0 ? make_uint4(xw[0], xw[1], xw[2], xw[3]) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __syncthreads();

  // ---- 2. groups of 64 columns against the resident x, one wave per group
  constexpr int RB = RM / 32;  // 32-row blocks
  const int nk = K / 16;       // K steps (K is a multiple of 32)
  const int kq = (lane >> 5) * 8;
  const int groups = (A.N + 63) / 64;
  for (int g = wave; g < groups; g += kProjThreads / 64) {
    // this lane's two rows of Wo (columns of y); past N the row is clamped to N - 1 and its
    // result is not stored
    const uint16_t* wr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) wr[j] = A.Wo + (size_t)min(g * 64 + 32 * j + (lane & 31), A.N - 1) * K + kq;
    float16_t acc[RB][2];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i][0] = acc[i][1] = float16_t{};
    uint4 bq[kProjAhead][2];
#pragma unroll
    for (int d = 0; d < kProjAhead; ++d)
      if (d < nk) {
        bq[d][0] = *(const uint4*)(wr[0] + 16 * d);
        bq[d][1] = *(const uint4*)(wr[1] + 16 * d);
      }
    for (int k0 = 0; k0 < nk; k0 += kProjAhead) {
#pragma unroll
      for (int d = 0; d < kProjAhead; ++d) {
        const int k = k0 + d;
        if (k < nk) {
          const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, bq[d][0]);
          const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, bq[d][1]);
          if (k + kProjAhead < nk) {
            bq[d][0] = *(const uint4*)(wr[0] + 16 * (k + kProjAhead));
            bq[d][1] = *(const uint4*)(wr[1] + 16 * (k + kProjAhead));
          }
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            const bf16x8_t a =
                __builtin_bit_cast(bf16x8_t, *(const uint4*)(As + (i * 32 + (lane & 31)) * PA + 16 * k + kq));
            acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[i][1], 0, 0, 0);
          }
        }
      }
    }
    // D[row][col]: lane holds col = lane % 32, rows 8*(e/4) + 4*(lane/32) + e%4
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = g * 64 + 32 * j + (lane & 31);
      if (col >= A.N) continue;
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const long long row = m0 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (row < A.M) A.y[row * A.N + col] = acc[i][j][e];
        }
    }
  }
}

template <bool ZBF16, int RM>
hipError_t launch_output_project_dv(const OutProjArgs& A, int d_v, hipStream_t stream) {
  const unsigned grid = (unsigned)((A.M + RM - 1) / RM);
  const size_t lds = output_project_lds(RM, A.H * d_v);
  const dim3 blk(kProjThreads);
  switch (d_v) {
    case 32: hipLaunchKernelGGL((output_project_kernel<ZBF16, 32, RM>), dim3(grid), blk, lds, stream, A); break;
    case 64: hipLaunchKernelGGL((output_project_kernel<ZBF16, 64, RM>), dim3(grid), blk, lds, stream, A); break;
    case 128: hipLaunchKernelGGL((output_project_kernel<ZBF16, 128, RM>), dim3(grid), blk, lds, stream, A); break;
    case 256: hipLaunchKernelGGL((output_project_kernel<ZBF16, 256, RM>), dim3(grid), blk, lds, stream, A); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// rows per workgroup: 64 while x of 64 rows fits in LDS, else 32
int output_project_rows(int K) { return output_project_lds(64, K) <= 160 * 1024 ? 64 : 32; }

}  // namespace

bool output_project_supported(int d_v, int H) {
  return (d_v == 32 || d_v == 64 || d_v == 128 || d_v == 256) && output_project_lds(32, H * d_v) <= 160 * 1024;
}

hipError_t launch_output_project(const sdm_shape& S, const float* o, const void* z, const float* w, float eps,
                                 const uint16_t* Wo, int d_model, float* y, hipStream_t stream) {
  if (!output_project_supported(S.d_v, S.H)) return hipErrorInvalidValue;
  OutProjArgs A;
  A.o = o;
  A.z = z;
  A.w = w;
  A.Wo = Wo;
  A.y = y;
  A.eps = eps;
  A.H = S.H;
  A.T = S.T;
  A.N = d_model;
  A.M = (long long)S.B * S.T;
  const bool zb = S.in_dtype == SDM_BF16;
  if (output_project_rows(S.H * S.d_v) == 64)
    return zb ? launch_output_project_dv<true, 64>(A, S.d_v, stream) : launch_output_project_dv<false, 64>(A, S.d_v, stream);
  return zb ? launch_output_project_dv<true, 32>(A, S.d_v, stream) : launch_output_project_dv<false, 32>(A, S.d_v, stream);
}

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
  if (S.d_v == 32 || S.d_v == 64 || S.d_v == 128 || S.d_v == 256) {
    const dim3 g((unsigned)((units * (S.d_v / 8) + 255) / 256));
    const bool zb = S.in_dtype == SDM_BF16;
#define SDM_GATE_VEC(DV)                                                                                           \
  if (S.d_v == DV) {                                                                                               \
    if (zb) hipLaunchKernelGGL((output_gate_vec_kernel<true, DV>), g, dim3(256), 0, stream, o, z, w, eps, x, S.H,  \
                               S.T, units);                                                                        \
    else hipLaunchKernelGGL((output_gate_vec_kernel<false, DV>), g, dim3(256), 0, stream, o, z, w, eps, x, S.H,    \
                            S.T, units);                                                                           \
  }
    SDM_GATE_VEC(32) SDM_GATE_VEC(64) SDM_GATE_VEC(128) SDM_GATE_VEC(256)
#undef SDM_GATE_VEC
    return hipGetLastError();
  }
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
