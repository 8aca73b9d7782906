// Fused decode step (T = 1): addressing of k and q, gated delta write of the W slots and
// weighted read of the R slots, one workgroup per (sequence, head), one launch.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Gated DeltaNet", §3 "Sparse memory
// updates", "Sparse addressing", "Sparse retrieval"; §4 softmax activations; atlas.scime.ai
// summary, "Approach"): the same rule as the sequence forward, for one token per unit.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"
#include "sdm_select.hpp"

namespace sdm {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxK16 = 8;  // MFMA scoring for half widths up to 128 (8 steps of 16)

struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const void* subkeys;
  void* M;
  float* o;
  double* lam;   // whole-table decay state [units][N] and [units], or null
  double* lrun;
  int H, s, h, kappa, W, R, d_v, stairW, stairR;
  long long N;
};

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, size_t i) {
  if (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

template <typename MemT>
struct DMem;
template <>
struct DMem<float> {
  static constexpr int kCols = 1;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = __uint_as_float(w); }
  __device__ static uint32_t pack(const float* x) { return __float_as_uint(x[0]); }
};
template <>
struct DMem<uint16_t> {
  static constexpr int kCols = 2;
  __device__ static void unpack(uint32_t w, float* x) { x[0] = bf16lo(w); x[1] = bf16hi(w); }
  __device__ static uint32_t pack(const float* x) { return pack_bf16x2(x[0], x[1]); }
};

struct DecLds {
  size_t sc, sel_i, sel_s, wbuf, widx, wgt, ridx, rgt, rmatch, fw, fr, wrow, part, delta, total;
};

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline DecLds dec_lds(int s, int kappa, int W, int R, int rowdw, int cpl) {
  DecLds L;
  size_t o = 0;
  L.sc = o; o = al16(o + (size_t)4 * (s + 1) * 4);
  L.sel_i = o; o = al16(o + (size_t)4 * kappa * 2);
  L.sel_s = o; o = al16(o + (size_t)4 * kappa * 4);
  L.wbuf = o; o = al16(o + (size_t)4 * 64 * 8);
  L.widx = o; o = al16(o + (size_t)W * 4);
  L.wgt = o; o = al16(o + (size_t)W * 4);
  L.ridx = o; o = al16(o + (size_t)R * 4);
  L.rgt = o; o = al16(o + (size_t)R * 4);
  L.rmatch = o; o = al16(o + (size_t)R * 4);
  L.fw = o; o = al16(o + (size_t)W * 4);
  L.fr = o; o = al16(o + (size_t)R * 4);
  L.wrow = o; o = al16(o + (size_t)W * rowdw * 4);
  L.part = o; o = al16(o + (size_t)kThreads * cpl * 4);
  L.delta = o; o = al16(o + (size_t)rowdw * cpl * 4);
  L.total = o;
  return L;
}

template <bool BF16, typename MemT, int ES, int EMW, int EMR>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecArgs A) {
  using MT = DMem<MemT>;
  constexpr int CPL = MT::kCols;
  extern __shared__ __align__(16) unsigned char smem[];
  const int s = A.s, hh = A.h, kappa = A.kappa, W = A.W, R = A.R;
  const int rowdw = A.d_v / CPL;
  const DecLds L = dec_lds(s, kappa, W, R, rowdw, CPL);
  float* sc = (float*)(smem + L.sc);
  int16_t* sel_i = (int16_t*)(smem + L.sel_i);
  float* sel_s = (float*)(smem + L.sel_s);
  uint64_t* wbuf = (uint64_t*)(smem + L.wbuf);
  int32_t* swidx = (int32_t*)(smem + L.widx);
  float* swgt = (float*)(smem + L.wgt);
  int32_t* sridx = (int32_t*)(smem + L.ridx);
  float* srgt = (float*)(smem + L.rgt);
  int32_t* rmatch = (int32_t*)(smem + L.rmatch);
  float* sfw = (float*)(smem + L.fw);
  float* sfr = (float*)(smem + L.fr);
  uint32_t* wrow = (uint32_t*)(smem + L.wrow);
  float* part = (float*)(smem + L.part);
  float* sdelta = (float*)(smem + L.delta);

  const int u = blockIdx.x;
  const int head = u % A.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int d_k = 2 * hh;

  // 1. scores of (k half 0, k half 1, q half 0, q half 1) against their sub-keys
  if (BF16 && (s % 32 == 0) && (hh % 16 == 0) && hh <= 16 * kMaxK16) {
    // MFMA (v_mfma_f32_32x32x16_bf16): a 32-sub-key tile of one half is the A operand; the B
    // operand's columns 0 and 1 are that half of k and of q (the other columns are zero), so
    // one pass scores both. Lane l carries k = 8 (l / 32) .. +7 of both operands.
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    typedef float float16_t __attribute__((ext_vector_type(16)));
    const int col = lane & 31, kq = (lane >> 5) * 8, nk = hh / 16;
    for (int half = 0; half < 2; ++half) {
      const uint16_t* xv = (const uint16_t*)(col == 0 ? A.k : A.q) + (size_t)u * d_k + (size_t)half * hh;
      uint4 xf[kMaxK16];
#pragma unroll
      for (int kk = 0; kk < kMaxK16; ++kk)
        if (kk < nk) xf[kk] = col < 2 ? *(const uint4*)(xv + 16 * kk + kq) : make_uint4(0u, 0u, 0u, 0u);
      const uint16_t* C = (const uint16_t*)A.subkeys + ((size_t)head * 2 + half) * (size_t)s * hh;
      for (int st = wave; st < s / 32; st += kThreads / 64) {
        const uint16_t* crow = C + (size_t)(st * 32 + col) * hh;
        uint4 cf[kMaxK16];
#pragma unroll
        for (int kk = 0; kk < kMaxK16; ++kk)
          if (kk < nk) cf[kk] = *(const uint4*)(crow + 16 * kk + kq);
        float16_t acc = {};
#pragma unroll
        for (int kk = 0; kk < kMaxK16; ++kk)
          if (kk < nk)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cf[kk]),
                                                          __builtin_bit_cast(bf16x8_t, xf[kk]), acc, 0, 0, 0);
        // D[row = sub-key][col]; lane holds col = lane % 32, rows 8*(i/4) + 4*(lane/32) + i%4
        if (col < 2) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            sc[(col * 2 + half) * (s + 1) + st * 32 + row] = acc[i];
          }
        }
      }
    }
  } else {
    for (int p = tid; p < 4 * s; p += kThreads) {
      const int c = p / s, m = p % s, half = c & 1;
      const void* x = c < 2 ? A.k : A.q;
      const size_t xo = (size_t)u * d_k + (size_t)half * hh;
      const size_t co = ((size_t)head * 2 + half) * (size_t)s * hh + (size_t)m * hh;
      float acc = 0.f;
      for (int i = 0; i < hh; ++i) acc = fmaf(ld_in<BF16>(x, xo + i), ld_in<BF16>(A.subkeys, co + i), acc);
      sc[c * (s + 1) + m] = acc;
    }
  }
  __syncthreads();
  // 2. per-half top-kappa, one wave per (vector, half)
  select_half<ES>(sc + wave * (s + 1), 0, s, kappa, wbuf + wave * 64, sel_i + wave * kappa, sel_s + wave * kappa);
  __syncthreads();
  // 3. kappa x kappa merge and softmax: wave 0 for the key (W), wave 1 for the query (R)
  if (wave < 2) {
    const int n_sel = wave == 0 ? W : R;
    const int base = wave * 2;
    uint64_t key;
    if (wave == 0) {
      int pr[EMW];
      stair_pairs<EMW>(kappa, n_sel, pr);
      key = merge_token<EMW>(sel_i + base * kappa, sel_s + base * kappa, sel_i + (base + 1) * kappa,
                             sel_s + (base + 1) * kappa, s, kappa, n_sel, pr, wbuf + wave * 64);
    } else {
      int pr[EMR];
      stair_pairs<EMR>(kappa, n_sel, pr);
      key = merge_token<EMR>(sel_i + base * kappa, sel_s + base * kappa, sel_i + (base + 1) * kappa,
                             sel_s + (base + 1) * kappa, s, kappa, n_sel, pr, wbuf + wave * 64);
    }
    float scv = lane < n_sel ? key_score(key) : -INFINITY;
    float mx = __shfl(scv, 0, kWave);
    float e = lane < n_sel ? expf(scv - mx) : 0.f;
    float tot = wave_sum_f32(e);
    if (lane < n_sel) {
      if (wave == 0) { swidx[lane] = (int32_t)key_index(key); swgt[lane] = e / tot; }
      else { sridx[lane] = (int32_t)key_index(key); srgt[lane] = e / tot; }
    }
  }
  __syncthreads();
  if (tid < R) {
    int pos = -1;
    for (int j = 0; j < W; ++j)
      if (swidx[j] == sridx[tid]) pos = j;
    rmatch[tid] = pos;
  }
  // whole-table decay: a write row's value before this token's decay is its stored value
  // times exp(lrun - lam); a read row's after it, times exp(lrun + log alpha - lam), or 1 for
  // a row this token writes
  double lnew = 0.0;
  if (A.lam) {
    const double lold = A.lrun[u];
    lnew = lold + fmax(log((double)A.alpha[u]), -1000.0);
    const double* lam = A.lam + (size_t)u * A.N;
    if (tid < W) sfw[tid] = expf((float)(lold - lam[swidx[tid]]));
    if (tid < R) sfr[tid] = rmatch[tid] >= 0 ? 1.f : expf((float)(lnew - lam[sridx[tid]]));
    __syncthreads();
  }
  // 4. rows: thread = (row group g, row word dw)
  const int G = kThreads / rowdw;
  const int g = tid / rowdw, dw = tid % rowdw;
  const bool act = g < G;
  uint32_t* Mu = (uint32_t*)A.M + (size_t)u * (size_t)A.N * rowdw;
  const float al = A.alpha[u], be = A.beta[u];
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  if (act) {
    for (int j = g; j < W; j += G) {
      uint32_t w = Mu[(size_t)swidx[j] * rowdw + dw];
      wrow[j * rowdw + dw] = w;
      float x[CPL];
      MT::unpack(w, x);
      const float wx = A.lam ? swgt[j] * sfw[j] : swgt[j];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wx, x[c], acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) part[tid * CPL + c] = acc[c];
  __syncthreads();
  if (tid < rowdw) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float rho = 0.f;
      for (int gg = 0; gg < G; ++gg) rho += part[(gg * rowdw + tid) * CPL + c];
      const float vv = ld_in<BF16>(A.v, (size_t)u * A.d_v + (size_t)tid * CPL + c);
      sdelta[tid * CPL + c] = be * (vv - al * rho);
    }
  }
  __syncthreads();
  if (act) {
    for (int j = g; j < W; j += G) {
      float x[CPL], y[CPL];
      MT::unpack(wrow[j * rowdw + dw], x);
      const float ax = A.lam ? al * sfw[j] : al;
#pragma unroll
      for (int c = 0; c < CPL; ++c) y[c] = fmaf(ax, x[c], swgt[j] * sdelta[dw * CPL + c]);
      const uint32_t nw = MT::pack(y);
      Mu[(size_t)swidx[j] * rowdw + dw] = nw;
      wrow[j * rowdw + dw] = nw;
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  if (act) {
    for (int r = g; r < R; r += G) {
      const int pos = rmatch[r];
      const uint32_t w = pos >= 0 ? wrow[pos * rowdw + dw] : Mu[(size_t)sridx[r] * rowdw + dw];
      float x[CPL];
      MT::unpack(w, x);
      const float wr = A.lam ? srgt[r] * sfr[r] : srgt[r];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wr, x[c], acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) part[tid * CPL + c] = acc[c];
  __syncthreads();
  if (tid < rowdw) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float ov = 0.f;
      for (int gg = 0; gg < G; ++gg) ov += part[(gg * rowdw + tid) * CPL + c];
      A.o[(size_t)u * A.d_v + (size_t)tid * CPL + c] = ov;
    }
  }
  if (A.lam) {
    // the written slots now hold values as of this token
    if (tid < W) A.lam[(size_t)u * A.N + swidx[tid]] = lnew;
    if (tid == 0) A.lrun[u] = lnew;
  }
}

int stair_of(int kappa, int n_sel) {
  int c = 0;
  for (int a = 0; a < kappa; ++a) {
    int k = n_sel / (a + 1);
    c += k < kappa ? k : kappa;
  }
  return c;
}

template <bool BF16, typename MemT, int ES, int EMW>
hipError_t dec_launch_r(const DecArgs& A, int units, size_t lds, hipStream_t st) {
  int emr = (A.stairR + 63) / 64;
  if (emr <= 1) hipLaunchKernelGGL((decode_kernel<BF16, MemT, ES, EMW, 1>), dim3(units), dim3(kThreads), lds, st, A);
  else if (emr <= 2) hipLaunchKernelGGL((decode_kernel<BF16, MemT, ES, EMW, 2>), dim3(units), dim3(kThreads), lds, st, A);
  else if (emr <= 4) hipLaunchKernelGGL((decode_kernel<BF16, MemT, ES, EMW, 4>), dim3(units), dim3(kThreads), lds, st, A);
  else hipLaunchKernelGGL((decode_kernel<BF16, MemT, ES, EMW, 8>), dim3(units), dim3(kThreads), lds, st, A);
  return hipGetLastError();
}
template <bool BF16, typename MemT, int ES>
hipError_t dec_launch_w(const DecArgs& A, int units, size_t lds, hipStream_t st) {
  int emw = (A.stairW + 63) / 64;
  if (emw <= 1) return dec_launch_r<BF16, MemT, ES, 1>(A, units, lds, st);
  if (emw <= 2) return dec_launch_r<BF16, MemT, ES, 2>(A, units, lds, st);
  if (emw <= 4) return dec_launch_r<BF16, MemT, ES, 4>(A, units, lds, st);
  return dec_launch_r<BF16, MemT, ES, 8>(A, units, lds, st);
}
template <bool BF16, typename MemT>
hipError_t dec_launch_s(const DecArgs& A, int units, size_t lds, hipStream_t st) {
  int es = (A.s + 63) / 64;
  if (es <= 1) return dec_launch_w<BF16, MemT, 1>(A, units, lds, st);
  if (es <= 2) return dec_launch_w<BF16, MemT, 2>(A, units, lds, st);
  if (es <= 4) return dec_launch_w<BF16, MemT, 4>(A, units, lds, st);
  return dec_launch_w<BF16, MemT, 8>(A, units, lds, st);
}

}  // namespace

size_t decode_lds_bytes(const sdm_shape& S) {
  const int cpl = S.mem_dtype == SDM_BF16 ? 2 : 1;
  const int rowdw = S.d_v / cpl;
  return dec_lds((int)isqrt64(S.N), S.kappa, S.W, S.R, rowdw, cpl).total;
}

hipError_t launch_decode(const sdm_shape& S, const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const void* subkeys, void* M, float* o, const DecayState* dk,
                         hipStream_t stream) {
  DecArgs A;
  A.lam = dk ? dk->lam : nullptr;
  A.lrun = dk ? dk->lrun : nullptr;
  A.q = q;
  A.k = k;
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  A.subkeys = subkeys;
  A.M = M;
  A.o = o;
  A.H = S.H;
  A.s = (int)isqrt64(S.N);
  A.h = S.d_k / 2;
  A.kappa = S.kappa;
  A.W = S.W;
  A.R = S.R;
  A.d_v = S.d_v;
  A.N = S.N;
  A.stairW = stair_of(S.kappa, S.W);
  A.stairR = stair_of(S.kappa, S.R);
  const int units = S.B * S.H;
  const size_t lds = decode_lds_bytes(S);
  const bool ib = S.in_dtype == SDM_BF16, mb = S.mem_dtype == SDM_BF16;
  if (ib && mb) return dec_launch_s<true, uint16_t>(A, units, lds, stream);
  if (ib && !mb) return dec_launch_s<true, float>(A, units, lds, stream);
  if (!ib && mb) return dec_launch_s<false, uint16_t>(A, units, lds, stream);
  return dec_launch_s<false, float>(A, units, lds, stream);
}

}  // namespace sdm
