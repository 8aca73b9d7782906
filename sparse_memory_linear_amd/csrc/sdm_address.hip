// Product-key addressing of every token: scores of both halves of x against the sub-keys
// (MFMA for bf16), per-half top-kappa, kappa x kappa merge to the top n_sel slots, softmax.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Product Key Memory", §3 "Sparse
// addressing", §4 "SDM Configuration"; atlas.scime.ai summary, "Approach"): each half of the
// query/key vector is compared with its own set of s sub-keys; a slot is a pair (i, j) of
// sub-keys, numbered n = i*s + j, scored by the sum of the two half scores; the best
// kappa sub-keys of each half form kappa^2 candidate slots, of which the best n_sel are
// kept and weighted by a softmax over their scores.
//
// One workgroup (4 waves) handles 32 tokens of one head. Scores of one half for the 32
// tokens are kept in LDS (never written to HBM); wave-level selection follows.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"
#include "sdm_select.hpp"

namespace sdm {

namespace {

constexpr int kTok = 32;      // tokens per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxK8 = 8;     // MFMA scoring for half widths up to 64 (8 steps of 8)

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

struct AddrArgs {
  const void* x;        // [B,H,T,d_k] in dtype
  const void* subkeys;  // [H,2,s,h]   in dtype
  int32_t* idx;         // [B,H,T,n_sel]
  float* weight;        // [B,H,T,n_sel]
  float* score;         // [B,H,T,n_sel] or null
  int B, H, T, s, h, kappa, n_sel;
  int stair_count;      // number of (a, b) rank pairs with (a+1)(b+1) <= n_sel, a,b < kappa
};

// Score tile [32 tokens][s]. The MFMA layout writes one token per lane; to keep those writes
// in different LDS banks, score m of token n sits at n * s + (m ^ n) when s is a multiple of
// 32 (the MFMA path); otherwise rows are padded by one float.
__host__ __device__ __forceinline__ int score_stride(int s) { return s % 32 == 0 ? s : s + 1; }
__host__ __device__ __forceinline__ int score_swz(int s, int n) { return s % 32 == 0 ? (n & 31) : 0; }

template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
  if (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

// ---------------------------------------------------------------- scoring
// Scores of half `half` for the 32 tokens rows r0..r0+31 of head `head` into sc[32][s+1].
template <bool BF16>
__device__ void score_half(const AddrArgs& A, int head, int r0, int half, float* sc) {
  const int s = A.s, h = A.h, d_k = 2 * h;
  const int BT = A.B * A.T;
  const int stride = score_stride(s);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool use_mfma = BF16 && (s % 32 == 0) && (h % 8 == 0) && h <= 8 * kMaxK8;
  if (use_mfma) {
    const uint16_t* X = (const uint16_t*)A.x;
    const uint16_t* C = (const uint16_t*)A.subkeys + ((size_t)head * 2 + half) * (size_t)s * h;
    int r = r0 + (lane & 31);
    if (r >= BT) r = BT - 1;  // rows past the end: valid address, result discarded
    const int b = r / A.T, t = r % A.T;
    const uint16_t* xrow = X + (((size_t)b * A.H + head) * A.T + t) * d_k + (size_t)half * h;
    const int kq = (lane >> 5) * 4;
    const int nk = h / 8;
    // this lane's token fragments for every k step, loaded once for all sub-key tiles
    uint2 xf[kMaxK8];
#pragma unroll
    for (int k = 0; k < kMaxK8; ++k)
      if (k < nk) xf[k] = *(const uint2*)(xrow + 8 * k + kq);
    for (int st = wave; st < s / 32; st += kWaves) {
      const uint16_t* crow = C + (size_t)(st * 32 + (lane & 31)) * h;
      uint2 cf[kMaxK8];
#pragma unroll
      for (int k = 0; k < kMaxK8; ++k)
        if (k < nk) cf[k] = *(const uint2*)(crow + 8 * k + kq);
      float16_t acc = {};
#pragma unroll
      for (int k = 0; k < kMaxK8; ++k)
        if (k < nk)
          acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(short4_t, cf[k]),
                                                         __builtin_bit_cast(short4_t, xf[k]), acc, 0, 0, 0);
      // D[row = sub-key][col = token]; lane holds col = lane%32,
      // rows 8*(i/4) + 4*(lane/32) + i%4.
      const int col = lane & 31;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        sc[col * stride + ((st * 32 + row) ^ col)] = acc[i];
      }
    }
  } else {
    const int n = tid & 31;
    int r = r0 + n;
    if (r >= BT) r = BT - 1;
    const int b = r / A.T, t = r % A.T;
    const size_t xoff = (((size_t)b * A.H + head) * A.T + t) * d_k + (size_t)half * h;
    const size_t coff = ((size_t)head * 2 + half) * (size_t)s * h;
    for (int m = tid >> 5; m < s; m += kThreads / 32) {
      float acc = 0.f;
      for (int c = 0; c < h; ++c)
        acc = fmaf(load_in<BF16>(A.x, xoff + c), load_in<BF16>(A.subkeys, coff + (size_t)m * h + c), acc);
      sc[n * stride + (m ^ score_swz(s, n))] = acc;
    }
  }
}

// ---------------------------------------------------------------- kernel
template <bool BF16, int ES, int EM>
__global__ void __launch_bounds__(kThreads, 4) address_kernel(AddrArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int s = A.s, kappa = A.kappa;
  const int stride = score_stride(s);
  float* sc = (float*)smem;                                     // [32][s+1]
  float* sel_s = sc + kTok * stride;                             // [32][2][kappa]
  int16_t* sel_i = (int16_t*)(sel_s + kTok * 2 * kappa);          // [32][2][kappa]
  uint64_t* wbuf_all = (uint64_t*)(((uintptr_t)(sel_i + kTok * 2 * kappa) + 15) & ~(uintptr_t)15);
  const int head = blockIdx.y;
  const int r0 = blockIdx.x * kTok;
  const int BT = A.B * A.T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t* wbuf = wbuf_all + wave * kWave;
  int pr[EM];
  stair_pairs<EM>(kappa, A.n_sel, pr);

  for (int half = 0; half < 2; ++half) {
    score_half<BF16>(A, head, r0, half, sc);
    __syncthreads();
    for (int n = wave; n < kTok; n += kWaves) {
      if (r0 + n >= BT) continue;
      select_half<ES>(sc + n * stride, score_swz(s, n), s, kappa, wbuf, sel_i + (n * 2 + half) * kappa,
                      sel_s + (n * 2 + half) * kappa);
    }
    __syncthreads();
  }
  for (int n = wave; n < kTok; n += kWaves) {
    const int r = r0 + n;
    if (r >= BT) continue;
    const int16_t* i1 = sel_i + (n * 2 + 0) * kappa;
    const int16_t* i2 = sel_i + (n * 2 + 1) * kappa;
    const float* s1 = sel_s + (n * 2 + 0) * kappa;
    const float* s2 = sel_s + (n * 2 + 1) * kappa;
    uint64_t k = merge_token<EM>(i1, s1, i2, s2, s, kappa, A.n_sel, pr, wbuf);
    float scv = lane < A.n_sel ? key_score(k) : -INFINITY;
    float mx = __shfl(scv, 0, kWave);
    float e = lane < A.n_sel ? expf(scv - mx) : 0.f;
    float tot = wave_sum_f32(e);
    const int b = r / A.T, t = r % A.T;
    const size_t o = (((size_t)b * A.H + head) * A.T + t) * A.n_sel;
    if (lane < A.n_sel) {
      A.idx[o + lane] = (int32_t)key_index(k);
      A.weight[o + lane] = e / tot;
      if (A.score) A.score[o + lane] = scv;
    }
  }
}

int stair_count_of(int kappa, int n_sel) {
  int c = 0;
  for (int a = 0; a < kappa; ++a) {
    int k = n_sel / (a + 1);
    c += k < kappa ? k : kappa;
  }
  return c;
}

template <bool BF16, int ES>
hipError_t launch_em(const AddrArgs& A, size_t lds, hipStream_t st) {
  dim3 grid((A.B * A.T + kTok - 1) / kTok, A.H);
  int em = (A.stair_count + kWave - 1) / kWave;
  if (em <= 1) hipLaunchKernelGGL((address_kernel<BF16, ES, 1>), grid, dim3(kThreads), lds, st, A);
  else if (em <= 2) hipLaunchKernelGGL((address_kernel<BF16, ES, 2>), grid, dim3(kThreads), lds, st, A);
  else if (em <= 4) hipLaunchKernelGGL((address_kernel<BF16, ES, 4>), grid, dim3(kThreads), lds, st, A);
  else hipLaunchKernelGGL((address_kernel<BF16, ES, 8>), grid, dim3(kThreads), lds, st, A);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_es(const AddrArgs& A, size_t lds, hipStream_t st) {
  int es = (A.s + kWave - 1) / kWave;
  if (es <= 1) return launch_em<BF16, 1>(A, lds, st);
  if (es <= 2) return launch_em<BF16, 2>(A, lds, st);
  if (es <= 4) return launch_em<BF16, 4>(A, lds, st);
  return launch_em<BF16, 8>(A, lds, st);
}

}  // namespace

size_t address_lds_bytes(int s, int kappa) {
  size_t b = (size_t)kTok * score_stride(s) * 4 + (size_t)kTok * 2 * kappa * 6;
  b = (b + 15) & ~(size_t)15;
  return b + kWaves * kWave * 8;
}

hipError_t launch_address(const sdm_shape& S, const void* x, const void* subkeys, int n_sel, int32_t* idx,
                          float* weight, float* score, hipStream_t stream) {
  AddrArgs A;
  A.x = x;
  A.subkeys = subkeys;
  A.idx = idx;
  A.weight = weight;
  A.score = score;
  A.B = S.B;
  A.H = S.H;
  A.T = S.T;
  A.s = isqrt64(S.N);
  A.h = S.d_k / 2;
  A.kappa = S.kappa;
  A.n_sel = n_sel;
  A.stair_count = stair_count_of(S.kappa, n_sel);
  if (S.B * S.T == 0) return hipSuccess;
  size_t lds = address_lds_bytes(A.s, A.kappa);
  if (S.in_dtype == SDM_BF16) return launch_es<true>(A, lds, stream);
  return launch_es<false>(A, lds, stream);
}

}  // namespace sdm
