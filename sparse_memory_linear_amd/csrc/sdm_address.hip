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
// One workgroup (8 waves) handles 32 tokens of one head. Scores of one half for the 32
// tokens are kept in LDS (never written to HBM); wave-level selection follows.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"
#include "sdm_select.hpp"

namespace sdm {

namespace {

constexpr int kTok = 32;      // tokens per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxK16 = 8;    // MFMA scoring for half widths up to 128 (8 steps of 16)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct AddrArgs {
  const void* x;        // [B,H,T,d_k] in dtype
  const void* subkeys;  // [H,2,s,h]   in dtype
  int32_t* idx;         // [B,H,T,n_sel]
  float* weight;        // [B,H,T,n_sel]
  float* score;         // [B,H,T,n_sel] or null
  int B, H, T, s, h, kappa, n_sel;
  int stair_count;      // number of (a, b) rank pairs with (a+1)(b+1) <= n_sel, a,b < kappa
  // optional slice [c0, c1) of the table initialisation M[b] = M0 (16-byte chunks of one
  // head-major copy of M0, written to each of the cB copies in M); null cM0 = none
  const u32x4* cM0;
  u32x4* cM;
  size_t chunks, c0, c1;
  int cB;
};

// The table initialisation rides on the addressing kernel, whose vector ALU is the bound while
// its memory pipe idles: each workgroup copies a share of the slice when it starts,
// kCopyUnroll chunks per thread in flight. (Holding the loaded chunks in registers across
// the first scoring pass, to hide their latency behind it, made the kernel spill.)
constexpr int kCopyUnroll = 8;
__device__ __forceinline__ void copy_share(const AddrArgs& A) {
  const size_t G = (size_t)gridDim.x * gridDim.y;
  const size_t g = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const size_t step = G * kThreads * kCopyUnroll;
  for (size_t base = A.c0 + g * kThreads * kCopyUnroll + threadIdx.x; base < A.c1; base += step) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      if (i < A.c1) v[u] = __builtin_nontemporal_load(&A.cM0[i]);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      if (i < A.c1)
        for (int b = 0; b < A.cB; ++b) __builtin_nontemporal_store(v[u], &A.cM[(size_t)b * A.chunks + i]);
    }
  }
}

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
// NK: K steps of 16 the fragment arrays hold (h <= 16 NK); a kernel built for half widths up
// to 64 keeps 32 fewer registers live through the scoring.
template <bool BF16, int NK>
__device__ void score_half(const AddrArgs& A, int head, int r0, int half, float* sc) {
  const int s = A.s, h = A.h, d_k = 2 * h;
  const int BT = A.B * A.T;
  const int stride = score_stride(s);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool use_mfma = BF16 && (s % 32 == 0) && (h % 16 == 0) && h <= 16 * NK;
  if (use_mfma) {
    // v_mfma_f32_32x32x16_bf16: lane l carries k = 8 (l / 32) .. +7 of row (or column) l % 32
    // of both operands; bf16 products are exact and summed in float32
    const uint16_t* X = (const uint16_t*)A.x;
    const uint16_t* C = (const uint16_t*)A.subkeys + ((size_t)head * 2 + half) * (size_t)s * h;
    int r = r0 + (lane & 31);
    if (r >= BT) r = BT - 1;  // rows past the end: valid address, result discarded
    const int b = r / A.T, t = r % A.T;
    const uint16_t* xrow = X + (((size_t)b * A.H + head) * A.T + t) * d_k + (size_t)half * h;
    const int kq = (lane >> 5) * 8;
    const int nk = h / 16;
    // this lane's token fragments for every k step, loaded once for all sub-key tiles
    uint4 xf[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k)
      if (k < nk) xf[k] = *(const uint4*)(xrow + 16 * k + kq);
    for (int st = wave; st < s / 32; st += kWaves) {
      const uint16_t* crow = C + (size_t)(st * 32 + (lane & 31)) * h;
      uint4 cf[NK];
#pragma unroll
      for (int k = 0; k < NK; ++k)
        if (k < nk) cf[k] = *(const uint4*)(crow + 16 * k + kq);
      float16_t acc = {};
#pragma unroll
      for (int k = 0; k < NK; ++k)
        if (k < nk)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cf[k]),
                                                        __builtin_bit_cast(bf16x8_t, xf[k]), acc, 0, 0, 0);
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
template <bool BF16, int ES, int EM, int NK>
__global__ void __launch_bounds__(kThreads, 4) address_kernel(AddrArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int s = A.s, kappa = A.kappa;
  const int stride = score_stride(s);
  float* sc = (float*)smem;                                     // [32][s+1]
  float* sel_s = sc + kTok * stride;                             // [32][2][kappa]
  int16_t* sel_i = (int16_t*)(sel_s + kTok * 2 * kappa);          // [32][2][kappa]
  // an offset from smem (not an integer-cast address), so that the compiler keeps LDS accesses
  const size_t wofs = ((size_t)((unsigned char*)(sel_i + kTok * 2 * kappa) - smem) + 15) & ~(size_t)15;
  uint64_t* wbuf_all = (uint64_t*)(smem + wofs);
  const int head = blockIdx.y;
  const int r0 = blockIdx.x * kTok;
  const int BT = A.B * A.T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (A.cM0) copy_share(A);
  uint64_t* wbuf = wbuf_all + wave * kWave;
  int pr[EM], bdiv;
  stair_pairs<EM>(kappa, A.n_sel, pr, &bdiv);

  // Two tokens per wave pass (their selections interleaved) where the score rows can hold the
  // candidate buffers: a token's row is dead once its scores are in registers, and rows of
  // at least 512 bytes at a stride of s floats keep them 8-byte aligned. Rows past the end
  // of the tokens hold scores of a clamped row and are selected but not written out.
  const bool pair = ES >= 2 && s % 32 == 0;
  auto rowbuf = [&](int n) { return (uint64_t*)(sc + n * stride); };
  for (int half = 0; half < 2; ++half) {
    score_half<BF16, NK>(A, head, r0, half, sc);
    __syncthreads();
    if (pair) {
      for (int n = wave; n < kTok; n += 2 * kWaves) {
        const int m = n + kWaves;
        select_half_x2<ES>(sc + n * stride, score_swz(s, n), sc + m * stride, score_swz(s, m), s, kappa, rowbuf(n),
                           rowbuf(m), sel_i + (n * 2 + half) * kappa, sel_s + (n * 2 + half) * kappa,
                           sel_i + (m * 2 + half) * kappa, sel_s + (m * 2 + half) * kappa);
      }
    } else {
      for (int n = wave; n < kTok; n += kWaves) {
        if (r0 + n >= BT) continue;
        select_half<ES>(sc + n * stride, score_swz(s, n), s, kappa, wbuf, sel_i + (n * 2 + half) * kappa,
                        sel_s + (n * 2 + half) * kappa);
      }
    }
    __syncthreads();
  }
  // softmax over a token's selected scores; idx, weight and score out
  auto emit = [&](int n, uint64_t k) {
    const int r = r0 + n;
    if (r >= BT) return;
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
  };
  auto sel = [&](int n, int h) { return sel_i + (n * 2 + h) * kappa; };
  auto sco = [&](int n, int h) { return sel_s + (n * 2 + h) * kappa; };
  if (pair) {
    for (int n = wave; n < kTok; n += 2 * kWaves) {
      const int m = n + kWaves;
      uint64_t ka, kb;
      merge_token_x2<EM>(sel(n, 0), sco(n, 0), sel(n, 1), sco(n, 1), sel(m, 0), sco(m, 0), sel(m, 1), sco(m, 1), s,
                         kappa, A.n_sel, pr, bdiv, rowbuf(n), rowbuf(m), &ka, &kb);
      emit(n, ka);
      emit(m, kb);
    }
  } else {
    for (int n = wave; n < kTok; n += kWaves) {
      if (r0 + n >= BT) continue;
      emit(n, merge_token<EM>(sel(n, 0), sco(n, 0), sel(n, 1), sco(n, 1), s, kappa, A.n_sel, pr, bdiv, wbuf));
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

template <bool BF16, int ES, int NK>
hipError_t launch_em(const AddrArgs& A, size_t lds, hipStream_t st) {
  dim3 grid((A.B * A.T + kTok - 1) / kTok, A.H);
  int em = (A.stair_count + kWave - 1) / kWave;
  if (em <= 1) hipLaunchKernelGGL((address_kernel<BF16, ES, 1, NK>), grid, dim3(kThreads), lds, st, A);
  else if (em <= 2) hipLaunchKernelGGL((address_kernel<BF16, ES, 2, NK>), grid, dim3(kThreads), lds, st, A);
  else if (em <= 4) hipLaunchKernelGGL((address_kernel<BF16, ES, 4, NK>), grid, dim3(kThreads), lds, st, A);
  else hipLaunchKernelGGL((address_kernel<BF16, ES, 8, NK>), grid, dim3(kThreads), lds, st, A);
  return hipGetLastError();
}

template <bool BF16, int ES>
hipError_t launch_nk(const AddrArgs& A, size_t lds, hipStream_t st) {
  if constexpr (BF16) {
    if (A.h <= 64) return launch_em<BF16, ES, 4>(A, lds, st);
  }
  return launch_em<BF16, ES, kMaxK16>(A, lds, st);
}

template <bool BF16>
hipError_t launch_es(const AddrArgs& A, size_t lds, hipStream_t st) {
  int es = (A.s + kWave - 1) / kWave;
  if (es <= 1) return launch_nk<BF16, 1>(A, lds, st);
  if (es <= 2) return launch_nk<BF16, 2>(A, lds, st);
  if (es <= 4) return launch_nk<BF16, 4>(A, lds, st);
  return launch_nk<BF16, 8>(A, lds, st);
}

}  // namespace

size_t address_lds_bytes(int s, int kappa) {
  size_t b = (size_t)kTok * score_stride(s) * 4 + (size_t)kTok * 2 * kappa * 6;
  b = (b + 15) & ~(size_t)15;
  return b + kWaves * kWave * 8;
}

hipError_t launch_address(const sdm_shape& S, const void* x, const void* subkeys, int n_sel, int32_t* idx,
                          float* weight, float* score, hipStream_t stream, const InitPart* init) {
  AddrArgs A;
  A.cM0 = nullptr;
  A.cM = nullptr;
  A.chunks = A.c0 = A.c1 = 0;
  A.cB = 0;
  if (init) {
    // slice `part` of `nparts` of the 16-byte chunks of one head-major copy of M0
    A.chunks = (size_t)S.H * (size_t)S.N * (size_t)S.d_v * dtype_size(S.mem_dtype) / 16;
    A.c0 = A.chunks * (size_t)init->part / (size_t)init->nparts;
    A.c1 = A.chunks * ((size_t)init->part + 1) / (size_t)init->nparts;
    A.cB = S.B;
    if (A.c1 > A.c0 && S.B > 0) {
      A.cM0 = (const u32x4*)init->M0;
      A.cM = (u32x4*)init->M;
    }
  }
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
  if (S.B * S.T == 0) return A.cM0 ? launch_init_part(S, init->M0, init->M, A.c0, A.c1, stream) : hipSuccess;
  size_t lds = address_lds_bytes(A.s, A.kappa);
  if (S.in_dtype == SDM_BF16) return launch_es<true>(A, lds, stream);
  return launch_es<false>(A, lds, stream);
}

}  // namespace sdm
