// Fused decode step (T = 1): addressing of k and q, gated delta write of the W slots and
// weighted read of the R slots, one launch.
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Gated DeltaNet", §3 "Sparse memory
// updates", "Sparse addressing", "Sparse retrieval"; §4 softmax activations; atlas.scime.ai
// summary, "Approach"): the same rule as the sequence forward, for one token per unit.
//
// One workgroup serves UPW sequences of one head (UPW x 256 threads, a group of four waves
// per sequence). The head's sub-keys are what a step reads most (2 s h values per head,
// 64 KB at s = 256, h = 64, against 8 KB of table rows per unit): each 32-sub-key tile is
// loaded once per workgroup and scored against the k and q of all its sequences in one MFMA
// (B operand columns 2 g and 2 g + 1 = k and q of sequence g). Selection, merge and the
// row work then run per sequence in its own group of waves; barriers span the workgroup.

#include "sdm_device.hpp"
#include "sdm_internal.hpp"
#include "sdm_select.hpp"

namespace sdm {

namespace {

constexpr int kGroup = 256;  // threads per sequence
constexpr int kMaxK16 = 8;   // MFMA scoring for half widths up to 128 (8 steps of 16)

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
  int B, H, s, h, kappa, W, R, d_v, stairW, stairR;
  long long N;
};

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, size_t i) {
  if (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

// Workgroup barrier that orders LDS accesses only (global stores in flight are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }

// LDS of one workgroup: shared part, then one block per sequence.
struct DecLds {
  size_t xs, wbuf, unit0, unit;  // k and q of every sequence; per-wave selection buffers; blocks
  // offsets inside a sequence's block
  size_t sc, sel_i, sel_s, widx, wgt, ridx, rgt, rmatch, fw, fr, wrow, part, opart, delta, flag;
  size_t total;
};

__host__ __device__ inline DecLds dec_lds(int upw, int s, int kappa, int W, int R, int rowdw, int cpl, int d_k) {
  DecLds L;
  size_t o = 0;
  L.xs = o; o = al16(o + (size_t)upw * 2 * d_k * 2);
  L.wbuf = o; o = al16(o + (size_t)upw * 4 * 64 * 8);
  L.unit0 = o;
  size_t p = 0;
  L.sc = p; p = al16(p + (size_t)4 * (s + 1) * 4);
  L.sel_i = p; p = al16(p + (size_t)4 * kappa * 2);
  L.sel_s = p; p = al16(p + (size_t)4 * kappa * 4);
  L.widx = p; p = al16(p + (size_t)W * 4);
  L.wgt = p; p = al16(p + (size_t)W * 4);
  L.ridx = p; p = al16(p + (size_t)R * 4);
  L.rgt = p; p = al16(p + (size_t)R * 4);
  L.rmatch = p; p = al16(p + (size_t)R * 4);
  L.fw = p; p = al16(p + (size_t)W * 4);
  L.fr = p; p = al16(p + (size_t)R * 4);
  L.wrow = p; p = al16(p + (size_t)W * rowdw * 4);
  L.part = p; p = al16(p + (size_t)kGroup * cpl * 4);
  L.opart = p; p = al16(p + (size_t)kGroup * cpl * 4);
  L.delta = p; p = al16(p + (size_t)rowdw * cpl * 4);
  L.flag = p; p = al16(p + 4);
  L.unit = p;
  L.total = o + (size_t)upw * p;
  return L;
}

template <bool BF16, typename MemT, int ES, int EM, int UPW>
__global__ void __launch_bounds__(kGroup * UPW) decode_kernel(DecArgs A) {
  using MT = DMem<MemT>;
  constexpr int CPL = MT::kCols;
  constexpr int NW = 4 * UPW;  // waves
  extern __shared__ __align__(16) unsigned char smem[];
  const int s = A.s, hh = A.h, kappa = A.kappa, W = A.W, R = A.R;
  const int d_k = 2 * hh;
  const int rowdw = A.d_v / CPL;
  const DecLds L = dec_lds(UPW, s, kappa, W, R, rowdw, CPL, d_k);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = tid / kGroup, ltid = tid % kGroup, lwave = ltid >> 6;
  const int head = blockIdx.x % A.H;
  const int b = (blockIdx.x / A.H) * UPW + grp;  // this group's sequence
  const bool live = b < A.B;
  const int u = live ? b * A.H + head : head;    // unit (a group past B stays in bounds and idle)

  unsigned char* ub = smem + L.unit0 + (size_t)grp * L.unit;
  float* sc = (float*)(ub + L.sc);
  int16_t* sel_i = (int16_t*)(ub + L.sel_i);
  float* sel_s = (float*)(ub + L.sel_s);
  int32_t* swidx = (int32_t*)(ub + L.widx);
  float* swgt = (float*)(ub + L.wgt);
  int32_t* sridx = (int32_t*)(ub + L.ridx);
  float* srgt = (float*)(ub + L.rgt);
  int32_t* rmatch = (int32_t*)(ub + L.rmatch);
  float* sfw = (float*)(ub + L.fw);
  float* sfr = (float*)(ub + L.fr);
  uint32_t* wrow = (uint32_t*)(ub + L.wrow);
  float* part = (float*)(ub + L.part);
  float* opart = (float*)(ub + L.opart);
  float* sdelta = (float*)(ub + L.delta);
  int* anymatch = (int*)(ub + L.flag);
  uint64_t* wbuf = (uint64_t*)(smem + L.wbuf) + (size_t)wave * 64;
  // the merge waves' staircase (it depends only on kappa and the list length): enumerated
  // now, while the workgroup waits for k and q
  int pr[EM], bdiv = 0;
#pragma unroll
  for (int e = 0; e < EM; ++e) pr[e] = -1;
  const bool merger = live && lwave < 2;

  // 1. scores of (k half 0, k half 1, q half 0, q half 1) of every sequence against the sub-keys
  if (BF16 && (s % 32 == 0) && (hh % 16 == 0) && hh <= 16 * kMaxK16) {
    // MFMA (v_mfma_f32_32x32x16_bf16): a 32-sub-key tile of one half is the A operand; the B
    // operand's columns 2 g and 2 g + 1 are that half of k and q of sequence g (the other
    // columns are zero). Lane l carries k = 8 (l / 32) .. +7 of both operands. Work items
    // (half, tile) are dealt to the waves; a wave's next item is loaded while the current one
    // is multiplied. k and q go through LDS; their loads are issued before the sub-key loads
    // so that the LDS write waits for them alone.
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    typedef float float16_t __attribute__((ext_vector_type(16)));
    uint16_t* xs = (uint16_t*)(smem + L.xs);  // [UPW][2][d_k]: k, then q of each sequence
    const int pieces = d_k / 8;               // 16-byte pieces of one vector
    uint4 xv = make_uint4(0u, 0u, 0u, 0u);
    const bool xl = tid < UPW * 2 * pieces;
    int xg = 0, xvec = 0, xpc = 0;
    if (xl) {
      xg = tid / (2 * pieces);
      xvec = (tid / pieces) & 1;
      xpc = tid % pieces;
      const int bx = (blockIdx.x / A.H) * UPW + xg;
      if (bx < A.B) {
        const size_t ux = (size_t)bx * A.H + head;
        xv = *(const uint4*)((const uint16_t*)(xvec == 0 ? A.k : A.q) + ux * d_k + xpc * 8);
      }
    }
    const int col = lane & 31, kq = (lane >> 5) * 8, nk = hh / 16;
    const int tiles = s / 32, items = 2 * tiles;
    auto item_load = [&](int it, uint4 (&buf)[kMaxK16]) {
      const int half = it / tiles, st = it % tiles;
      const uint16_t* crow =
          (const uint16_t*)A.subkeys + ((size_t)head * 2 + half) * (size_t)s * hh + (size_t)(st * 32 + col) * hh;
#pragma unroll
      for (int k = 0; k < kMaxK16; ++k)
        if (k < nk) buf[k] = *(const uint4*)(crow + 16 * k + kq);
    };
    auto item_mul = [&](int it, const uint4 (&buf)[kMaxK16]) {
      const int half = it / tiles, st = it % tiles;
      float16_t acc = {};
#pragma unroll
      for (int k = 0; k < kMaxK16; ++k) {
        if (k < nk) {
          const uint4 xf = col < 2 * UPW ? *(const uint4*)(xs + col * d_k + half * hh + 16 * k + kq)
                                         : make_uint4(0u, 0u, 0u, 0u);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, buf[k]),
                                                        __builtin_bit_cast(bf16x8_t, xf), acc, 0, 0, 0);
        }
      }
      // D[row = sub-key][col]; lane holds col = lane % 32, rows 8*(i/4) + 4*(lane/32) + i%4
      if (col < 2 * UPW) {
        float* dst = (float*)(smem + L.unit0 + (size_t)(col >> 1) * L.unit + L.sc) +
                     ((col & 1) * 2 + half) * (s + 1) + st * 32;
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)] = acc[i];
      }
    };
    uint4 bufA[kMaxK16], bufB[kMaxK16];
    if (wave < items) item_load(wave, bufA);
    if (merger) stair_pairs<EM>(kappa, lwave == 0 ? W : R, pr, &bdiv);
    if (xl) *(uint4*)(xs + (xg * 2 + xvec) * d_k + xpc * 8) = xv;
    lds_barrier();  // k and q in LDS; the first item's loads stay in flight
    for (int it = wave; it < items; it += 2 * NW) {
      if (it + NW < items) item_load(it + NW, bufB);
      item_mul(it, bufA);
      if (it + NW < items) {
        if (it + 2 * NW < items) item_load(it + 2 * NW, bufA);
        item_mul(it + NW, bufB);
      }
    }
  } else {
    if (merger) stair_pairs<EM>(kappa, lwave == 0 ? W : R, pr, &bdiv);
    if (live) {
      for (int p = ltid; p < 4 * s; p += kGroup) {
        const int c = p / s, m = p % s, half = c & 1;
        const void* x = c < 2 ? A.k : A.q;
        const size_t xo = (size_t)u * d_k + (size_t)half * hh;
        const size_t co = ((size_t)head * 2 + half) * (size_t)s * hh + (size_t)m * hh;
        float acc = 0.f;
        for (int i = 0; i < hh; ++i) acc = fmaf(ld_in<BF16>(x, xo + i), ld_in<BF16>(A.subkeys, co + i), acc);
        sc[c * (s + 1) + m] = acc;
      }
    }
  }
  // this token's v, alpha and beta: their latency hides behind the selection
  float vpre[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    vpre[c] = (live && ltid < rowdw) ? ld_in<BF16>(A.v, (size_t)u * A.d_v + (size_t)ltid * CPL + c) : 0.f;
  const float al = A.alpha[u], be = A.beta[u];
  lds_barrier();
  // 2. per-half top-kappa, one wave per (vector, half) of each sequence
  if (live)
    select_half<ES>(sc + lwave * (s + 1), 0, s, kappa, wbuf, sel_i + lwave * kappa, sel_s + lwave * kappa);
  lds_barrier();
  // 3. kappa x kappa merge and softmax: the group's wave 0 for the key (W), wave 1 for the query (R)
  if (merger) {
    const int n_sel = lwave == 0 ? W : R;
    const int base = lwave * 2;
    const uint64_t key = merge_token<EM>(sel_i + base * kappa, sel_s + base * kappa, sel_i + (base + 1) * kappa,
                                         sel_s + (base + 1) * kappa, s, kappa, n_sel, pr, bdiv, wbuf);
    const float scv = lane < n_sel ? key_score(key) : -INFINITY;
    const float mx = __shfl(scv, 0, kWave);
    const float e = lane < n_sel ? expf(scv - mx) : 0.f;
    const float tot = wave_sum_f32(e);
    if (lane < n_sel) {
      if (lwave == 0) { swidx[lane] = (int32_t)key_index(key); swgt[lane] = e / tot; }
      else { sridx[lane] = (int32_t)key_index(key); srgt[lane] = e / tot; rmatch[lane] = -1; }
    }
    if (lwave == 0 && lane == 0) *anymatch = 0;
  }
  lds_barrier();
  // read slots that are write slots of this token: every (write, read) pair at once; write
  // slots are distinct, so at most one pair matches a read slot
  if (live) {
    for (int p = ltid; p < W * R; p += kGroup) {
      const int j = p / R, r = p - j * R;
      if (swidx[j] == sridx[r]) {
        rmatch[r] = j;
        *anymatch = 1;
      }
    }
  }
  lds_barrier();
  // whole-table decay: a write row's value before this token's decay is its stored value
  // times exp(lrun - lam); a read row's after it, times exp(lrun + log alpha - lam), or 1 for
  // a row this token writes
  double lnew = 0.0;
  if (A.lam) {
    if (live) {
      const double lold = A.lrun[u];
      lnew = lold + fmax(log((double)al), -1000.0);
      const double* lam = A.lam + (size_t)u * A.N;
      if (ltid < W) sfw[ltid] = expf((float)(lold - lam[swidx[ltid]]));
      if (ltid < R) sfr[ltid] = rmatch[ltid] >= 0 ? 1.f : expf((float)(lnew - lam[sridx[ltid]]));
    }
    __syncthreads();
  }
  // a read row written by its own token in any sequence of the workgroup: every group takes
  // the extra steps (barriers are workgroup-wide)
  bool matched_any = false;
#pragma unroll
  for (int gi = 0; gi < UPW; ++gi) {
    const int bg = (blockIdx.x / A.H) * UPW + gi;
    if (bg < A.B) matched_any |= *(const int*)(smem + L.unit0 + (size_t)gi * L.unit + L.flag) != 0;
  }
  const bool matched = live && *anymatch != 0;

  // 4. rows: thread = (row group g, row word dw). Every row the token touches is loaded in one
  // batch: its write rows, and the read rows it does not write (this token leaves them
  // unchanged), whose weighted sum is taken at once with the residual's. The output is final
  // before the write-back unless a read row is also a write row (then that row's new value is
  // added after the update). Barriers order LDS only: the write-back stores are never waited
  // for inside the kernel.
  const int G = kGroup / rowdw;
  const int g = ltid / rowdw, dw = ltid % rowdw;
  const bool act = live && g < G;
  uint32_t* Mu = (uint32_t*)A.M + (size_t)u * (size_t)A.N * rowdw;
  float acc[CPL], oacc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = oacc[c] = 0.f;
  if (act) {
    constexpr int kB = 8;  // rows of each list per thread in flight
    const int nw = (W - g + G - 1) / G, nr = (R - g + G - 1) / G;
    const int nb = nw > nr ? nw : nr;
    for (int b0 = 0; b0 < nb; b0 += kB) {
      uint32_t wv[kB], rv[kB];
#pragma unroll
      for (int bb = 0; bb < kB; ++bb) {
        const int j = g + G * (b0 + bb);
        wv[bb] = j < W ? Mu[(size_t)swidx[j] * rowdw + dw] : 0u;
        rv[bb] = (j < R && rmatch[j] < 0) ? Mu[(size_t)sridx[j] * rowdw + dw] : 0u;
      }
#pragma unroll
      for (int bb = 0; bb < kB; ++bb) {
        const int j = g + G * (b0 + bb);
        if (j < W) {
          wrow[j * rowdw + dw] = wv[bb];
          float x[CPL];
          MT::unpack(wv[bb], x);
          const float wx = A.lam ? swgt[j] * sfw[j] : swgt[j];
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wx, x[c], acc[c]);
        }
        if (j < R && rmatch[j] < 0) {
          float y[CPL];
          MT::unpack(rv[bb], y);
          const float wr = A.lam ? srgt[j] * sfr[j] : srgt[j];
#pragma unroll
          for (int c = 0; c < CPL; ++c) oacc[c] = fmaf(wr, y[c], oacc[c]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    part[ltid * CPL + c] = acc[c];
    opart[ltid * CPL + c] = oacc[c];
  }
  lds_barrier();
  float ov[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) ov[c] = 0.f;
  if (live && ltid < rowdw) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float rho = 0.f, os = 0.f;
      for (int gg = 0; gg < G; ++gg) {
        rho += part[(gg * rowdw + ltid) * CPL + c];
        os += opart[(gg * rowdw + ltid) * CPL + c];
      }
      sdelta[ltid * CPL + c] = be * (vpre[c] - al * rho);
      ov[c] = os;
    }
    if (!matched) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) A.o[(size_t)u * A.d_v + (size_t)ltid * CPL + c] = ov[c];
    }
  }
  lds_barrier();
  if (act) {
    for (int j = g; j < W; j += G) {
      float x[CPL], y[CPL];
      MT::unpack(wrow[j * rowdw + dw], x);
      const float ax = A.lam ? al * sfw[j] : al;
#pragma unroll
      for (int c = 0; c < CPL; ++c) y[c] = fmaf(ax, x[c], swgt[j] * sdelta[dw * CPL + c]);
      const uint32_t nw = MT::pack(y);
      Mu[(size_t)swidx[j] * rowdw + dw] = nw;
      if (matched) wrow[j * rowdw + dw] = nw;
    }
  }
  if (matched_any) {
    // read rows this token wrote, at their new values (decay factor 1)
    lds_barrier();
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    if (act && matched) {
      for (int r = g; r < R; r += G) {
        const int pos = rmatch[r];
        if (pos >= 0) {
          float x[CPL];
          MT::unpack(wrow[pos * rowdw + dw], x);
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] = fmaf(srgt[r], x[c], acc[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) part[ltid * CPL + c] = acc[c];
    lds_barrier();
    if (matched && ltid < rowdw) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float os = ov[c];
        for (int gg = 0; gg < G; ++gg) os += part[(gg * rowdw + ltid) * CPL + c];
        A.o[(size_t)u * A.d_v + (size_t)ltid * CPL + c] = os;
      }
    }
  }
  if (A.lam && live) {
    // the written slots now hold values as of this token
    if (ltid < W) A.lam[(size_t)u * A.N + swidx[ltid]] = lnew;
    if (ltid == 0) A.lrun[u] = lnew;
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

// Sequences per workgroup: 4 while the workgroup's LDS fits, else 1.
int dec_upw(const sdm_shape& S) {
  const int cpl = S.mem_dtype == SDM_BF16 ? 2 : 1;
  const int rowdw = S.d_v / cpl;
  return dec_lds(4, (int)isqrt64(S.N), S.kappa, S.W, S.R, rowdw, cpl, S.d_k).total <= 160 * 1024 ? 4 : 1;
}

template <bool BF16, typename MemT, int ES, int EM>
hipError_t dec_launch_u(const DecArgs& A, int upw, size_t lds, hipStream_t st) {
  const dim3 grid((unsigned)(A.H * ((A.B + upw - 1) / upw)));
  if (upw == 4) hipLaunchKernelGGL((decode_kernel<BF16, MemT, ES, EM, 4>), grid, dim3(kGroup * 4), lds, st, A);
  else hipLaunchKernelGGL((decode_kernel<BF16, MemT, ES, EM, 1>), grid, dim3(kGroup), lds, st, A);
  return hipGetLastError();
}
template <bool BF16, typename MemT, int ES>
hipError_t dec_launch_m(const DecArgs& A, int upw, size_t lds, hipStream_t st) {
  const int st_max = A.stairW > A.stairR ? A.stairW : A.stairR;
  const int em = (st_max + 63) / 64;
  if (em <= 1) return dec_launch_u<BF16, MemT, ES, 1>(A, upw, lds, st);
  if (em <= 2) return dec_launch_u<BF16, MemT, ES, 2>(A, upw, lds, st);
  if (em <= 4) return dec_launch_u<BF16, MemT, ES, 4>(A, upw, lds, st);
  return dec_launch_u<BF16, MemT, ES, 8>(A, upw, lds, st);
}
template <bool BF16, typename MemT>
hipError_t dec_launch_s(const DecArgs& A, int upw, size_t lds, hipStream_t st) {
  int es = (A.s + 63) / 64;
  if (es <= 1) return dec_launch_m<BF16, MemT, 1>(A, upw, lds, st);
  if (es <= 2) return dec_launch_m<BF16, MemT, 2>(A, upw, lds, st);
  if (es <= 4) return dec_launch_m<BF16, MemT, 4>(A, upw, lds, st);
  return dec_launch_m<BF16, MemT, 8>(A, upw, lds, st);
}

}  // namespace

size_t decode_lds_bytes(const sdm_shape& S) {
  const int cpl = S.mem_dtype == SDM_BF16 ? 2 : 1;
  const int rowdw = S.d_v / cpl;
  return dec_lds(dec_upw(S), (int)isqrt64(S.N), S.kappa, S.W, S.R, rowdw, cpl, S.d_k).total;
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
  A.B = S.B;
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
  const int upw = dec_upw(S);
  const size_t lds = decode_lds_bytes(S);
  const bool ib = S.in_dtype == SDM_BF16, mb = S.mem_dtype == SDM_BF16;
  if (ib && mb) return dec_launch_s<true, uint16_t>(A, upw, lds, stream);
  if (ib && !mb) return dec_launch_s<true, float>(A, upw, lds, stream);
  if (!ib && mb) return dec_launch_s<false, uint16_t>(A, upw, lds, stream);
  return dec_launch_s<false, float>(A, upw, lds, stream);
}

}  // namespace sdm
