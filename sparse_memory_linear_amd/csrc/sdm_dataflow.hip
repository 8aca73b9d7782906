// Pipelined execution of the sparse gated-delta recurrence, one workgroup per (unit, column
// block).
//
// Method (paperlayer.ai summary of arXiv:2607.07386v1, §2 "Gated DeltaNet", §3 "Sparse memory
// updates" and "Sparse retrieval"; App. A.2: two tokens interact only through the slots
// they share): token t of a (batch, head) unit reads its W write slots, writes them back,
// and reads its R read slots after its write. Two facts make this parallel without changing
// the result:
//   * every column of the table evolves on its own given the slots and weights, so a unit's
//     rows are split into P column blocks handled by P independent workgroups;
//   * two tokens depend on each other only through a slot they share; a token that finds
//     the latest writer of each of its slots among the last `win` tokens can take the row
//     from that writer on chip, and every other row from the table once all tokens older
//     than the window are stored.
//
// Inside a workgroup the tokens stream through two LDS rings: a token ring of S slots
// (S = 2 win: gathered rows, new write rows, output block) and a metadata ring of SM slots
// (packed slot words, weights, gates, v columns).
//   * wave 0 (meta) copies the metadata of each token into its ring with direct-to-LDS
//     loads, up to SM tokens ahead of the store wave;
//   * waves 1 and 3 (gather) load the table rows of each token's slots into registers, a
//     few 4-token steps in flight, and write them to the token ring; a token is gathered
//     once every token older than the window is in the table and its ring slot is free;
//   * waves 4.. (compute) take tokens in order; a token runs when its rows are in the ring
//     and its writers inside the window have published their new rows. It replaces its
//     write rows in the ring by their new values and leaves its output block there. It
//     never touches HBM;
//   * wave 2 (store) writes new rows and outputs to HBM in token order, several tokens per
//     instruction, and advances the watermark of completed stores. Storing in token order
//     keeps writes to one slot in order and after every earlier read of it.
// Each CU serves a bounded rate of vector-memory instructions; the gather and store paths
// are laid out to move each row block with one 8-byte lane and as few instructions as
// possible.
// The result is bit-identical to processing the tokens one after another.
//
// deps_kernel precomputes, per token and slot position, a packed word: the slot, and the
// latest writer inside the window (distance, position) if there is one.

#include <algorithm>

#include "sdm_device.hpp"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int kDepBlk = 128;       // tokens per deps workgroup (window offsets of entries stay below 256)
constexpr int kDepThreads = 512;
constexpr int kMaxHashBits = 15;   // deps hash table: at most 32768 entries, at most half full
constexpr int kDepFilterWords = 2048;  // 64K-bit filter of the slots in the deps hash table
constexpr uint32_t kEmpty = 0xFFFFFFFFu;
constexpr int kMaxWin = 127;
// packed slot word: [31] coded | [30:24] distance | [23:18] writer position | [17:0] slot,
// or [30] alone for a slot outside [0, N)
constexpr uint32_t kCoded = 0x80000000u;
constexpr uint32_t kInvalid = 0x40000000u;
constexpr uint32_t kSlotMask = 0x3FFFFu;
constexpr int kWaves = 16;         // meta, 2 gather, store, 12 compute waves
constexpr int kGatherWaves = 2;    // waves 1 and 3
constexpr int kGatherRegs = 80;    // registers a gather wave spends on rows in flight
constexpr int kMetaDepth = 4;      // meta batches in flight (3 loads each)
constexpr int kMetaRing = 64;      // metadata ring slots
constexpr int kGatherGroup = 4;    // tokens per gather step
constexpr int kStoreBatch = 8;     // tokens per store step (watermark granularity)
constexpr size_t kLdsBudget = 156 * 1024;
// Longest a wave waits (in units of s_sleep 2, ~53 ns): about 3.5 s. When it runs out the
// workgroup gives up (abort flag), every wave exits, and the workspace error word records
// it: the result is then invalid, but the kernel always terminates.
constexpr long long kSpinBudget = 1ll << 26;

typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ dependency pass
struct DepArgs {
  const int32_t* widx;  // [U][T][W]
  const int32_t* ridx;  // [U][T][R]
  uint32_t* pk;         // [U][T][W+R] packed slot words
  int T, W, R, win, bits;  // hash table of 2^bits entries
  long long N;
};

__device__ __forceinline__ uint32_t dep_hash(uint32_t slot, int bits) { return (slot * 2654435761u) >> (32 - bits); }
__device__ __forceinline__ uint32_t dep_filter_bit(uint32_t slot) { return (slot * 0x9E3779B1u) >> 16; }  // 16 bits

// hash entry = slot << 14 | window offset << 6 | writer position
__global__ void __launch_bounds__(kDepThreads) deps_kernel(DepArgs A) {
  extern __shared__ uint32_t table[];  // 2^bits entries, then the filter
  uint32_t* filt = table + (1 << A.bits);  // kDepFilterWords: a slot whose bit is clear is not in the table
  const int bits = A.bits;
  const uint32_t hmask = (1u << bits) - 1;
  const int u = blockIdx.y;
  const int t0 = blockIdx.x * kDepBlk;
  const int wlo = t0 - A.win > 0 ? t0 - A.win : 0;
  const int whi = t0 + kDepBlk < A.T ? t0 + kDepBlk : A.T;
  const int W = A.W, R = A.R, per = W + R;
  for (int i = threadIdx.x; i < (1 << bits); i += kDepThreads) table[i] = kEmpty;
  for (int i = threadIdx.x; i < kDepFilterWords; i += kDepThreads) filt[i] = 0u;
  __syncthreads();
  const int32_t* wi = A.widx + (size_t)u * A.T * W;
  const int32_t* ri = A.ridx + (size_t)u * A.T * R;
  // eight entries per thread at a time: their slot loads are in flight together
  constexpr int kB = 8;
  const int nins = (whi - wlo) * W;
  for (int e0 = threadIdx.x; e0 < nins; e0 += kDepThreads * kB) {
    int32_t sl[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int e = e0 + kDepThreads * b, k = e / W, j = e - k * W;
      sl[b] = e < nins ? wi[(size_t)(wlo + k) * W + j] : -1;
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int e = e0 + kDepThreads * b, k = e / W, j = e - k * W;
      const int32_t slot = sl[b];
      if (slot < 0 || slot >= A.N) continue;
      const uint32_t ent = ((uint32_t)slot << 14) | ((uint32_t)k << 6) | (uint32_t)j;
      uint32_t h = dep_hash((uint32_t)slot, bits);
      while (atomicCAS(&table[h], kEmpty, ent) != kEmpty) h = (h + 1) & hmask;
      const uint32_t fb = dep_filter_bit((uint32_t)slot);
      atomicOr(&filt[fb >> 5], 1u << (fb & 31));
    }
  }
  __syncthreads();
  uint32_t* out = A.pk + ((size_t)u * A.T + t0) * per;
  const int nlook = (whi - t0) * per;
  for (int e0 = threadIdx.x; e0 < nlook; e0 += kDepThreads * kB) {
    int32_t sl[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int e = e0 + kDepThreads * b, kk = e / per, p = e - kk * per, t = t0 + kk;
      sl[b] = e < nlook ? (p >= W ? ri[(size_t)t * R + (p - W)] : wi[(size_t)t * W + p]) : -1;
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int e = e0 + kDepThreads * b;
      if (e >= nlook) continue;
      const int kk = e / per, p = e - kk * per;
      const int t = t0 + kk, kt = t - wlo;
      const bool rd = p >= W;
      const int32_t slot = sl[b];
      uint32_t word = kInvalid;
      if (slot >= 0 && slot < A.N) {
        int best = -1, bestj = 0;
        const uint32_t fb = dep_filter_bit((uint32_t)slot);
        if ((filt[fb >> 5] >> (fb & 31)) & 1u) {
          uint32_t h = dep_hash((uint32_t)slot, bits);
          while (true) {
            const uint32_t ent = table[h];
            if (ent == kEmpty) break;
            if ((ent >> 14) == (uint32_t)slot) {
              const int k = (ent >> 6) & 255;
              const int d = kt - k;
              // latest writer: an earlier token, or this token itself for a read slot
              if ((rd ? d >= 0 : d >= 1) && d <= A.win && k > best) {
                best = k;
                bestj = ent & 63;
              }
            }
            h = (h + 1) & hmask;
          }
        }
        word = (uint32_t)slot;
        if (best >= 0) word |= kCoded | ((uint32_t)(kt - best) << 24) | ((uint32_t)bestj << 18);
      }
      out[e] = word;
    }
  }
}

// ------------------------------------------------------------------ recurrence pipeline
struct PipeArgs {
  const uint32_t* pk;  // [U][T][E] packed slot words (E = W + R: write slots, then read slots)
  const float* wgt;    // [U][T][W]
  const float* rgt;    // [U][T][R]
  const void* v;       // [U][T][d_v]
  const float* alpha;  // [U][T]
  const float* beta;   // [U][T]
  void* M;             // [U][N][d_v]
  float* o;            // [U][T][d_v]
  unsigned long long* err;
  int U, T, W, R, E, d_v, P;
  int S, RS, SM, win, tpb, vw, rowbytes;
  const float* fac;  // [U][T][E] decay factors of the accesses (whole-table decay), or null
  void* xlog;        // [U][T][W][d_v] pre-update write rows for the backward, or null
  int pack2;  // two tokens' write rows per store instruction
  int nh;     // compute passes per half wave: ceil(max(W, R) / (32 / lanes per row))
  long long N;
};

// The LB bytes of a row that one lane moves (8 or 16): LB/4 words of float32 or bf16 pairs.
template <int LB>
struct LaneVec;
template <>
struct LaneVec<8> {
  using V = u2;
};
template <>
struct LaneVec<16> {
  using V = u4;
};

template <typename MemT, int LB>
struct Lane {
  using V = typename LaneVec<LB>::V;
  static constexpr int kWords = LB / 4;
  static constexpr int kCols = LB / (int)sizeof(MemT);
  __device__ static void unpack(V w, float* x) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) {
      if constexpr (sizeof(MemT) == 2) {
        x[2 * i] = bf16lo(w[i]);
        x[2 * i + 1] = bf16hi(w[i]);
      } else {
        x[i] = __uint_as_float(w[i]);
      }
    }
  }
  __device__ static V pack(const float* x) {
    V w;
#pragma unroll
    for (int i = 0; i < kWords; ++i) {
      if constexpr (sizeof(MemT) == 2) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
      else w[i] = __float_as_uint(x[i]);
    }
    return w;
  }
};

__device__ __forceinline__ void buf_load(u2& d, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  d = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
}
__device__ __forceinline__ void buf_load(u4& d, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  d = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}
__device__ __forceinline__ void buf_store(u2 d, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(d, rs, off, 0, 0);
}
__device__ __forceinline__ void buf_store(u4 d, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(d, rs, off, 0, 0);
}

__device__ __forceinline__ int lds_ld(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// A word every lane reads at the same address, as a wave-uniform value: the loops and
// branches that depend on it stay scalar, and so does the token counter they advance.
__device__ __forceinline__ int lds_ld_u(const int* p) { return __builtin_amdgcn_readfirstlane(lds_ld(p)); }
__device__ __forceinline__ void lds_st(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void acquire_lds() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local"); }
__device__ __forceinline__ void release_lds() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local"); }

// The meta and gather waves keep direct-to-LDS loads in flight; the compiler would make every
// LDS access of those waves wait for all of them. Their LDS accesses are therefore written
// out: reads that wait for themselves only, and writes.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ int dma_wave_read(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ void dma_wave_write(int* p, int v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Control words at the start of LDS.
enum { kMetaDone = 1, kWm = 2, kStoreIssued = 3, kAbort = 4, kCtrlWords = 16 };

// Workgroup of kWaves waves serving one (unit, column block) of RB bytes per row. Lane
// layout of row work: LPC = RB/LB lanes (LB bytes each) per row, G = 64/LPC rows per pass;
// NP passes cover max(W, R) rows, NG passes cover the E = W + R rows gathered per token.
template <typename MemT, typename InT, int RB, int LB, int NP, int NG>
__global__ void __launch_bounds__(kWaves * 64) pipe_kernel(PipeArgs A) {
  using PT = Lane<MemT, LB>;
  using LV = typename PT::V;
  constexpr int CPL = PT::kCols;              // columns per lane
  constexpr int LPC = RB / LB;
  constexpr int G = 64 / LPC;
  constexpr int CPR = RB / (int)sizeof(MemT);  // columns per row block
  // outputs leave in pieces of OPL float32 columns, PPT pieces per token
  constexpr int OPL = CPR < 4 ? CPR : 4;
  constexpr int PPT = CPR / OPL;
  extern __shared__ __align__(16) unsigned char smem[];

  const int T = A.T, W = A.W, R = A.R, E = A.E, S = A.S, smask = A.S - 1, win = A.win, rmask = A.RS - 1;
  const int SM = A.SM, mmask = A.SM - 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane / LPC, l = lane % LPC;
  // XCD-aware placement: all column blocks of a unit go to the same XCD (workgroups are
  // dealt to the 8 XCDs round-robin), so they share its L2 for rows and per-token inputs.
  const int xcd = blockIdx.x & 7, kb = blockIdx.x >> 3;
  const int u = xcd + 8 * (kb / A.P);
  const int cb = kb % A.P;
  if (u >= A.U) return;

  int* ctrl = (int*)smem;
  int* g_tok = ctrl + kCtrlWords;  // [S] token whose rows are gathered in ring slot i
  int* f_tok = g_tok + S;          // [S] token whose new write rows are in slot i
  int* c_tok = f_tok + S;          // [S] token whose compute is complete in slot i
  // token ring (S slots): gathered then new write rows, write slots, output block; the
  // gathered read rows live in a shorter ring of RS slots (they are dead once the token's
  // compute is done, and a gather runs at most RS tokens ahead of the stores)
  unsigned char* wrows = (unsigned char*)(c_tok + S);                // [S][W][RB]
  unsigned char* rrows = wrows + (size_t)S * W * RB;                 // [RS][R][RB]
  int32_t* slot_w = (int32_t*)(rrows + (size_t)A.RS * R * RB);       // [S][W] slot of each write row, -1 = skip
  float* obuf = (float*)(slot_w + (size_t)S * W);                    // [S][CPR]
  // metadata ring (SM slots): packed slot words, weights, v columns and gates
  uint32_t* pk_r = (uint32_t*)(obuf + (size_t)S * CPR);             // [SM][E]
  float* wt_r = (float*)(pk_r + (size_t)SM * E);                    // [SM][E]
  uint32_t* vab_r = (uint32_t*)(wt_r + (size_t)SM * E);             // [SM][vw]
  float* fac_r = (float*)(vab_r + (size_t)SM * A.vw);                // [SM][E] decay factors (if any)

  for (int i = threadIdx.x; i < kCtrlWords; i += blockDim.x) ctrl[i] = 0;
  for (int i = threadIdx.x; i < 3 * S; i += blockDim.x) g_tok[i] = -1;
  __syncthreads();

  const size_t ut0 = (size_t)u * T;
  const uint32_t oob = 0x7FFFFFF0u;  // buffer offset past the end: loads give 0, stores are dropped
  const uint32_t colb = (uint32_t)(cb * RB + l * LB);
  auto wrow_ptr = [&](int sl, int j) -> LV* { return (LV*)(wrows + ((size_t)sl * W + j) * RB + l * LB); };
  auto rrow_ptr = [&](int rl, int r) -> LV* { return (LV*)(rrows + ((size_t)rl * R + r) * RB + l * LB); };
  auto give_up = [&]() {
    if (lane == 0) {
      lds_st(&ctrl[kAbort], 1);
      atomicAdd(A.err, 1ull << 40);
    }
  };

  if (wave == 0) {
    // ================================================================ meta wave
    const int tpb = A.tpb, vw = A.vw, vw2 = A.vw - 2;
    const int nb = (T + tpb - 1) / tpb;
    const size_t vrow = (size_t)A.d_v * sizeof(InT) / 4;         // words per token of v
    const size_t vcol = (size_t)cb * CPR * sizeof(InT) / 4;      // first word of this block
    // Each lane's sources for batch 0 and their per-batch strides (elements): the wave gates
    // the whole pipeline, so a batch advances one pointer per array instead of recomputing
    // 64-bit addresses. Lane q/4 carries words q..q+3 of the batch's packed words and weights
    // (token q / E, position q % E); lane l carries word l % vw of token l / vw's v columns
    // and gates.
    const int q4 = lane * 4, ttq = q4 / E, eq = q4 - ttq * E;
    const bool lq = q4 < tpb * E;
    const int ttv = lane / vw, kv = lane - ttv * vw;
    const bool lv = lane < tpb * vw;
    const uint32_t* pk_src = A.pk + (ut0 + ttq) * E + eq;
    const float* wt_src = eq < W ? A.wgt + (ut0 + ttq) * W + eq : A.rgt + (ut0 + ttq) * R + (eq - W);
    const uint32_t* v_src = kv < vw2 ? (const uint32_t*)A.v + (ut0 + ttv) * vrow + vcol + kv
                                     : (const uint32_t*)(kv == vw2 ? A.alpha : A.beta) + ut0 + ttv;
    const float* fac_src = A.fac ? A.fac + (ut0 + ttq) * E + eq : nullptr;
    const size_t pk_step = (size_t)E * tpb, wt_step = (size_t)(eq < W ? W : R) * tpb;
    const size_t v_step = (kv < vw2 ? vrow : (size_t)1) * tpb;
    int published = 0, s_seen = 0;
    long long budget = kSpinBudget;
    for (int b = 0; b < nb; ++b) {
      const int tb = b * tpb;
      const int need = tb + tpb - SM;  // metadata slots of this batch are free (older tokens stored)
      if (s_seen < need) {
        s_seen = dma_wave_read(&ctrl[kStoreIssued]);
        if (s_seen < need) {
          __builtin_amdgcn_s_waitcnt(0);
          if (tb > published) {
            published = tb;
            dma_wave_write(&ctrl[kMetaDone], published);
          }
          while ((s_seen = dma_wave_read(&ctrl[kStoreIssued])) < need) {
            if (--budget <= 0 || dma_wave_read(&ctrl[kAbort])) {
              give_up();
              return;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
      }
      const int sl0 = tb & mmask;
      {
        // every token of a full batch is valid; only the last batch checks them (a batch
        // always issues its 3 or 4 loads: its first token is valid)
        const bool full = tb + tpb <= T;
        const bool okq = lq && (full || tb + ttq < T);
        const bool okv = lv && (full || tb + ttv < T);
        if (okq) __builtin_amdgcn_global_load_lds(pk_src, (void*)(pk_r + (size_t)sl0 * E), 16, 0, 0);
        if (okq) __builtin_amdgcn_global_load_lds(wt_src, (void*)(wt_r + (size_t)sl0 * E), 16, 0, 0);
        if (okv) __builtin_amdgcn_global_load_lds(v_src, (void*)(vab_r + (size_t)sl0 * vw), 4, 0, 0);
        if (A.fac && okq) __builtin_amdgcn_global_load_lds(fac_src, (void*)(fac_r + (size_t)sl0 * E), 16, 0, 0);
        pk_src += pk_step;
        wt_src += wt_step;
        v_src += v_step;
        if (A.fac) fac_src += pk_step;
      }
      if (b >= kMetaDepth) {
        // exactly 3 (4 with decay factors) loads per batch: the batch kMetaDepth back is complete
        if (A.fac) wait_vmcnt<4 * kMetaDepth>();
        else wait_vmcnt<3 * kMetaDepth>();
        const int done = (b - kMetaDepth + 1) * tpb;
        if (done > published) {
          published = done;
          dma_wave_write(&ctrl[kMetaDone], published);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    dma_wave_write(&ctrl[kMetaDone], T);
    return;
  }

  if (wave == 1 || wave == 3) {
    // ================================================================ gather waves
    // Table rows of each token's slots, GB tokens per step, loaded into registers (LB bytes
    // a lane) and written to the rings GD own steps later. The two
    // waves take alternate steps. Slots with a writer inside the window come from the ring
    // instead: their loads (and those of slots outside [0, N)) are out of range and give 0.
    constexpr int GB = kGatherGroup;
    // own steps in flight: as many as kGatherRegs row registers hold, 3 to 6 (2 for four
    // passes per token)
    constexpr int GD0 = kGatherRegs / (GB * NG * (LB / 4));
    constexpr int GDmin = NG >= 4 ? 2 : 3;
    constexpr int GD = GD0 < GDmin ? GDmin : (GD0 > 6 ? 6 : GD0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (char*)A.M + (size_t)u * (size_t)A.N * A.rowbytes, (short)0, (int)((size_t)A.N * A.rowbytes), 0x00020000);
    const int nsteps = (T + GB - 1) / GB;
    const int gw = wave == 1 ? 0 : 1;  // own steps gw, gw + kGatherWaves, ...
    const int nown = nsteps > gw ? (nsteps - gw + kGatherWaves - 1) / kGatherWaves : 0;
    int m_seen = 0, wm_seen = 0, s_seen = 0;
    int done = -1;  // own step index last written to the ring
    bool aborted = false;
    long long budget = kSpinBudget;
    LV data[GD][GB][NG];
    // metadata in, every token older than the window stored, ring slots free (RS <= S - win)
    auto ready = [&](int tl) { return m_seen >= tl && wm_seen >= tl - 1 - win && s_seen >= tl - A.RS; };
    // own step i (held in d) into the ring, unless already written
    auto complete = [&](int i, const LV (&d)[GB][NG]) {
      if (i <= done) return;
      const int t0 = (gw + i * kGatherWaves) * GB;
#pragma unroll
      for (int tt = 0; tt < GB; ++tt) {
        const int t = t0 + tt;
        if (t < T) {
#pragma unroll
          for (int n = 0; n < NG; ++n) {
            const int e = n * G + g;
            if (e < W) *wrow_ptr(t & smask, e) = d[tt][n];
            else if (e < E) *rrow_ptr(t & rmask, e - W) = d[tt][n];
          }
        }
      }
      release_lds();
      if (lane < GB && t0 + lane < T) lds_st(&g_tok[(t0 + lane) & smask], t0 + lane);
      done = i;
    };
    auto issue = [&](int i, LV (&d)[GB][NG]) {
      const int t0 = (gw + i * kGatherWaves) * GB;
#pragma unroll
      for (int tt = 0; tt < GB; ++tt) {
        const int t = t0 + tt;
        const bool tv = t < T && !aborted;
        const int ml = t & mmask;
#pragma unroll
        for (int n = 0; n < NG; ++n) {
          const int e = n * G + g;
          const uint32_t p = (tv && e < E) ? pk_r[(size_t)ml * E + e] : kInvalid;
          const uint32_t off = (p & (kCoded | kInvalid)) ? oob : (p & kSlotMask) * (uint32_t)A.rowbytes + colb;
          buf_load(d[tt][n], rs, off);
        }
      }
    };
    for (int base = 0; base < nown + GD; base += GD) {
#pragma unroll
      for (int sidx = 0; sidx < GD; ++sidx) {
        const int i = base + sidx;
        // register set sidx holds own step i - GD: write it out
        if (i >= GD && i - GD < nown) complete(i - GD, data[sidx]);
        if (i < nown) {
          const int t0 = (gw + i * kGatherWaves) * GB;
          const int tl = t0 + GB < T ? t0 + GB : T;
          if (!ready(tl) && !aborted) {
            m_seen = lds_ld_u(&ctrl[kMetaDone]);
            wm_seen = lds_ld_u(&ctrl[kWm]);
            s_seen = lds_ld_u(&ctrl[kStoreIssued]);
            if (!ready(tl)) {
              // blocked: first write out every own step still in flight, oldest first
#pragma unroll
              for (int j = 1; j < GD; ++j)
                if (i - GD + j >= 0) complete(i - GD + j, data[(sidx + j) % GD]);
              while (true) {
                m_seen = lds_ld_u(&ctrl[kMetaDone]);
                wm_seen = lds_ld_u(&ctrl[kWm]);
                s_seen = lds_ld_u(&ctrl[kStoreIssued]);
                if (ready(tl)) break;
                if (--budget <= 0 || lds_ld_u(&ctrl[kAbort])) {
                  aborted = true;
                  break;
                }
                __builtin_amdgcn_s_sleep(1);
              }
            }
            acquire_lds();
          }
        }
        // every position issues its loads (past the end: out of range), so the number of
        // loads in flight is the same on every path and the waits above stay exact
        issue(i, data[sidx]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (aborted) give_up();
    return;
  }

  if (wave == 2) {
    // ================================================================ store wave
    constexpr int SB = kStoreBatch;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (char*)A.M + (size_t)u * (size_t)A.N * A.rowbytes, (short)0, (int)((size_t)A.N * A.rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        A.o + (size_t)u * T * A.d_v, (short)0, (int)((size_t)T * A.d_v * 4), 0x00020000);
    long long budget = kSpinBudget;
    for (int t0 = 0; t0 < T; t0 += SB) {
      bool drained = false;
      while (true) {
        const int t = t0 + lane;
        const bool wait = lane < SB && t < T && lds_ld(&c_tok[t & smask]) != t;
        if (ballot(wait) == 0ull) break;
        if (!drained) {
          // blocked: let the watermark cover every store issued so far
          __builtin_amdgcn_s_waitcnt(0);
          if (lane == 0) lds_st(&ctrl[kWm], t0);
          drained = true;
        }
        if (--budget <= 0 || lds_ld_u(&ctrl[kAbort])) {
          give_up();
          return;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      acquire_lds();
      // outputs of the whole batch in one instruction: lane k * PPT + p carries piece p of
      // token k
      float ov[OPL];
      uint32_t ooff;
      {
        const int k = lane / PPT, p = lane % PPT;
        const int t = t0 + k;
        const bool live = k < SB && t < T;
        const int sl = t & smask;
#pragma unroll
        for (int c = 0; c < OPL; ++c) ov[c] = live ? obuf[(size_t)sl * CPR + p * OPL + c] : 0.f;
        ooff = live ? (uint32_t)(((size_t)t * A.d_v + cb * CPR + p * OPL) * 4) : oob;
      }
      if (A.pack2) {
        // two tokens per row instruction (the write rows of a token fill at most half a wave)
        constexpr int HG = G / 2;
        const int h = g / HG, j = g % HG;
        LV val[SB / 2];
        uint32_t off[SB / 2];
#pragma unroll
        for (int m = 0; m < SB / 2; ++m) {
          const int t = t0 + 2 * m + h;
          const int sl = t & smask;
          const int n = (t < T && j < W) ? slot_w[(size_t)sl * W + j] : -1;
          val[m] = *wrow_ptr(sl, j < W ? j : 0);
          off[m] = n >= 0 ? (uint32_t)n * (uint32_t)A.rowbytes + colb : oob;
        }
#pragma unroll
        for (int m = 0; m < SB / 2; ++m) buf_store(val[m], rs, off[m]);
      } else {
        LV val[SB][NP];
        uint32_t off[SB][NP];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const int t = t0 + k;
          const int sl = t & smask;
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            const int j = i * G + g;
            const int n = (t < T && j < W) ? slot_w[(size_t)sl * W + j] : -1;
            val[k][i] = *wrow_ptr(sl, j < W ? j : W - 1);
            off[k][i] = n >= 0 ? (uint32_t)n * (uint32_t)A.rowbytes + colb : oob;
          }
        }
#pragma unroll
        for (int k = 0; k < SB; ++k)
#pragma unroll
          for (int i = 0; i < NP; ++i) buf_store(val[k][i], rs, off[k][i]);
      }
      if constexpr (OPL == 4) {
        u4 o4 = {__float_as_uint(ov[0]), __float_as_uint(ov[1]), __float_as_uint(ov[2]), __float_as_uint(ov[3])};
        __builtin_amdgcn_raw_buffer_store_b128(o4, ro, ooff, 0, 0);
      } else {
        u2 o2 = {__float_as_uint(ov[0]), __float_as_uint(ov[1])};
        __builtin_amdgcn_raw_buffer_store_b64(o2, ro, ooff, 0, 0);
      }
      release_lds();
      if (lane == 0) lds_st(&ctrl[kStoreIssued], t0 + SB);
      // the previous batch's stores are complete: every token before t0 is in the table
      // (a batch issues exactly SB/2 + 1 or SB * NP + 1 store instructions)
      if (A.pack2) wait_vmcnt<SB / 2 + 1>();
      else wait_vmcnt<SB * NP + 1>();
      if (lane == 0) lds_st(&ctrl[kWm], t0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) lds_st(&ctrl[kWm], T);
    return;
  }

  // ================================================================== compute waves
  // The lower half of the wave holds the token's write rows, the upper half its read rows
  // (GH rows per pass, NH passes). One butterfly inside each half gives at once the weighted
  // read of the write rows (lower half, the residual's read before decay) and the weighted
  // read of the read rows (upper half). A read row that the token itself writes is taken
  // after the write, with a second butterfly, only when the token has one.
  // Compute wave c takes tokens c, c + NC, c + 2 NC, ...
  constexpr int GH = 32 / LPC;
  constexpr int NH = 2 * NP;  // passes per half at most; A.nh of them are live
  constexpr int NC = kWaves - 4;
  const int hh = lane >> 5;
  const int gh = (lane & 31) / LPC;
  const int nrows = hh ? R : W, rbase = hh ? W : 0, nh = A.nh;
  bool aborted = false;
  for (int t = wave - 4; t < T && !aborted; t += NC) {
    const int sl = t & smask, rl = t & rmask;
    {
      long long budget = kSpinBudget;
      while (lds_ld_u(&g_tok[sl]) != t) {
        if (--budget <= 0 || lds_ld_u(&ctrl[kAbort])) {
          aborted = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (aborted) break;
    }
    acquire_lds();
    const int ml = t & mmask;
    const uint32_t* pks = pk_r + (size_t)ml * E;
    const float* wts = wt_r + (size_t)ml * E;
    const uint32_t* vab = vab_r + (size_t)ml * A.vw;
    uint32_t pw[NH];
    float wv[NH], xs[NH];  // weight; scale of the gathered row (decay factor of a write row)
    LV xv[NH];
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int j = i * GH + gh;
      const bool live = i < nh && j < nrows;
      const int jl = live ? j : 0;
      pw[i] = pks[rbase + jl];
      wv[i] = wts[rbase + jl];
      xs[i] = 1.f;
      if (A.fac) {
        // whole-table decay: a write row is scaled to its value before this token's decay,
        // a read row's weight to its value after it
        const float f = fac_r[(size_t)ml * E + rbase + jl];
        if (hh == 0) xs[i] = f;
        else wv[i] *= f;
      }
      // rows of this token's ring slot, all written by the gather (0 where not loaded)
      xv[i] = hh ? *rrow_ptr(rl, jl) : *wrow_ptr(sl, jl);
      if (!live) pw[i] = kInvalid;
    }
#pragma unroll
    for (int i = 0; i < NH; ++i)
      if ((pw[i] & (kCoded | kInvalid)) == kInvalid) wv[i] = 0.f;  // slots outside [0, N) carry no weight
    float vv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if constexpr (sizeof(InT) == 2) {
        const uint32_t w = vab[(l * CPL + c) >> 1];
        vv[c] = ((l * CPL + c) & 1) ? bf16hi(w) : bf16lo(w);
      } else {
        vv[c] = __uint_as_float(vab[l * CPL + c]);
      }
    }
    const float al = __uint_as_float(vab[A.vw - 2]);
    const float be = __uint_as_float(vab[A.vw - 1]);
    // wait for the writers inside the window to publish their new rows
    bool fwd = false;
#pragma unroll
    for (int i = 0; i < NH; ++i) fwd |= (pw[i] & kCoded) && ((pw[i] >> 24) & 127) > 0;
    bool own = false;  // a read row written by this token
#pragma unroll
    for (int i = 0; i < NH; ++i) own |= (pw[i] & kCoded) && ((pw[i] >> 24) & 127) == 0;
    if (ballot(fwd)) {
      long long budget = kSpinBudget;
      while (true) {
        bool wait = false;
#pragma unroll
        for (int i = 0; i < NH; ++i) {
          if (pw[i] & kCoded) {
            const int d = (pw[i] >> 24) & 127;
            if (d > 0) wait |= lds_ld(&f_tok[(sl - d) & smask]) != t - d;
          }
        }
        if (ballot(wait) == 0ull) break;
        if (--budget <= 0 || lds_ld_u(&ctrl[kAbort])) {
          aborted = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (aborted) break;
      acquire_lds();
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        if (pw[i] & kCoded) {
          const int d = (pw[i] >> 24) & 127, jj = (pw[i] >> 18) & 63;
          if (d > 0) xv[i] = *wrow_ptr((sl - d) & smask, jj);
        }
      }
    }
    if (A.xlog && hh == 0) {
      // the pre-update write rows as this token read them, for the backward's undo
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
          (char*)A.xlog + (size_t)u * T * W * A.rowbytes, (short)0, (int)((size_t)T * W * A.rowbytes), 0x00020000);
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int j = i * GH + gh;
        if (i < nh && j < W) buf_store(xv[i], xr, (uint32_t)(((size_t)t * W + j) * A.rowbytes) + colb);
      }
    }
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      if (i < nh) {
        float x[CPL];
        PT::unpack(xv[i], x);
        const float wx = wv[i] * xs[i];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wx, x[c], acc[c]);
      }
    }
#pragma unroll
    for (int s = LPC; s < 32; s <<= 1)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = add_xor_f32(acc[c], s);
    // lower half: delta = beta (v - alpha * read of the write rows); new write rows
    if (hh == 0) {
      float dl[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) dl[c] = be * (vv[c] - al * acc[c]);
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int j = i * GH + gh;
        if (i < nh && j < W) {
          float x[CPL], y[CPL];
          PT::unpack(xv[i], x);
          const float ax = al * xs[i];
#pragma unroll
          for (int c = 0; c < CPL; ++c) y[c] = fmaf(ax, x[c], wv[i] * dl[c]);
          *wrow_ptr(sl, j) = PT::pack(y);
          if (l == 0) slot_w[(size_t)sl * W + j] = (pw[i] & (kCoded | kInvalid)) == kInvalid ? -1 : (int)(pw[i] & kSlotMask);
          // a row rewritten by the next token goes out in the same store instruction as that
          // token's, where lane order is not defined: only the later token stores it
          if (A.pack2 && (t & 1) && l == 0 && (pw[i] & kCoded) && ((pw[i] >> 24) & 127) == 1)
            slot_w[(size_t)((sl - 1) & smask) * W + ((pw[i] >> 18) & 63)] = -1;
        }
      }
    }
    // upper half: read rows this token wrote, at their new values (own rows written just
    // above by this wave: its LDS accesses take effect in order)
    if (ballot(own)) {
      float cr[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) cr[c] = 0.f;
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        if ((pw[i] & kCoded) && ((pw[i] >> 24) & 127) == 0) {
          float y[CPL];
          PT::unpack(*wrow_ptr(sl, (pw[i] >> 18) & 63), y);
#pragma unroll
          for (int c = 0; c < CPL; ++c) cr[c] = fmaf(wv[i], y[c], cr[c]);
        }
      }
#pragma unroll
      for (int s = LPC; s < 32; s <<= 1)
#pragma unroll
        for (int c = 0; c < CPL; ++c) cr[c] = add_xor_f32(cr[c], s);
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += cr[c];
    }
    if (hh == 1 && gh == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) obuf[(size_t)sl * CPR + l * CPL + c] = acc[c];
    }
    // slot indices outside [0, N) were skipped; the first column block counts them
    if (cb == 0) {
      int bad = 0;
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int j = i * GH + gh;
        bad += popc64(ballot(l == 0 && i < nh && j < nrows && (pw[i] & (kCoded | kInvalid)) == kInvalid));
      }
      if (bad && lane == 0) atomicAdd(A.err, (unsigned long long)bad);
    }
    // new rows and output published together
    release_lds();
    if (lane == 0) {
      lds_st(&f_tok[sl], t);
      lds_st(&c_tok[sl], t);
    }
  }
  if (aborted) give_up();
}

// ------------------------------------------------------------------ configuration
struct PipeCfg {
  int rb, lb, P, S, RS, SM, win, tpb, vw, np, ng, nh;
  size_t lds;
};

int pow2_floor(int x) {
  int p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

// Ring and batch sizes for a block width of rb bytes per row moved in lanes of lb bytes;
// false if it does not fit.
bool pipe_fits(const sdm_shape& S, int rb, int lb, bool decay, PipeCfg* c) {
  const int msz = (int)dtype_size(S.mem_dtype), isz = (int)dtype_size(S.in_dtype);
  const int rowbytes = S.d_v * msz;
  if (rowbytes % rb || rb % lb) return false;
  const int E = S.W + S.R;
  const int lpc = rb / lb, G = 64 / lpc;
  const int np = (std::max(S.W, S.R) + G - 1) / G;
  int ng = (E + G - 1) / G;
  if (ng == 3) ng = 4;
  if (np > 2 || ng > 4 || np > ng) return false;
  if (lb == 16 && ng > 2) return false;  // the gather registers would not fit
  const int nh = (std::max(S.W, S.R) + G / 2 - 1) / (G / 2);  // compute passes per half wave
  if (nh > 2 * np) return false;
  const int cpr = rb / msz;
  if ((cpr * isz) % 4) return false;
  const int vw = cpr * isz / 4 + 2;
  if (vw > 64) return false;
  const int tpb = std::min(pow2_floor(std::max(1, 256 / E)), pow2_floor(64 / vw));
  const size_t tslot = 12 + (size_t)S.W * rb + (size_t)S.W * 4 + (size_t)cpr * 4;  // token ring slot
  const size_t rslot = (size_t)S.R * rb;                                          // read-row ring slot
  const size_t mslot = (size_t)E * (decay ? 12 : 8) + (size_t)vw * 4;              // metadata ring slot
  const size_t fixed = kCtrlWords * 4;
  // A metadata ring of 64 slots (32 only if nothing fits beside 64) and the longest token
  // ring that fits beside it. A longer metadata ring lets the metadata wave run far ahead and
  // take vector-memory issue slots from the gathers: measured slower at 128 slots, and slower
  // at 32 even with a token ring twice as long.
  int ring = 0, mring = 0, rring = 0;
  size_t bytes = 0;
  for (int m = kMetaRing; m >= kMetaRing / 2 && !ring; m /= 2)
    for (int r = 256; r >= 64; r /= 2) {
      const int w = std::min(kMaxWin, r / 2);
      const int rr = pow2_floor(r - w);
      // progress: a blocked gather step fits between the store wave and the window and
      // between the store wave and the end of the read-row ring, and a metadata batch
      // between the store wave and the end of the metadata ring
      if (kGatherGroup + kStoreBatch > w || kGatherGroup + kStoreBatch > rr) continue;
      if (kGatherGroup + tpb + kStoreBatch > m) continue;
      const size_t b = fixed + r * tslot + rr * rslot + m * mslot;
      if (b <= kLdsBudget) {
        ring = r;
        mring = m;
        rring = rr;
        bytes = b;
        break;
      }
    }
  if (!ring) return false;
  c->rb = rb;
  c->lb = lb;
  c->P = rowbytes / rb;
  c->S = ring;
  c->RS = rring;
  c->SM = mring;
  c->win = std::min(kMaxWin, ring / 2);
  c->tpb = tpb;
  c->vw = vw;
  c->np = np;
  c->ng = ng;
  c->nh = nh;
  c->lds = bytes;
  return true;
}

// Each workgroup processes every token of its unit, so its time per token bounds the whole
// unit: pick the block width that needs the fewest rounds of workgroups over the CUs. With
// one round and CUs to spare, narrower blocks (more workgroups, each with less arithmetic per
// token) are faster; once the chip is full, 16-byte lanes (half the row requests of 8-byte
// lanes for the same bytes) are.
bool pipe_config(const sdm_shape& S, int cus, bool decay, PipeCfg* out) {
  bool any = false;
  long long best_rounds = 0, best_wgs = 0;
  const long long U = (long long)S.B * S.H;
  for (int lb = 16; lb >= 8; lb /= 2)
    for (int rb = lb; rb <= 32; rb *= 2) {
      PipeCfg c;
      if (!pipe_fits(S, rb, lb, decay, &c) || c.S < 64) continue;
      const long long wgs = U * c.P;
      const long long rounds = (wgs + cus - 1) / cus;  // one 16-wave workgroup per CU
      const bool better = !any || rounds < best_rounds ||
                          (rounds == best_rounds && wgs <= cus && best_wgs <= cus && wgs > best_wgs);
      if (better) {
        *out = c;
        best_rounds = rounds;
        best_wgs = wgs;
        any = true;
      }
    }
  return any;
}

template <typename MemT, typename InT, int RB, int LB>
hipError_t pipe_launch_rb(const PipeArgs& A, const PipeCfg& c, hipStream_t st) {
  const int groups = (A.U + 7) / 8;
  dim3 grid(8 * groups * A.P);
  dim3 block(kWaves * 64);
  if (c.np == 1 && c.ng == 1) hipLaunchKernelGGL((pipe_kernel<MemT, InT, RB, LB, 1, 1>), grid, block, c.lds, st, A);
  else if (c.np == 1 && c.ng == 2) hipLaunchKernelGGL((pipe_kernel<MemT, InT, RB, LB, 1, 2>), grid, block, c.lds, st, A);
  else if (c.np == 2 && c.ng == 2) hipLaunchKernelGGL((pipe_kernel<MemT, InT, RB, LB, 2, 2>), grid, block, c.lds, st, A);
  else if constexpr (LB == 8) {
    if (c.np == 2 && c.ng == 4) hipLaunchKernelGGL((pipe_kernel<MemT, InT, RB, LB, 2, 4>), grid, block, c.lds, st, A);
    else if (c.np == 1 && c.ng == 4) hipLaunchKernelGGL((pipe_kernel<MemT, InT, RB, LB, 1, 4>), grid, block, c.lds, st, A);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename MemT, typename InT>
hipError_t pipe_launch(const PipeArgs& A, const PipeCfg& c, hipStream_t st) {
  if (c.lb == 16) {
    switch (c.rb) {
      case 16: return pipe_launch_rb<MemT, InT, 16, 16>(A, c, st);
      case 32: return pipe_launch_rb<MemT, InT, 32, 16>(A, c, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (c.rb) {
    case 8: return pipe_launch_rb<MemT, InT, 8, 8>(A, c, st);
    case 16: return pipe_launch_rb<MemT, InT, 16, 8>(A, c, st);
    case 32: return pipe_launch_rb<MemT, InT, 32, 8>(A, c, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  return cus;
}

bool dataflow_supported(const sdm_shape& S, bool decay) {
  if (S.W % 4 || S.R % 4) return false;  // weight lists move in 16-byte pieces
  if (S.N > (1 << 18)) return false;     // packed slot words hold 18-bit slots
  if ((size_t)S.N * S.d_v * dtype_size(S.mem_dtype) > 0x7FFFFFFFull) return false;  // buffer offsets
  if ((size_t)S.T * S.d_v * 4 > 0x7FFFFFFFull) return false;
  PipeCfg c;
  return pipe_config(S, 256, decay, &c);
}

size_t dataflow_deps_bytes(const sdm_shape& S) {
  return (size_t)S.B * S.H * (size_t)S.T * (size_t)(S.W + S.R) * 4;
}

size_t dataflow_sched_words(const sdm_shape& S) {
  (void)S;
  return 0;
}

hipError_t launch_dataflow(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                           const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                           void* ws, const WsLayout& L, const DecayState* dk, void* xlog, hipStream_t stream) {
  PipeCfg c;
  if (!pipe_config(S, device_cus(), dk != nullptr, &c)) return hipErrorInvalidValue;
  const int U = S.B * S.H;
  char* w = (char*)ws;
  uint32_t* pk = (uint32_t*)(w + L.deps);
  DepArgs D;
  D.widx = widx;
  D.ridx = ridx;
  D.pk = pk;
  D.T = S.T;
  D.W = S.W;
  D.R = S.R;
  D.win = c.win;
  D.N = S.N;
  // at most half full: writers of one block and its window
  D.bits = 10;
  while (D.bits < kMaxHashBits && (1 << D.bits) < 2 * (kDepBlk + c.win) * S.W) ++D.bits;
  hipLaunchKernelGGL(deps_kernel, dim3((S.T + kDepBlk - 1) / kDepBlk, U), dim3(kDepThreads), ((size_t)4 << D.bits) + kDepFilterWords * 4, stream, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* fac = nullptr;
  if (dk) {
    // whole-table decay: cumulative log-decay per token, then every access's factor
    double* Ltok = (double*)(w + L.ltok);
    fac = (float*)(w + L.fac);
    e = launch_log_decay_scan(S, alpha, Ltok, dk->lrun, stream);
    if (e != hipSuccess) return e;
    e = launch_decay_pass(S, pk, Ltok, dk->lam, fac, (int*)(w + L.lastw), (int*)(w + L.segl), c.win, stream);
    if (e != hipSuccess) return e;
  }
  PipeArgs A;
  A.pk = pk;
  A.fac = fac;
  A.xlog = xlog;
  A.wgt = wgt;
  A.rgt = rgt;
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  A.M = M;
  A.o = o;
  A.err = (unsigned long long*)(w + L.err);
  A.U = U;
  A.T = S.T;
  A.W = S.W;
  A.R = S.R;
  A.E = S.W + S.R;
  A.d_v = S.d_v;
  A.P = c.P;
  A.S = c.S;
  A.RS = c.RS;
  A.SM = c.SM;
  A.win = c.win;
  A.tpb = c.tpb;
  A.vw = c.vw;
  A.rowbytes = S.d_v * (int)dtype_size(S.mem_dtype);
  A.N = S.N;
  A.pack2 = (c.np == 1 && 2 * S.W <= 64 / (c.rb / c.lb)) ? 1 : 0;
  A.nh = c.nh;
  const bool mb = S.mem_dtype == SDM_BF16, ib = S.in_dtype == SDM_BF16;
  if (mb && ib) return pipe_launch<uint16_t, uint16_t>(A, c, stream);
  if (mb && !ib) return pipe_launch<uint16_t, float>(A, c, stream);
  if (!mb && ib) return pipe_launch<float, uint16_t>(A, c, stream);
  return pipe_launch<float, float>(A, c, stream);
}

}  // namespace sdm
