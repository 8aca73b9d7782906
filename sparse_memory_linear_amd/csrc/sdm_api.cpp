// C ABI of the SDM layer forward: argument validation, workspace layout, launches.
// Every check runs on the host before the first HIP call, so argument errors never touch
// the GPU.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/sdm.h"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int64_t kMaxN = 262144;  // s <= 512: one half's scores of 32 tokens fit in LDS
constexpr int kMaxSel = 64;
constexpr size_t kAlign = 256;
constexpr size_t kMaxLds = 160 * 1024;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// sdm_forward runs the recurrence in its chunkwise two-phase form instead of the pipeline
// where the two agree up to float32 summation order and the chunkwise form was measured
// faster: a float32 table (the chunkwise form rounds rows to the table dtype only at each
// chunk's write-back, which for float32 changes nothing but the order of the float32 sums)
// and at least 32 units (their chunk workgroups fill the chip; with one unit the pipeline is
// faster). Not for the whole-table decay variant, which runs on the pipeline only.
bool forward_uses_chunkwise(const sdm_shape& S, bool decay) {
  return !decay && S.mem_dtype == SDM_F32 && (int64_t)S.B * S.H >= 32 && chunked_supported(S);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

// [p, p+n) and [q, q+m) overlap?
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + m && b < a + n;
}

sdm_status check_shape(const sdm_shape* S, bool allow_t0) {
  if (!S) return SDM_ERR_INVALID_ARG;
  if (S->B < 1 || S->H < 1 || S->T < (allow_t0 ? 0 : 1)) return SDM_ERR_INVALID_ARG;
  if (S->in_dtype != SDM_F32 && S->in_dtype != SDM_BF16) return SDM_ERR_INVALID_ARG;
  if (S->mem_dtype != SDM_F32 && S->mem_dtype != SDM_BF16) return SDM_ERR_INVALID_ARG;
  if (S->N < 4) return SDM_ERR_INVALID_ARG;
  const int64_t s = isqrt64(S->N);
  if (s * s != S->N) return SDM_ERR_INVALID_ARG;
  if (S->N > kMaxN) return SDM_ERR_UNSUPPORTED;
  if (S->d_k < 2 || (S->d_k & 1)) return SDM_ERR_INVALID_ARG;
  if (S->d_k > 256) return SDM_ERR_UNSUPPORTED;
  if (S->d_v < 1) return SDM_ERR_INVALID_ARG;
  const size_t rowbytes = (size_t)S->d_v * dtype_size(S->mem_dtype);
  if (rowbytes % 16 != 0) return SDM_ERR_UNSUPPORTED;
  if (rowbytes > 1024) return SDM_ERR_UNSUPPORTED;
  if (S->kappa < 1 || S->kappa > s) return SDM_ERR_INVALID_ARG;
  if (S->kappa > kMaxSel) return SDM_ERR_UNSUPPORTED;
  const int64_t k2 = (int64_t)S->kappa * S->kappa;
  if (S->W < 1 || S->R < 1 || S->W > k2 || S->R > k2) return SDM_ERR_INVALID_ARG;
  if (S->W > kMaxSel || S->R > kMaxSel) return SDM_ERR_UNSUPPORTED;
  // index arithmetic: tokens per head and elements per tensor stay in range
  const int64_t BT = (int64_t)S->B * S->T;
  if (BT > (int64_t)INT32_MAX / 2) return SDM_ERR_UNSUPPORTED;
  size_t n;
  if (!mul_ok((size_t)S->B * (size_t)S->H, (size_t)S->N, &n) || !mul_ok(n, rowbytes, &n)) return SDM_ERR_UNSUPPORTED;
  if ((size_t)S->B * S->H > 65535u * 64u) return SDM_ERR_UNSUPPORTED;
  if (address_lds_bytes((int)s, S->kappa) > kMaxLds) return SDM_ERR_UNSUPPORTED;
  return SDM_OK;
}

size_t tensor_bytes(const sdm_shape& S, int64_t last, size_t esize) {
  return (size_t)S.B * S.H * (size_t)S.T * (size_t)last * esize;
}

sdm_status hip_status(hipError_t e) { return e == hipSuccess ? SDM_OK : SDM_ERR_HIP; }

// Validation of the whole-table decay state against the table, outputs and workspace.
sdm_status check_decay(const sdm_shape* S, const double* lam, const double* lrun, const void* M, size_t mb,
                       const void* o, size_t ob, const void* ws, size_t ws_bytes) {
  if (!lam && !lrun) return SDM_OK;
  if (!lam || !lrun || !aligned16(lam) || !aligned16(lrun)) return SDM_ERR_INVALID_ARG;
  const size_t U = (size_t)S->B * S->H;
  const size_t lb = U * (size_t)S->N * 8, rb = U * 8;
  if (overlaps(lam, lb, lrun, rb) || overlaps(lam, lb, M, mb) || overlaps(lrun, rb, M, mb) || overlaps(lam, lb, o, ob) ||
      overlaps(lrun, rb, o, ob) || overlaps(lam, lb, ws, ws_bytes) || overlaps(lrun, rb, ws, ws_bytes))
    return SDM_ERR_INVALID_ARG;
  return SDM_OK;
}

sdm_status recurrent_impl(const sdm_shape* S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                          const float* rgt, const void* v, const float* alpha, const float* beta, void* M, double* lam,
                          double* lrun, float* o, void* ws, size_t ws_bytes, void* stream, void* xlog = nullptr) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!widx || !wgt || !ridx || !rgt || !v || !alpha || !beta || !M || !o) return SDM_ERR_INVALID_ARG;
  const void* ptrs[] = {widx, wgt, ridx, rgt, v, alpha, beta, M, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDM_ERR_INVALID_ARG;
  const bool decay = lam != nullptr;
  if (decay && !dataflow_supported(*S, true)) return SDM_ERR_UNSUPPORTED;
  const WsLayout L = workspace_layout(*S, decay);
  if (!ws || ws_bytes < L.total) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_INVALID_ARG;
  const size_t mb = (size_t)S->B * S->H * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  const size_t ob = tensor_bytes(*S, S->d_v, 4);
  if (overlaps(M, mb, o, ob) || overlaps(M, mb, ws, ws_bytes) || overlaps(o, ob, ws, ws_bytes)) return SDM_ERR_INVALID_ARG;
  st = check_decay(S, lam, lrun, M, mb, o, ob, ws, ws_bytes);
  if (st != SDM_OK) return st;
  if (xlog) {
    if (!aligned16(xlog)) return SDM_ERR_INVALID_ARG;
    const size_t lb = tensor_bytes(*S, (int64_t)S->W * S->d_v, dtype_size(S->mem_dtype));
    if (overlaps(xlog, lb, M, mb) || overlaps(xlog, lb, o, ob) || overlaps(xlog, lb, ws, ws_bytes))
      return SDM_ERR_INVALID_ARG;
    // one unit's log is addressed with 32-bit buffer offsets
    if ((size_t)S->T * S->W * S->d_v * dtype_size(S->mem_dtype) > 0x7FFFFFFFull) return SDM_ERR_UNSUPPORTED;
  }
  if (S->T == 0) return SDM_OK;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = launch_zero((char*)ws + L.err, 1, hs);
  if (e != hipSuccess) return SDM_ERR_HIP;
  DecayState dk{lam, lrun};
  return hip_status(
      launch_recurrent(*S, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, L, decay ? &dk : nullptr, hs, xlog));
}

// Workspace of sdm_forward_static: one array per GPU (each device holds its own copy of a
// __device__ variable), never passed to a kernel by name; its device address is looked up
// once per device and kept.
__device__ __align__(256) unsigned char scratch[SDM_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, or null on a HIP error.
void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

// use_static: the workspace is the library's scratch array (ws and ws_bytes are ignored);
// it is looked up only after every argument check has passed.
sdm_status forward_impl(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const void* subkeys, void* M, double* lam, double* lrun, float* o,
                        int32_t* widx_out, int32_t* ridx_out, void* ws, size_t ws_bytes, void* stream,
                        bool use_static = false) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!q || !k || !v || !alpha || !beta || !subkeys || !M || !o) return SDM_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, alpha, beta, subkeys, M, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDM_ERR_INVALID_ARG;
  if ((widx_out && !aligned16(widx_out)) || (ridx_out && !aligned16(ridx_out))) return SDM_ERR_INVALID_ARG;
  const bool decay = lam != nullptr;
  if (decay && !dataflow_supported(*S, true)) return SDM_ERR_UNSUPPORTED;
  const WsLayout L = workspace_layout(*S, decay);
  if (use_static) {
    if (L.total > SDM_STATIC_SCRATCH_BYTES) return SDM_ERR_WORKSPACE;
    ws = nullptr;  // not known yet: it overlaps no caller buffer
    ws_bytes = 0;
  } else {
    if (!ws || ws_bytes < L.total) return SDM_ERR_WORKSPACE;
    if (!aligned16(ws)) return SDM_ERR_INVALID_ARG;
  }
  const size_t mb = (size_t)S->B * S->H * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  const size_t ob = tensor_bytes(*S, S->d_v, 4);
  const size_t xb = tensor_bytes(*S, S->d_k, dtype_size(S->in_dtype));
  const size_t vb = tensor_bytes(*S, S->d_v, dtype_size(S->in_dtype));
  const size_t wb = tensor_bytes(*S, S->W, 4), rb = tensor_bytes(*S, S->R, 4);
  if (overlaps(M, mb, o, ob) || overlaps(M, mb, ws, ws_bytes) || overlaps(o, ob, ws, ws_bytes) ||
      overlaps(M, mb, q, xb) || overlaps(M, mb, k, xb) || overlaps(M, mb, v, vb) || overlaps(o, ob, q, xb) ||
      overlaps(o, ob, k, xb) || overlaps(o, ob, v, vb) || overlaps(widx_out, wb, ws, ws_bytes) ||
      overlaps(ridx_out, rb, ws, ws_bytes) || overlaps(widx_out, wb, M, mb) || overlaps(ridx_out, rb, M, mb) ||
      overlaps(widx_out, wb, ridx_out, rb))
    return SDM_ERR_INVALID_ARG;
  st = check_decay(S, lam, lrun, M, mb, o, ob, ws, ws_bytes);
  if (st != SDM_OK) return st;
  if (S->T == 0) return SDM_OK;
  if (use_static) {
    ws = static_scratch();
    if (!ws) return SDM_ERR_HIP;
    ws_bytes = SDM_STATIC_SCRATCH_BYTES;
  }
  hipStream_t hs = (hipStream_t)stream;
  char* w = (char*)ws;
  int32_t* widx = widx_out ? widx_out : (int32_t*)(w + L.widx);
  int32_t* ridx = ridx_out ? ridx_out : (int32_t*)(w + L.ridx);
  float* wgt = (float*)(w + L.wgt);
  float* rgt = (float*)(w + L.rgt);
  hipError_t e = launch_address(*S, k, subkeys, S->W, widx, wgt, nullptr, hs);
  if (e != hipSuccess) return SDM_ERR_HIP;
  e = launch_address(*S, q, subkeys, S->R, ridx, rgt, nullptr, hs);
  if (e != hipSuccess) return SDM_ERR_HIP;
  e = launch_zero(w + L.err, 1, hs);
  if (e != hipSuccess) return SDM_ERR_HIP;
  if (forward_uses_chunkwise(*S, decay))
    return hip_status(launch_chunked(*S, widx, wgt, ridx, rgt, v, alpha, beta, M, o, w + L.chunk, hs));
  DecayState dk{lam, lrun};
  return hip_status(launch_recurrent(*S, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, L, decay ? &dk : nullptr, hs));
}

sdm_status decode_impl(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const void* subkeys, void* M, double* lam, double* lrun, float* o,
                       void* stream) {
  sdm_status st = check_shape(S, false);
  if (st != SDM_OK) return st;
  if (S->T != 1) return SDM_ERR_INVALID_ARG;
  if (!q || !k || !v || !alpha || !beta || !subkeys || !M || !o) return SDM_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, alpha, beta, subkeys, M, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDM_ERR_INVALID_ARG;
  const int cpl = S->mem_dtype == SDM_BF16 ? 2 : 1;
  if (S->d_v / cpl > 256) return SDM_ERR_UNSUPPORTED;
  if (decode_lds_bytes(*S) > kMaxLds) return SDM_ERR_UNSUPPORTED;
  const size_t mb = (size_t)S->B * S->H * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  const size_t ob = tensor_bytes(*S, S->d_v, 4);
  if (overlaps(M, mb, o, ob)) return SDM_ERR_INVALID_ARG;
  st = check_decay(S, lam, lrun, M, mb, o, ob, nullptr, 0);
  if (st != SDM_OK) return st;
  DecayState dk{lam, lrun};
  return hip_status(launch_decode(*S, q, k, v, alpha, beta, subkeys, M, o, lam ? &dk : nullptr, (hipStream_t)stream));
}

}  // namespace

WsLayout workspace_layout(const sdm_shape& S, bool decay) {
  WsLayout L;
  const size_t tok = (size_t)S.B * S.H * (size_t)S.T;
  size_t o = 0;
  L.err = o; o = align_up(o + 8);  // fixed place: offset 0 (read by sdm_workspace_error)
  L.widx = o; o = align_up(o + tok * S.W * 4);
  L.wgt = o; o = align_up(o + tok * S.W * 4);
  L.ridx = o; o = align_up(o + tok * S.R * 4);
  L.rgt = o; o = align_up(o + tok * S.R * 4);
  L.deps = o;
  L.sched = o;
  L.ltok = o;
  L.fac = o;
  L.lastw = o;
  L.segl = o;
  if (dataflow_supported(S, decay)) {
    o = align_up(o + dataflow_deps_bytes(S));
    L.sched = o;
    o = align_up(o + dataflow_sched_words(S) * 4);
    if (decay) {
      L.ltok = o;
      o = align_up(o + (size_t)S.B * S.H * ((size_t)S.T + 1) * 8);
      L.fac = o;
      o = align_up(o + tensor_bytes(S, (int64_t)S.W + S.R, 4));
      L.lastw = o;
      o = align_up(o + (size_t)S.B * S.H * (size_t)S.N * 4);
      L.segl = o;
      o = align_up(o + (size_t)(decay_segments(S) - 1) * S.B * S.H * (size_t)S.N * 4);
    }
  }
  // the chunkwise form's per-chunk lists, where sdm_forward takes it (same region as the
  // pipeline's dependency words: a call uses one or the other)
  L.chunk = L.deps;
  if (forward_uses_chunkwise(S, decay)) o = std::max(o, align_up(L.chunk + chunked_workspace_bytes(S)));
  L.total = o;
  return L;
}

}  // namespace sdm

using namespace sdm;

extern "C" {

const char* sdm_status_string(int status) {
  switch (status) {
    case SDM_OK: return "SDM_OK";
    case SDM_ERR_INVALID_ARG: return "SDM_ERR_INVALID_ARG";
    case SDM_ERR_UNSUPPORTED: return "SDM_ERR_UNSUPPORTED";
    case SDM_ERR_WORKSPACE: return "SDM_ERR_WORKSPACE";
    case SDM_ERR_HIP: return "SDM_ERR_HIP";
    case SDM_ERR_INTERNAL: return "SDM_ERR_INTERNAL";
    default: return "SDM_ERR_UNKNOWN";
  }
}

int sdm_abi_version(void) { return SDM_ABI_VERSION; }

int sdm_forward_uses_chunkwise(const sdm_shape* shape) {
  if (check_shape(shape, true) != SDM_OK) return -1;
  return forward_uses_chunkwise(*shape, false) ? 1 : 0;
}

sdm_status sdm_check_shape(const sdm_shape* shape) { return check_shape(shape, true); }

size_t sdm_workspace_bytes(const sdm_shape* shape) {
  if (check_shape(shape, true) != SDM_OK) return 0;
  return workspace_layout(*shape).total;
}

sdm_status sdm_init_from_M0(const sdm_shape* S, const void* M0, void* M, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!M0 || !M || !aligned16(M0) || !aligned16(M)) return SDM_ERR_INVALID_ARG;
  const size_t head_bytes = (size_t)S->H * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  if (overlaps(M0, head_bytes, M, head_bytes * S->B)) return SDM_ERR_INVALID_ARG;
  return hip_status(launch_init(*S, M0, M, (hipStream_t)stream));
}

namespace {
sdm_status address_checks(const sdm_shape* S, const void* x, const void* subkeys, int32_t n_sel, int32_t* idx,
                          float* weight, float* score) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (n_sel < 1 || (int64_t)n_sel > (int64_t)S->kappa * S->kappa) return SDM_ERR_INVALID_ARG;
  if (n_sel > kMaxSel) return SDM_ERR_UNSUPPORTED;
  if (!x || !subkeys || !idx || !weight) return SDM_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(subkeys) || !aligned16(idx) || !aligned16(weight) || (score && !aligned16(score)))
    return SDM_ERR_INVALID_ARG;
  const size_t ob = tensor_bytes(*S, n_sel, 4);
  const size_t xb = tensor_bytes(*S, S->d_k, dtype_size(S->in_dtype));
  if (overlaps(idx, ob, weight, ob) || (score && (overlaps(score, ob, idx, ob) || overlaps(score, ob, weight, ob))) ||
      overlaps(idx, ob, x, xb) || overlaps(weight, ob, x, xb))
    return SDM_ERR_INVALID_ARG;
  return SDM_OK;
}
}  // namespace

sdm_status sdm_address(const sdm_shape* S, const void* x, const void* subkeys, int32_t n_sel, int32_t* idx,
                       float* weight, float* score, void* stream) {
  sdm_status st = address_checks(S, x, subkeys, n_sel, idx, weight, score);
  if (st != SDM_OK) return st;
  if (S->T == 0) return SDM_OK;
  return hip_status(launch_address(*S, x, subkeys, n_sel, idx, weight, score, (hipStream_t)stream));
}

sdm_status sdm_address_init(const sdm_shape* S, const void* x, const void* subkeys, int32_t n_sel, int32_t* idx,
                            float* weight, float* score, const void* M0, void* M, int32_t part, int32_t nparts,
                            void* stream) {
  sdm_status st = address_checks(S, x, subkeys, n_sel, idx, weight, score);
  if (st != SDM_OK) return st;
  if (nparts < 1 || nparts > 64 || part < 0 || part >= nparts) return SDM_ERR_INVALID_ARG;
  if (!M0 || !M || !aligned16(M0) || !aligned16(M)) return SDM_ERR_INVALID_ARG;
  const size_t head_bytes = (size_t)S->H * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  const size_t mb = head_bytes * S->B;
  const size_t ob = tensor_bytes(*S, n_sel, 4);
  const size_t xb = tensor_bytes(*S, S->d_k, dtype_size(S->in_dtype));
  const size_t cb = (size_t)S->H * 2 * (size_t)isqrt64(S->N) * (S->d_k / 2) * dtype_size(S->in_dtype);
  if (overlaps(M0, head_bytes, M, mb) || overlaps(M, mb, x, xb) || overlaps(M, mb, subkeys, cb) ||
      overlaps(M, mb, idx, ob) || overlaps(M, mb, weight, ob) || (score && overlaps(M, mb, score, ob)))
    return SDM_ERR_INVALID_ARG;
  const InitPart ip{M0, M, part, nparts};
  return hip_status(launch_address(*S, x, subkeys, n_sel, idx, weight, score, (hipStream_t)stream, &ip));
}

sdm_status sdm_recurrent(const sdm_shape* S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                         const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                         void* ws, size_t ws_bytes, void* stream) {
  return recurrent_impl(S, widx, wgt, ridx, rgt, v, alpha, beta, M, nullptr, nullptr, o, ws, ws_bytes, stream);
}

sdm_status sdm_forward(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const void* subkeys, void* M, float* o, int32_t* widx_out,
                       int32_t* ridx_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(S, q, k, v, alpha, beta, subkeys, M, nullptr, nullptr, o, widx_out, ridx_out, ws, ws_bytes,
                      stream);
}

sdm_status sdm_forward_static(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const void* subkeys, void* M, float* o, int32_t* widx_out,
                              int32_t* ridx_out, void* stream) {
  return forward_impl(S, q, k, v, alpha, beta, subkeys, M, nullptr, nullptr, o, widx_out, ridx_out, nullptr, 0,
                      stream, true);
}

sdm_status sdm_decode_step(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const void* subkeys, void* M, float* o, void* stream) {
  return decode_impl(S, q, k, v, alpha, beta, subkeys, M, nullptr, nullptr, o, stream);
}

sdm_status sdm_recurrent_log(const sdm_shape* S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                             const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                             void* xlog, void* ws, size_t ws_bytes, void* stream) {
  if (!xlog) return SDM_ERR_INVALID_ARG;
  return recurrent_impl(S, widx, wgt, ridx, rgt, v, alpha, beta, M, nullptr, nullptr, o, ws, ws_bytes, stream, xlog);
}

sdm_status sdm_address_backward(const sdm_shape* S, const void* x, const void* subkeys, int32_t n_sel,
                                const int32_t* idx, const float* weight, const float* dweight, float* dx,
                                float* dsub, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (n_sel < 1 || (int64_t)n_sel > (int64_t)S->kappa * S->kappa) return SDM_ERR_INVALID_ARG;
  if (n_sel > kMaxSel) return SDM_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, subkeys, idx, weight, dweight, dx, dsub};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return SDM_ERR_INVALID_ARG;
  const int64_t s = isqrt64(S->N);
  const size_t xb = tensor_bytes(*S, S->d_k, dtype_size(S->in_dtype));
  const size_t kb = (size_t)S->H * 2 * (size_t)s * (S->d_k / 2) * dtype_size(S->in_dtype);
  const size_t ib = tensor_bytes(*S, n_sel, 4);
  const size_t dxb = tensor_bytes(*S, S->d_k, 4), dsb = (size_t)S->H * 2 * (size_t)s * (S->d_k / 2) * 4;
  const void* ins[] = {x, subkeys, idx, weight, dweight};
  const size_t isz[] = {xb, kb, ib, ib, ib};
  for (int j = 0; j < 5; ++j)
    if (overlaps(dx, dxb, ins[j], isz[j]) || overlaps(dsub, dsb, ins[j], isz[j])) return SDM_ERR_INVALID_ARG;
  if (overlaps(dx, dxb, dsub, dsb)) return SDM_ERR_INVALID_ARG;
  if (S->T == 0) return SDM_OK;
  return hip_status(launch_address_backward(*S, x, subkeys, n_sel, idx, weight, dweight, dx, dsub,
                                            (hipStream_t)stream));
}

size_t sdm_workspace_bytes_chunked(const sdm_shape* shape) {
  if (check_shape(shape, true) != SDM_OK || !chunked_supported(*shape)) return 0;
  return chunked_workspace_bytes(*shape);
}

sdm_status sdm_recurrent_chunked(const sdm_shape* S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                                 const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                                 float* o, void* ws, size_t ws_bytes, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!chunked_supported(*S)) return SDM_ERR_UNSUPPORTED;
  const void* ptrs[] = {widx, wgt, ridx, rgt, v, alpha, beta, M, o};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return SDM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < chunked_workspace_bytes(*S)) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_INVALID_ARG;
  const size_t mb = (size_t)S->B * S->H * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  const size_t ob = tensor_bytes(*S, S->d_v, 4);
  const size_t wb = tensor_bytes(*S, S->W, 4), rb = tensor_bytes(*S, S->R, 4), sb = tensor_bytes(*S, 1, 4);
  const size_t vb = tensor_bytes(*S, S->d_v, dtype_size(S->in_dtype));
  const void* outs[] = {M, o, ws};
  const size_t osz[] = {mb, ob, ws_bytes};
  const void* ins[] = {widx, wgt, ridx, rgt, v, alpha, beta};
  const size_t isz[] = {wb, wb, rb, rb, vb, sb, sb};
  for (int i = 0; i < 3; ++i) {
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], osz[i], outs[j], osz[j])) return SDM_ERR_INVALID_ARG;
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return SDM_ERR_INVALID_ARG;
  }
  if (S->T == 0) return SDM_OK;
  return hip_status(launch_chunked(*S, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, (hipStream_t)stream));
}

size_t sdm_backward_workspace_bytes(const sdm_shape* shape) {
  if (check_shape(shape, true) != SDM_OK) return 0;
  return backward_workspace_bytes(*shape);
}

sdm_status sdm_recurrent_backward(const sdm_shape* S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                                  const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                                  const void* xlog, const float* go, float* G, float* dv, float* dalpha, float* dbeta,
                                  float* dwgt, float* drgt, void* ws, size_t ws_bytes, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  const void* ptrs[] = {widx, wgt, ridx, rgt, v, alpha, beta, M, xlog, go, G, dv, dalpha, dbeta, dwgt, drgt};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return SDM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < backward_workspace_bytes(*S)) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_INVALID_ARG;
  const size_t U = (size_t)S->B * S->H;
  // per-unit row traffic uses byte offsets below 2^31, with a sentinel past every table
  if ((size_t)S->N * S->d_v * 4 >= 0x7FFFFFF0ull || (size_t)S->T * S->d_v * 4 >= 0x7FFFFFF0ull ||
      (size_t)S->T * S->W * S->d_v * dtype_size(S->mem_dtype) >= 0x7FFFFFF0ull)
    return SDM_ERR_INVALID_ARG;
  const size_t mb = U * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype), gb = U * (size_t)S->N * S->d_v * 4;
  const size_t lb = tensor_bytes(*S, (int64_t)S->W * S->d_v, dtype_size(S->mem_dtype));
  const size_t vb = tensor_bytes(*S, S->d_v, 4), sb = tensor_bytes(*S, 1, 4);
  const size_t wb = tensor_bytes(*S, S->W, 4), rb = tensor_bytes(*S, S->R, 4);
  // outputs (and the workspace) apart from each other and from every input
  const void* outs[] = {M, G, dv, dalpha, dbeta, dwgt, drgt, ws};
  const size_t osz[] = {mb, gb, vb, sb, sb, wb, rb, ws_bytes};
  const void* ins[] = {widx, wgt, ridx, rgt, v, alpha, beta, xlog, go};
  const size_t isz[] = {wb, wb, rb, rb, tensor_bytes(*S, S->d_v, dtype_size(S->in_dtype)), sb, sb, lb, vb};
  for (int i = 0; i < 8; ++i) {
    for (int j = i + 1; j < 8; ++j)
      if (overlaps(outs[i], osz[i], outs[j], osz[j])) return SDM_ERR_INVALID_ARG;
    for (int j = 0; j < 9; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return SDM_ERR_INVALID_ARG;
  }
  if (S->T == 0) return SDM_OK;
  return hip_status(launch_backward(*S, widx, wgt, ridx, rgt, v, alpha, beta, M, xlog, go, G, dv, dalpha, dbeta,
                                    dwgt, drgt, ws, (hipStream_t)stream));
}

size_t sdm_workspace_bytes_decay(const sdm_shape* shape) {
  if (check_shape(shape, true) != SDM_OK) return 0;
  return workspace_layout(*shape, true).total;
}

sdm_status sdm_decay_state_init(const sdm_shape* S, double* lam, double* lrun, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!lam || !lrun || !aligned16(lam) || !aligned16(lrun)) return SDM_ERR_INVALID_ARG;
  const size_t U = (size_t)S->B * S->H;
  if (overlaps(lam, U * (size_t)S->N * 8, lrun, U * 8)) return SDM_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (launch_zero(lam, U * (size_t)S->N, hs) != hipSuccess) return SDM_ERR_HIP;
  return hip_status(launch_zero(lrun, U, hs));
}

sdm_status sdm_recurrent_decay(const sdm_shape* S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                               const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                               double* lam, double* lrun, float* o, void* ws, size_t ws_bytes, void* stream) {
  if (!lam || !lrun) return SDM_ERR_INVALID_ARG;
  return recurrent_impl(S, widx, wgt, ridx, rgt, v, alpha, beta, M, lam, lrun, o, ws, ws_bytes, stream);
}

sdm_status sdm_forward_decay(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const void* subkeys, void* M, double* lam, double* lrun, float* o,
                             int32_t* widx_out, int32_t* ridx_out, void* ws, size_t ws_bytes, void* stream) {
  if (!lam || !lrun) return SDM_ERR_INVALID_ARG;
  return forward_impl(S, q, k, v, alpha, beta, subkeys, M, lam, lrun, o, widx_out, ridx_out, ws, ws_bytes, stream);
}

sdm_status sdm_decode_step_decay(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, const void* subkeys, void* M, double* lam, double* lrun, float* o,
                                 void* stream) {
  if (!lam || !lrun) return SDM_ERR_INVALID_ARG;
  return decode_impl(S, q, k, v, alpha, beta, subkeys, M, lam, lrun, o, stream);
}

sdm_status sdm_materialize(const sdm_shape* S, const void* M, const double* lam, const double* lrun, float* out,
                           void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!M || !lam || !lrun || !out) return SDM_ERR_INVALID_ARG;
  if (!aligned16(M) || !aligned16(lam) || !aligned16(lrun) || !aligned16(out)) return SDM_ERR_INVALID_ARG;
  const size_t U = (size_t)S->B * S->H;
  const size_t mb = U * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  const size_t outb = U * (size_t)S->N * S->d_v * 4;
  if (overlaps(out, outb, M, mb) || overlaps(out, outb, lam, U * (size_t)S->N * 8) || overlaps(out, outb, lrun, U * 8))
    return SDM_ERR_INVALID_ARG;
  return hip_status(launch_materialize(*S, M, lam, lrun, out, (hipStream_t)stream));
}

sdm_status sdm_gates(const sdm_shape* S, const float* a, const float* b, const float* A_log, const float* dt_bias,
                     float* alpha, float* beta, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  const void* ptrs[] = {a, b, A_log, dt_bias, alpha, beta};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return SDM_ERR_INVALID_ARG;
  const size_t gb = tensor_bytes(*S, 1, 4), hb = (size_t)S->H * 4;
  const void* ins[] = {a, b};
  for (const void* p : ins)
    if (overlaps(p, gb, alpha, gb) || overlaps(p, gb, beta, gb)) return SDM_ERR_INVALID_ARG;
  if (overlaps(alpha, gb, beta, gb) || overlaps(A_log, hb, alpha, gb) || overlaps(A_log, hb, beta, gb) ||
      overlaps(dt_bias, hb, alpha, gb) || overlaps(dt_bias, hb, beta, gb))
    return SDM_ERR_INVALID_ARG;
  if (S->T == 0) return SDM_OK;
  return hip_status(launch_gates(*S, a, b, A_log, dt_bias, alpha, beta, (hipStream_t)stream));
}

sdm_status sdm_output_gate(const sdm_shape* S, const float* o, const void* z, const float* w, float eps, void* x,
                           void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!o || !z || !w || !x || !aligned16(o) || !aligned16(z) || !aligned16(w) || !aligned16(x))
    return SDM_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || eps > 1.f) return SDM_ERR_INVALID_ARG;
  // grid: one thread per 8 values (at most 2^32 threads)
  if ((int64_t)S->B * S->H * S->T * S->d_v > ((int64_t)1 << 34)) return SDM_ERR_UNSUPPORTED;
  const size_t ob = tensor_bytes(*S, S->d_v, 4), zb = tensor_bytes(*S, S->d_v, dtype_size(S->in_dtype));
  const size_t xb = tensor_bytes(*S, S->d_v, 2);
  if (overlaps(x, xb, o, ob) || overlaps(x, xb, z, zb) || overlaps(x, xb, w, (size_t)S->d_v * 4))
    return SDM_ERR_INVALID_ARG;
  if (S->T == 0) return SDM_OK;
  return hip_status(launch_output_gate(*S, o, z, w, eps, (uint16_t*)x, (hipStream_t)stream));
}

sdm_status sdm_head_mix(const void* x, const void* Wo, float* y, int64_t M, int32_t K, int32_t N, void* stream) {
  if (M < 0 || K < 32 || K % 32 != 0 || N < 1) return SDM_ERR_INVALID_ARG;
  // grid: ceil(M/128) workgroups of 256 threads along x stay below 2^32 threads
  if (M > ((int64_t)1 << 30) || K > (1 << 20) || N > (1 << 22)) return SDM_ERR_UNSUPPORTED;
  if (!x || !Wo || !y || !aligned16(x) || !aligned16(Wo) || !aligned16(y)) return SDM_ERR_INVALID_ARG;
  const size_t xb = (size_t)M * K * 2, wb = (size_t)N * K * 2, yb = (size_t)M * N * 4;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, Wo, wb)) return SDM_ERR_INVALID_ARG;
  if (M == 0) return SDM_OK;
  return hip_status(launch_head_mix((const uint16_t*)x, (const uint16_t*)Wo, y, (long long)M, K, N, (hipStream_t)stream));
}

sdm_status sdm_output_project(const sdm_shape* S, const float* o, const void* z, const float* w, float eps,
                              const void* Wo, int32_t d_model, float* y, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!o || !z || !w || !Wo || !y || !aligned16(o) || !aligned16(z) || !aligned16(w) || !aligned16(Wo) ||
      !aligned16(y))
    return SDM_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || eps > 1.f || d_model < 1) return SDM_ERR_INVALID_ARG;
  if (!output_project_supported(S->d_v, S->H) || d_model > (1 << 22)) return SDM_ERR_UNSUPPORTED;
  // row bases of o and z are 32-bit token-head counts
  if ((int64_t)S->B * S->H * S->T > (int64_t)INT32_MAX - S->H * (int64_t)S->T) return SDM_ERR_UNSUPPORTED;
  if ((int64_t)S->B * S->T > ((int64_t)1 << 27)) return SDM_ERR_UNSUPPORTED;  // grid of 32-token workgroups
  const size_t ob = tensor_bytes(*S, S->d_v, 4), zb = tensor_bytes(*S, S->d_v, dtype_size(S->in_dtype));
  const size_t wob = (size_t)d_model * S->H * S->d_v * 2, yb = (size_t)S->B * S->T * d_model * 4;
  if (overlaps(y, yb, o, ob) || overlaps(y, yb, z, zb) || overlaps(y, yb, w, (size_t)S->d_v * 4) ||
      overlaps(y, yb, Wo, wob))
    return SDM_ERR_INVALID_ARG;
  if (S->T == 0) return SDM_OK;
  return hip_status(
      launch_output_project(*S, o, z, w, eps, (const uint16_t*)Wo, d_model, y, (hipStream_t)stream));
}

sdm_status sdm_workspace_error(const void* ws, size_t ws_bytes, int64_t* host_count, void* stream) {
  if (!ws || !host_count || ws_bytes < 8 || !aligned16(ws)) return SDM_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  uint64_t v = 0;
  if (hipMemcpyAsync(&v, ws, 8, hipMemcpyDeviceToHost, hs) != hipSuccess) return SDM_ERR_HIP;
  if (hipStreamSynchronize(hs) != hipSuccess) return SDM_ERR_HIP;
  *host_count = (int64_t)v;
  return SDM_OK;
}

}  // extern "C"
