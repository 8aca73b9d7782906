// C ABI of the SDM layer forward: argument validation, workspace layout, launches.
// Every check runs on the host before the first HIP call, so argument errors never touch
// the GPU.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/sdm.h"
#include "sdm_internal.hpp"

namespace sdm {

namespace {

constexpr int64_t kMaxN = 262144;  // s <= 512: one half's scores of 32 tokens fit in LDS
constexpr int kMaxSel = 64;
constexpr size_t kAlign = 256;
constexpr size_t kMaxLds = 160 * 1024;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

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

}  // namespace

WsLayout workspace_layout(const sdm_shape& S) {
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
  if (dataflow_supported(S)) {
    o = align_up(o + dataflow_deps_bytes(S));
    L.sched = o;
    o = align_up(o + dataflow_sched_words(S) * 4);
  }
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

sdm_status sdm_address(const sdm_shape* S, const void* x, const void* subkeys, int32_t n_sel, int32_t* idx,
                       float* weight, float* score, void* stream) {
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
  if (S->T == 0) return SDM_OK;
  return hip_status(launch_address(*S, x, subkeys, n_sel, idx, weight, score, (hipStream_t)stream));
}

sdm_status sdm_recurrent(const sdm_shape* S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                         const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                         void* ws, size_t ws_bytes, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!widx || !wgt || !ridx || !rgt || !v || !alpha || !beta || !M || !o) return SDM_ERR_INVALID_ARG;
  const void* ptrs[] = {widx, wgt, ridx, rgt, v, alpha, beta, M, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDM_ERR_INVALID_ARG;
  const WsLayout L = workspace_layout(*S);
  if (!ws || ws_bytes < L.total) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_INVALID_ARG;
  const size_t mb = (size_t)S->B * S->H * (size_t)S->N * S->d_v * dtype_size(S->mem_dtype);
  const size_t ob = tensor_bytes(*S, S->d_v, 4);
  if (overlaps(M, mb, o, ob) || overlaps(M, mb, ws, ws_bytes) || overlaps(o, ob, ws, ws_bytes)) return SDM_ERR_INVALID_ARG;
  if (S->T == 0) return SDM_OK;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = launch_zero((char*)ws + L.err, 1, hs);
  if (e != hipSuccess) return SDM_ERR_HIP;
  return hip_status(launch_recurrent(*S, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, L, hs));
}

sdm_status sdm_forward(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const void* subkeys, void* M, float* o, int32_t* widx_out,
                       int32_t* ridx_out, void* ws, size_t ws_bytes, void* stream) {
  sdm_status st = check_shape(S, true);
  if (st != SDM_OK) return st;
  if (!q || !k || !v || !alpha || !beta || !subkeys || !M || !o) return SDM_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, alpha, beta, subkeys, M, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDM_ERR_INVALID_ARG;
  if ((widx_out && !aligned16(widx_out)) || (ridx_out && !aligned16(ridx_out))) return SDM_ERR_INVALID_ARG;
  const WsLayout L = workspace_layout(*S);
  if (!ws || ws_bytes < L.total) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_INVALID_ARG;
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
  if (S->T == 0) return SDM_OK;
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
  return hip_status(launch_recurrent(*S, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, L, hs));
}

sdm_status sdm_decode_step(const sdm_shape* S, const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const void* subkeys, void* M, float* o, void* stream) {
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
  return hip_status(launch_decode(*S, q, k, v, alpha, beta, subkeys, M, o, (hipStream_t)stream));
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
