// Host-side declarations shared by the launch wrappers and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sdm.h"

namespace sdm {

inline int64_t isqrt64(int64_t n) {
  if (n <= 0) return 0;
  int64_t r = 0;
  while ((r + 1) * (r + 1) <= n) ++r;
  return r;
}
inline size_t dtype_size(int dt) { return dt == SDM_BF16 ? 2 : 4; }

// Workspace layout of sdm_forward / sdm_recurrent (all offsets 256-byte aligned).
struct WsLayout {
  size_t widx, wgt, ridx, rgt;  // per-token slot lists and weights (forward only)
  size_t err;                   // int64 error counter
  size_t deps;                  // dependency lists (dataflow scheduler)
  size_t sched;                 // scheduler counters and done flags
  size_t ltok, fac, lastw;      // whole-table decay: log-decay per token [U][T+1], factors [U][T][E],
                                // latest writer per slot [U][N]
  size_t segl;                  // whole-table decay: latest writer per token segment [U][nseg-1][N]
  size_t chunk;                 // chunkwise form's per-chunk lists (sdm_forward on float32 tables)
  size_t total;
};
WsLayout workspace_layout(const sdm_shape& S, bool decay = false);

// Whole-table decay state of the caller: lam [U][N] (cumulative log-decay at each slot's
// last write), lrun [U] (cumulative log-decay of every token so far).
struct DecayState {
  double* lam;
  double* lrun;
};

hipError_t launch_zero(void* p, size_t n_words, hipStream_t stream);
size_t address_lds_bytes(int s, int kappa);
// Slice `part` of `nparts` of the table initialisation M[b, h] = M0[h] (16-byte chunks of one
// head-major copy of M0, split into nparts equal ranges), carried out by an addressing call.
struct InitPart {
  const void* M0;
  void* M;
  int part, nparts;
};
hipError_t launch_address(const sdm_shape& S, const void* x, const void* subkeys, int n_sel, int32_t* idx,
                          float* weight, float* score, hipStream_t stream, const InitPart* init = nullptr);
hipError_t launch_init(const sdm_shape& S, const void* M0, void* M, hipStream_t stream);
// chunks [c0, c1) of the initialisation (of H*N*rowbytes/16 chunks per copy)
hipError_t launch_init_part(const sdm_shape& S, const void* M0, void* M, size_t c0, size_t c1, hipStream_t stream);
hipError_t launch_recurrent(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                            const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                            void* ws, const WsLayout& L, const DecayState* dk, hipStream_t stream,
                            void* xlog = nullptr);
hipError_t launch_decode(const sdm_shape& S, const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const void* subkeys, void* M, float* o, const DecayState* dk,
                         hipStream_t stream);
size_t decode_lds_bytes(const sdm_shape& S);

bool dataflow_supported(const sdm_shape& S, bool decay = false);
size_t dataflow_deps_bytes(const sdm_shape& S);
size_t dataflow_sched_words(const sdm_shape& S);
hipError_t launch_dataflow(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                           const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                           void* ws, const WsLayout& L, const DecayState* dk, void* xlog, hipStream_t stream);
int device_cus();  // compute units of the current device
size_t chunked_workspace_bytes(const sdm_shape& S);
bool chunked_supported(const sdm_shape& S);
hipError_t launch_chunked(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                          const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                          void* ws, hipStream_t stream);
hipError_t launch_address_backward(const sdm_shape& S, const void* x, const void* subkeys, int n_sel,
                                   const int32_t* idx, const float* w, const float* dw, float* dx, float* dsub,
                                   hipStream_t stream);
size_t backward_workspace_bytes(const sdm_shape& S);
hipError_t launch_backward(const sdm_shape& S, const int32_t* widx, const float* wgt, const int32_t* ridx,
                           const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                           const void* xlog, const float* go, float* G, float* dv, float* dalpha, float* dbeta,
                           float* dwgt, float* drgt, void* ws, hipStream_t stream);

hipError_t launch_log_decay_scan(const sdm_shape& S, const float* alpha, double* L, double* lrun, hipStream_t stream);
int decay_segments(const sdm_shape& S);  // token segments of the decay order pass
hipError_t launch_decay_pass(const sdm_shape& S, const uint32_t* pk, const double* L, double* lam, float* fac,
                             int* lastw, int* segl, int win, hipStream_t stream);
hipError_t launch_gates(const sdm_shape& S, const float* a, const float* b, const float* A_log, const float* dt_bias,
                        float* alpha, float* beta, hipStream_t stream);
hipError_t launch_output_gate(const sdm_shape& S, const float* o, const void* z, const float* w, float eps,
                              uint16_t* x, hipStream_t stream);
hipError_t launch_head_mix(const uint16_t* x, const uint16_t* Wo, float* y, long long M, int K, int N,
                           hipStream_t stream);
bool output_project_supported(int d_v, int H);  // d_v and K = H d_v the fused epilogue takes
hipError_t launch_output_project(const sdm_shape& S, const float* o, const void* z, const float* w, float eps,
                                 const uint16_t* Wo, int d_model, float* y, hipStream_t stream);
hipError_t launch_materialize(const sdm_shape& S, const void* M, const double* lam, const double* lrun, float* out,
                              hipStream_t stream);

}  // namespace sdm
