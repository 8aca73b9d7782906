/*
 * sdm.h -- C ABI of the Sparse Delta Memory (SDM) layer forward on AMD Instinct MI355X
 * (gfx950).
 *
 * The method: a Gated DeltaNet whose dense key-value state is replaced by an N-slot table
 * per head that starts from a learned M0. For each token, product-key addressing picks W
 * write slots from the key and R read slots from the query (softmax weights); a gated
 * delta write updates only the W write slots, and a weighted read of the R read slots
 * gives the token's output.
 *
 * Sources ("PL" = the paperlayer.ai summary of arXiv:2607.07386v1, "Sparse Delta Memory:
 * Scaling the State of Linear RNNs through Sparsity"; "Atlas" = the atlas.scime.ai
 * summary of the same paper):
 *   PL §2 "Gated DeltaNet" and "Product Key Memory"; PL §3 "Sparse memory updates",
 *   "Sparse addressing", "Sparse retrieval", "Learned initial state"; PL §4 "SDM
 *   Configuration" (softmax-normalised activations); Atlas "Approach" (product-key top-k).
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer to a contiguous, row-major buffer owned by
 *     the caller; the library never frees or keeps it. Pointers must be 16-byte aligned.
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream). Each call only
 *     enqueues work on that stream and returns; results are ready when the stream is.
 *   - Arguments are validated on the host before any HIP call. A failed validation returns
 *     a negative sdm_status and enqueues nothing, so every argument error can be observed
 *     without a GPU. Launch failures return SDM_ERR_HIP.
 *   - Calls keep no state between them; calls on different streams with disjoint outputs
 *     may run concurrently.
 *   - Units: a unit is one (batch b, head h) pair; unit u = b*H + h. Units are independent.
 *
 * Dtypes: q, k, v and the sub-keys share `in_dtype` (SDM_F32 or SDM_BF16); M0 and the
 * table share `mem_dtype`. Gates alpha, beta, weights and the output o are float32.
 */
#ifndef SDM_H_
#define SDM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDM_ABI_VERSION 1

typedef enum {
  SDM_OK = 0,
  SDM_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned or aliasing buffers   */
  SDM_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement (see limits) */
  SDM_ERR_WORKSPACE = -3,   /* workspace missing or smaller than sdm_workspace_bytes()   */
  SDM_ERR_HIP = -4,         /* a HIP launch or runtime call failed                       */
  SDM_ERR_INTERNAL = -5
} sdm_status;

typedef enum { SDM_F32 = 0, SDM_BF16 = 1 } sdm_dtype;

/* Problem shape. Limits checked by every call (SDM_ERR_INVALID_ARG for a malformed shape,
 * SDM_ERR_UNSUPPORTED for a valid one past what the kernels implement):
 *   B, H >= 1; T >= 1 (T may be 0 only where stated); B*T <= 2^30 - 1; B*H <= 65535*64;
 *   N = s*s a perfect square with 4 <= N <= 262144 (s <= 512); d_k even, 2 <= d_k <= 256;
 *   d_v >= 1 with a table row of d_v*sizeof(mem) bytes a multiple of 16 and at most 1024
 *   (d_v <= 256 for a float32 table, <= 512 for bf16); 1 <= kappa <= min(s, 64);
 *   1 <= W, R <= min(kappa*kappa, 64). Some entry points narrow these further (stated at
 *   each). */
typedef struct {
  int32_t B, H, T;      /* batch, heads, tokens in this call                            */
  int64_t N;            /* slots per head (perfect square; s = sqrt(N) sub-keys/half)   */
  int32_t d_k, d_v;     /* key/query width (two halves of d_k/2), value width           */
  int32_t kappa;        /* sub-keys kept per half before the kappa x kappa merge        */
  int32_t W, R;         /* write slots per token (from k), read slots per token (from q)*/
  int32_t in_dtype;     /* sdm_dtype of q, k, v, sub-keys                               */
  int32_t mem_dtype;    /* sdm_dtype of M0 and the table                                */
} sdm_shape;

/* Human-readable name of a status code (static string). */
const char* sdm_status_string(int status);

/* SDM_ABI_VERSION of the loaded library. */
int sdm_abi_version(void);

/* Checks a shape against the limits above without touching any buffer: SDM_OK or the
 * error code any call would return for it. */
sdm_status sdm_check_shape(const sdm_shape* shape);

/* Bytes of workspace sdm_forward (and sdm_recurrent) need for this shape: the per-token
 * slot lists and weights, the token dependency lists and the scheduler's counters. 0 if
 * the shape is invalid. */
size_t sdm_workspace_bytes(const sdm_shape* shape);

/* M0 copy-on-init (PL §3 "Learned initial state": the table starts from M0).
 *   M0 [H, N, d_v] mem_dtype (read); M [B, H, N, d_v] mem_dtype (written): M[b,h] = M0[h]
 *   bit for bit, for every b. M must not overlap M0. */
sdm_status sdm_init_from_M0(const sdm_shape* shape, const void* M0, void* M, void* stream);

/* Product-key addressing of every token (PL §2 "Product Key Memory", PL §3 "Sparse
 * addressing", PL §4 softmax activations, Atlas "Approach").
 *   x       [B, H, T, d_k] in_dtype: keys (for write slots) or queries (for read slots)
 *   subkeys [H, 2, s, d_k/2] in_dtype: half p of x is scored against subkeys[h, p]
 *   n_sel   slots to select per token (W for keys, R for queries), 1..min(kappa^2, 64)
 *   idx     [B, H, T, n_sel] int32 out: slot n = i*s + j, in rank order
 *   weight  [B, H, T, n_sel] float32 out: softmax of the selected scores
 *   score   [B, H, T, n_sel] float32 out, may be NULL: the selected scores
 * Per half the kappa best sub-keys are kept, the kappa*kappa sums are ranked, and the
 * first n_sel are returned. Every ranking orders by float32 score descending, then by
 * index ascending. Scores are float32 sums of exact products (bf16) or float32 products;
 * where two slots' exact scores agree to within float32 rounding, the order between them
 * can differ from an exact-arithmetic ranking (the two are then an equally good choice). */
sdm_status sdm_address(const sdm_shape* shape, const void* x, const void* subkeys, int32_t n_sel,
                       int32_t* idx, float* weight, float* score, void* stream);

/* sdm_address that also carries out slice `part` of `nparts` of sdm_init_from_M0 in the
 * same kernel launch (PL §3 "Learned initial state"; the addressing is bound by its vector
 * ALU and leaves the memory pipe idle, so the copy rides on it). The initialisation is split
 * into nparts equal ranges of the 16-byte chunks of one head-major copy of M0; once calls
 * with part = 0 .. nparts-1 have all completed, M[b,h] = M0[h] bit for bit for every b,
 * exactly as after sdm_init_from_M0. idx, weight and score are those of sdm_address bit for
 * bit. With B*T = 0 only the copy slice runs.
 *   M0 [H, N, d_v] mem_dtype (read); M [B, H, N, d_v] mem_dtype (written, this slice only)
 *   1 <= nparts <= 64 and 0 <= part < nparts, else SDM_ERR_INVALID_ARG. M must be 16-byte
 *   aligned and overlap none of M0, x, subkeys, idx, weight, score (SDM_ERR_INVALID_ARG);
 *   every other argument and error as for sdm_address. */
sdm_status sdm_address_init(const sdm_shape* shape, const void* x, const void* subkeys, int32_t n_sel,
                            int32_t* idx, float* weight, float* score, const void* M0, void* M,
                            int32_t part, int32_t nparts, void* stream);

/* The sparse gated-delta recurrence with caller-supplied slots and weights (PL §2 "Gated
 * DeltaNet", PL §3 "Sparse memory updates" / "Sparse retrieval"). For each unit, tokens
 * t = 0..T-1 in order:
 *   rho   = alpha_t * sum_j wgt_j * M[widx_j]
 *   delta = beta_t * (v_t - rho)
 *   M[widx_j] = round_mem(alpha_t * M[widx_j] + wgt_j * delta)      (only these W rows)
 *   o_t   = sum_r rgt_r * M[ridx_r]                                  (after the write)
 * with float32 arithmetic and one rounding to mem_dtype per written value.
 *   widx [B,H,T,W] int32, wgt [B,H,T,W] f32, ridx [B,H,T,R] int32, rgt [B,H,T,R] f32
 *   v [B,H,T,d_v] in_dtype, alpha/beta [B,H,T] f32, M [B,H,N,d_v] in/out, o [B,H,T,d_v] out
 * The W slots of one token must be distinct. A slot index outside [0, N) is skipped (its
 * weight contributes nothing and no row is touched) and counted in the workspace's error
 * word (sdm_workspace_error). ws: at least sdm_workspace_bytes(shape) bytes. */
sdm_status sdm_recurrent(const sdm_shape* shape, const int32_t* widx, const float* wgt, const int32_t* ridx,
                         const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                         void* ws, size_t ws_bytes, void* stream);

/* One SDM layer forward over a [B, H, T] token block: addressing of k (W write slots) and
 * q (R read slots) followed by the recurrence above (for a float32 table with at least 32
 * units, by its chunkwise two-phase form, which agrees with it up to float32 summation order;
 * see sdm_forward_uses_chunkwise), continuing from the table in M (call
 * sdm_init_from_M0 first for a fresh sequence; calling again with the carried M continues
 * the sequence).
 *   q, k [B,H,T,d_k] in_dtype; v [B,H,T,d_v] in_dtype; alpha, beta [B,H,T] f32
 *   subkeys [H,2,s,d_k/2] in_dtype; M [B,H,N,d_v] mem_dtype in/out; o [B,H,T,d_v] f32 out
 *   widx_out [B,H,T,W] int32 and ridx_out [B,H,T,R] int32: optional (NULL) copies of the
 *   selected slots, in rank order.
 * ws: at least sdm_workspace_bytes(shape) bytes of device memory. */
sdm_status sdm_forward(const sdm_shape* shape, const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const void* subkeys, void* M, float* o, int32_t* widx_out,
                       int32_t* ridx_out, void* ws, size_t ws_bytes, void* stream);

/* Largest workspace sdm_forward_static can use: its library-owned device array (bytes). */
#define SDM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* sdm_forward without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops and harnesses that forbid allocation. The
 * slot lists, weights, dependency words and error word that sdm_forward keeps in `ws` live
 * in a library-owned device array of SDM_STATIC_SCRATCH_BYTES, one per GPU, whose address
 * is looked up the first time the call runs on that GPU and which stays until the process
 * ends. Arguments, layouts and results are those of sdm_forward (bit for bit).
 * Errors: those of sdm_forward; SDM_ERR_WORKSPACE, with nothing enqueued, when
 * sdm_workspace_bytes(shape) exceeds SDM_STATIC_SCRATCH_BYTES; SDM_ERR_HIP if the array's
 * address cannot be obtained. The call allocates nothing.
 * Every call on one GPU shares that GPU's array and leaves the last call's contents there:
 * calls that overlap in time on one GPU (other streams, other host threads) race and give
 * undefined results; calls ordered on one stream are safe. The recurrence's error word is
 * not exposed to the caller (the forward's own addressing never produces a slot outside
 * [0, N)). */
sdm_status sdm_forward_static(const sdm_shape* shape, const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const void* subkeys, void* M, float* o, int32_t* widx_out,
                              int32_t* ridx_out, void* stream);

/* Which form of the recurrence sdm_forward (and sdm_forward_static) runs for this shape:
 * 0 = the pipelined token-by-token recurrence (the result of sdm_recurrent), 1 = the
 * chunkwise two-phase form of sdm_recurrent_chunked, -1 = invalid shape. The chunkwise form
 * is taken for a float32 table with at least 32 units (B*H), where it agrees with the token
 * rule up to float32 summation order and was measured faster. That order can differ from run
 * to run (its first phase accumulates couplings with LDS float atomics), so with the
 * chunkwise form results and the state carried across calls agree up to float32 summation
 * order rather than bit for bit; the pipeline is deterministic. */
int sdm_forward_uses_chunkwise(const sdm_shape* shape);

/* One decode step: T must be 1. The rule of sdm_forward with T = 1 (the same slots; sums
 * equal up to the order of the float32 additions), fused into one kernel launch on `stream`
 * and nothing else (no allocation, no memory fill), so a sequence of steps may be captured
 * into a HIP graph and replayed; needs no workspace.
 *   q, k [B,H,1,d_k]; v [B,H,1,d_v]; alpha, beta [B,H,1]; M in/out; o [B,H,1,d_v] f32. */
sdm_status sdm_decode_step(const sdm_shape* shape, const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const void* subkeys, void* M, float* o, void* stream);

/* Copies the workspace's error word (number of out-of-range slot indices met by the last
 * sdm_recurrent on this workspace) to *host_count after synchronising `stream`. */
sdm_status sdm_workspace_error(const void* ws, size_t ws_bytes, int64_t* host_count, void* stream);

/* ---------------------------------------------------------------------------------------
 * Chunkwise two-phase form of the recurrence (PL App. A.1 "Phase 1" / "Phase 2", App. A.2:
 * inside a chunk of 64 tokens every quantity is the chunk-start table plus a combination of
 * the chunk's write residuals). Phase 1, in parallel over all chunks, forms from slots,
 * weights and gates alone each occurrence's decay coefficients and the tokens' couplings over
 * shared slots (kept as sparse row-sorted lists); Phase 2, chunk after chunk, gathers the
 * chunk's rows, solves the unit lower-triangular system for the residuals by a forward sweep
 * over those lists, forms the outputs and writes each written row back once.
 * --------------------------------------------------------------------------------------- */

/* Bytes of device memory sdm_recurrent_chunked needs as workspace (0 for a shape it does not
 * take: W or R above 32, a table of 2^31 - 16 bytes or more per (batch, head), or an invalid
 * shape). About 90 KB per 64 tokens per (batch, head) at W = R = 32. */
size_t sdm_workspace_bytes_chunked(const sdm_shape* shape);

/* The recurrence of sdm_recurrent (written-rows rule), computed chunk by chunk: same
 * arguments, layouts and stream semantics (the call is asynchronous on `stream`; M is read
 * and updated in place; o [B,H,T,d_v] float32 is written), same o and final table up to
 * float32 summation order, except that written rows are rounded to mem_dtype once per chunk
 * (when written back) instead of at every write. Each token's W write slots must be distinct
 * (the addressing produces them so); a slot outside [0, N) touches nothing.
 * W, R <= 32; ws: at least sdm_workspace_bytes_chunked(shape) bytes, 16-byte aligned, owned by
 * the caller and not shared with a call that may run concurrently.
 * Errors (nothing is launched): SDM_ERR_INVALID_ARG for a bad shape, a null or misaligned
 * pointer, or outputs (M, o, ws) that overlap each other or an input; SDM_ERR_UNSUPPORTED
 * for W or R above 32 or a table too large for 32-bit row offsets; SDM_ERR_WORKSPACE for a
 * missing or short workspace; SDM_ERR_HIP if a launch fails. */
sdm_status sdm_recurrent_chunked(const sdm_shape* shape, const int32_t* widx, const float* wgt, const int32_t* ridx,
                                 const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                                 float* o, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Memory-efficient backward of the recurrence (PL App. A.3: the forward's sparse updates
 * are undone in place during the backward, so memory stays O(N d + T W d)).
 * --------------------------------------------------------------------------------------- */

/* sdm_recurrent that also logs, for the backward, the pre-update value of every written row
 * as its token read it: xlog [B,H,T,W,d_v] mem_dtype out (rows of slots outside [0, N) are
 * 0). T*W*d_v*sizeof(mem) must stay below 2^31 bytes per unit. Written-rows rule only; any W,
 * R that sdm_recurrent takes (shapes the pipelined path does not take log on the sequential
 * path). */
sdm_status sdm_recurrent_log(const sdm_shape* shape, const int32_t* widx, const float* wgt, const int32_t* ridx,
                             const float* rgt, const void* v, const float* alpha, const float* beta, void* M, float* o,
                             void* xlog, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device memory sdm_recurrent_backward needs as workspace (0 for an invalid shape):
 * per token a dependency mask, a store mask and the read-write coupling tables (W + R floats),
 * and the error word at offset 0 (sdm_workspace_error reads it). */
size_t sdm_backward_workspace_bytes(const sdm_shape* shape);

/* Gradients of L = sum <go, o> + <G_in, M_T> through the recurrence of sdm_recurrent_log,
 * walking the tokens in reverse (for token t, x_j = xlog[t, j], s = sum_j wgt_j x_j,
 * rho = alpha_t s, delta = beta_t (v_t - rho), G the gradient of the current table):
 *   drgt_r = <go_t, M[ridx_r]>;  G[ridx_r] += rgt_r go_t
 *   dy_j = G[widx_j];  dd = sum_j wgt_j dy_j;  dv_t = beta_t dd;  drho = -beta_t dd
 *   dwgt_j = <dy_j, delta> + alpha_t <drho, x_j>
 *   dalpha_t = sum_j <dy_j, x_j> + <drho, s>;  dbeta_t = <dd, v_t - rho>
 *   G[widx_j] = alpha_t dy_j + alpha_t wgt_j drho;  M[widx_j] = x_j  (undo)
 * The rounding of written rows to mem_dtype is passed through (straight-through).
 *   M [B,H,N,d_v] mem_dtype: the table after the forward in, M0 out (restored in place)
 *   G [B,H,N,d_v] f32: gradient of the final table in (zeros if none), of M0 out
 *   go, dv [B,H,T,d_v] f32; dalpha, dbeta [B,H,T] f32; dwgt [B,H,T,W], drgt [B,H,T,R] f32
 * Other arguments as for sdm_recurrent; W, R <= 64; read slots may repeat and may equal the
 * token's write slots; a slot outside [0, N) touches nothing and gets zero gradients.
 * Per unit, N*d_v*4, T*d_v*4 and T*W*d_v*sizeof(mem) bytes must each stay below 2^31 - 16.
 * ws: at least sdm_backward_workspace_bytes(shape) bytes, apart from every other buffer; its
 * error word counts workgroups that gave up waiting (about 3.6 s; the result is then
 * invalid). Floating-point sums over columns are added with atomics: the summation order of
 * dwgt, drgt, dalpha and dbeta can differ from run to run. */
sdm_status sdm_recurrent_backward(const sdm_shape* shape, const int32_t* widx, const float* wgt, const int32_t* ridx,
                                  const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                                  const void* xlog, const float* go, float* G, float* dv, float* dalpha, float* dbeta,
                                  float* dwgt, float* drgt, void* ws, size_t ws_bytes, void* stream);

/* Gradients through the addressing (PL §4 "SDM Configuration": softmax over the selected
 * scores; PL §2 "Product Key Memory": slot n = i*s + j scores x[:h].C1[i] + x[h:].C2[j] with
 * h = d_k/2, C1 = subkeys[h,0], C2 = subkeys[h,1]), the selected slots held fixed:
 *   dscore_k = weight_k (dweight_k - sum_l weight_l dweight_l)
 *   dx[:h] = sum_k dscore_k C1[i_k];  dx[h:] = sum_k dscore_k C2[j_k]
 *   dsub[h,0,i] += sum over tokens and k with i_k = i of dscore_k x[:h]; dsub[h,1,j] likewise
 *   x [B,H,T,d_k] in_dtype (k for the write slots, q for the read slots); subkeys as for
 *   sdm_address; idx, weight [B,H,T,n_sel] as sdm_address returns them; dweight
 *   [B,H,T,n_sel] f32 (dwgt or drgt of sdm_recurrent_backward); dx [B,H,T,d_k] f32 out;
 *   dsub [H,2,s,d_k/2] f32 in/out: the sub-key gradient is added to it (zero it once, then
 *   call for k and for q). A slot outside [0, N) adds nothing. Float32 sums; the order of
 *   the additions into dsub can differ from run to run. */
sdm_status sdm_address_backward(const sdm_shape* shape, const void* x, const void* subkeys, int32_t n_sel,
                                const int32_t* idx, const float* weight, const float* dweight, float* dx,
                                float* dsub, void* stream);

/* ---------------------------------------------------------------------------------------
 * The steps on either side of the recurrence (PL App. B "Gate dynamics": forget gate
 * exp(g), input gate sigma(b); PL §4 "SDM Configuration": gate and time-step bias as in
 * Gated DeltaNet; PL §3 "Sparse retrieval": the read is RMS-normalised, elementwise gated
 * and projected into the layer output).
 * --------------------------------------------------------------------------------------- */

/* Gates from their per token-head pre-activations a, b [B,H,T] f32 and per-head parameters
 * A_log, dt_bias [H] f32:  alpha = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])) in (0, 1],
 * beta = sigmoid(b); alpha, beta [B,H,T] f32 out (float32 arithmetic). */
sdm_status sdm_gates(const sdm_shape* shape, const float* a, const float* b, const float* A_log, const float* dt_bias,
                     float* alpha, float* beta, void* stream);

/* Normalised, gated output of every token-head:
 *   x[b,t,h,:] = o[b,h,t,:] / sqrt(mean(o[b,h,t,:]^2) + eps) * w * silu(z[b,t,h,:])
 * o [B,H,T,d_v] f32 (the recurrence's output); z [B,T,H,d_v] in_dtype (the gate's
 * pre-activation, token-major); w [d_v] f32 shared by the heads; x [B,T,H,d_v] bf16 out
 * (token-major: row b*T + t of x is the concatenation of the heads, the input of
 * sdm_head_mix). 0 <= eps <= 1. */
sdm_status sdm_output_gate(const sdm_shape* shape, const float* o, const void* z, const float* w, float eps, void* x,
                           void* stream);

/* Mixing of the heads into the layer output: y = x . Wo^T, i.e. y[m, n] = sum_k x[m,k] Wo[n,k]
 *   x [M, K] bf16 (K = H*d_v, rows from sdm_output_gate), Wo [N, K] bf16 (d_model = N
 *   rows), y [M, N] f32 out. K a multiple of 32; bf16 products, float32 sums (MFMA). */
sdm_status sdm_head_mix(const void* x, const void* Wo, float* y, int64_t M, int32_t K, int32_t N, void* stream);

/* The two calls above in one pass, without the bf16 x in memory (PL §3 "Sparse retrieval":
 * RMS-normalised, elementwise gated, projected into the layer output):
 *   y[b*T + t, n] = sum_h sum_c x[b,t,h,c] Wo[n, h*d_v + c]
 * with x[b,t,h,:] = bf16(o[b,h,t,:] / sqrt(mean(o[b,h,t,:]^2) + eps) * w * silu(z[b,t,h,:])),
 * bit for bit the x that sdm_output_gate stores (both sum the squares in the same order). o [B,H,T,d_v] f32; z [B,T,H,d_v] in_dtype; w [d_v] f32; Wo [d_model, H*d_v] bf16;
 * y [B*T, d_model] f32 out, which may not overlap the inputs. d_v one of 32, 64, 128, 256
 * and H*d_v <= 2552 (x of 32 tokens stays in one workgroup's LDS), B*T <= 2^27, else
 * SDM_ERR_UNSUPPORTED; 1 <= d_model <= 2^22; 0 <= eps <= 1; every pointer 16-byte aligned.
 * bf16 products, float32 sums (MFMA). */
sdm_status sdm_output_project(const sdm_shape* shape, const float* o, const void* z, const float* w, float eps,
                              const void* Wo, int32_t d_model, float* y, void* stream);

/* ---------------------------------------------------------------------------------------
 * Whole-table decay variant. The calls above decay only the W written rows by alpha_t. If
 * alpha_t instead decays every row of the table, as the dense state of Gated DeltaNet
 * decays (PL §2 "Gated DeltaNet"; PL §3 "Connection to GDN": the rule is then Gated
 * DeltaNet's with the sparse key sum_j wgt_j e_{widx_j}), the calls below apply that decay
 * lazily and never touch a row no token addresses. Beside the table the state holds
 *   lam  [B,H,N] float64: the cumulative log-decay (sum of log alpha) at each slot's last
 *        write; a row's current value is its stored value times exp(lrun - lam)
 *   lrun [B,H]   float64: the cumulative log-decay of all tokens so far
 * Stored rows are rounded to mem_dtype when written; an untouched row's value is its
 * stored value times the exact decay since (it is never stored again). A gate of 0 decays
 * fully (log alpha is floored at -1000). These calls take the pipelined recurrence only:
 * shapes it cannot take return SDM_ERR_UNSUPPORTED.
 * --------------------------------------------------------------------------------------- */

/* lam = 0 and lrun = 0: the state of a table fresh from sdm_init_from_M0. */
sdm_status sdm_decay_state_init(const sdm_shape* shape, double* lam, double* lrun, void* stream);

/* Workspace bytes of sdm_forward_decay / sdm_recurrent_decay: sdm_workspace_bytes plus the
 * per-token cumulative log-decay [B,H,T+1] float64, one factor per token-slot [B,H,T,W+R]
 * float32, the latest writer of each slot [B,H,N] int32 and, when few units leave compute
 * units idle, up to three more such int32 tables (one per extra token segment of the pass
 * that finds each access's latest writer). 0 if the shape is invalid. */
size_t sdm_workspace_bytes_decay(const sdm_shape* shape);

/* sdm_recurrent with whole-table decay: for each unit, tokens in order,
 *   x_j   = M[widx_j] * exp(L_{t-1} - lam[widx_j])        (the row's value before token t)
 *   rho   = alpha_t * sum_j wgt_j x_j ;  delta = beta_t * (v_t - rho)
 *   M[widx_j] = round_mem(alpha_t x_j + wgt_j delta) ;  lam[widx_j] = L_t
 *   o_t   = sum_r rgt_r * M[ridx_r] * exp(L_t - lam[ridx_r])
 * with L_t = lrun + sum_{s<=t} log alpha_s; lrun becomes L_{T-1}. lam, lrun in/out; other
 * arguments as for sdm_recurrent. ws: at least sdm_workspace_bytes_decay(shape) bytes. */
sdm_status sdm_recurrent_decay(const sdm_shape* shape, const int32_t* widx, const float* wgt, const int32_t* ridx,
                               const float* rgt, const void* v, const float* alpha, const float* beta, void* M,
                               double* lam, double* lrun, float* o, void* ws, size_t ws_bytes, void* stream);

/* sdm_forward with whole-table decay (addressing, then sdm_recurrent_decay's rule). */
sdm_status sdm_forward_decay(const sdm_shape* shape, const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const void* subkeys, void* M, double* lam, double* lrun, float* o,
                             int32_t* widx_out, int32_t* ridx_out, void* ws, size_t ws_bytes, void* stream);

/* sdm_decode_step with whole-table decay (T must be 1; needs no workspace). */
sdm_status sdm_decode_step_decay(const sdm_shape* shape, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const void* subkeys, void* M, double* lam,
                                 double* lrun, float* o, void* stream);

/* The current table of the whole-table decay variant: out[b,h,n,:] = M[b,h,n,:] *
 * exp(lrun[b,h] - lam[b,h,n]), float32 [B,H,N,d_v] (out must not overlap the state). */
sdm_status sdm_materialize(const sdm_shape* shape, const void* M, const double* lam, const double* lrun, float* out,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H_ */
