/*
 * sslp.h -- C ABI of libsslp.so: the per-token sparse-routed gated delta-rule
 * recurrence on AMD MI355X (gfx950), as hand-written HIP kernels.
 *
 * Methods (all from public reading slides; citations name the slide):
 *   SDM  "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity"
 *   GDN/KDA  "Linear Attention Architectures: Mechanisms, Trade-offs, and
 *            Cross-Layer Routing"
 *   SSE  "Scaling Linear Attention with Sparse State Expansion"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer except the shape structs,
 *   which are host pointers read during the call.  The caller owns all
 *   memory (inputs, in/out states, outputs, workspace); the library never
 *   allocates, frees or synchronises.
 * - Each call validates its arguments on the host BEFORE any HIP call, then
 *   enqueues its kernels on `stream` (a hipStream_t passed as void*; NULL is
 *   the default stream) and returns (sslp_device_error alone synchronises).  Results are valid once the stream has
 *   completed.  States are updated in place in stream order.
 * - Tensors are dense, contiguous, row-major in the layouts written next to
 *   each argument; device pointers must be 16-byte aligned.  Inputs must not
 *   alias outputs unless stated.  Optional outputs may be NULL.
 * - dtype: SSLP_FP32 or SSLP_BF16.  It applies to score halves, q/k/v and the
 *   y/o outputs.  Gates (alpha, beta, lambda, logits), weights and states are
 *   always fp32.
 * - Values must be finite; behaviour on NaN/Inf inputs is unspecified.
 * - Calls on different streams may run concurrently if they touch disjoint
 *   memory.  The only global state is a thread-local last-error string.
 * - Return value: SSLP_OK or a negative status below; sslp_last_error()
 *   describes the last failure on the calling thread.
 */
#ifndef SSLP_H
#define SSLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSLP_VERSION 1

/* status codes */
#define SSLP_OK 0
#define SSLP_ERR_INVALID_ARG (-1) /* NULL required pointer, bad dimension, k > sqrtN, W > k^2, misalignment */
#define SSLP_ERR_UNSUPPORTED (-2) /* dimension outside what the kernels support */
#define SSLP_ERR_WORKSPACE (-3)   /* workspace NULL or smaller than the *_workspace_size() value */
#define SSLP_ERR_HIP (-4)         /* a HIP launch or runtime call failed */

/* dtype */
#define SSLP_FP32 0
#define SSLP_BF16 1

/* SDM residual form (slide "A v1 inconsistency matters for reproducing the update") */
#define SSLP_RESIDUAL_SHARED 0   /* figure form: v_hat = sum_n wt_n M~[i_n] shared by every slot (default) */
#define SSLP_RESIDUAL_PER_SLOT 1 /* Eq. (4) as printed: residual v - M~[i] per slot */

/* GDN/KDA decay granularity (slide "GDN and KDA change the granularity of forgetting") */
#define SSLP_DECAY_SCALAR 0  /* Gated DeltaNet: one alpha per (b,t,h) */
#define SSLP_DECAY_CHANNEL 1 /* Kimi Delta Attention: one alpha per (b,t,h,key channel) */

/* ------------------------------------------------------------------------ */
/* Sparse Delta Memory                                                       */
/* ------------------------------------------------------------------------ */

/*
 * SDM problem shape.  N = sqrtN * sqrtN slots per (sequence, head); slot of
 * the pair (a, b) is a*sqrtN + b with a indexing half 1.
 *   B, T, H  batch, tokens, heads (>= 1; T may be 0 for a no-op, in which case
 *            only M is required and the per-token pointers may be NULL)
 *   sqrtN    length of each score half, 1..1024
 *   d_v      value width, multiple of 4, <= 4096
 *   k_w, k_r per-half top-k for writes / reads, 1..min(sqrtN, 64)
 *   W, R     write / read budgets, 1..min(k^2, 128)
 */
typedef struct {
    int B, T, H, sqrtN, d_v, k_w, k_r, W, R;
} sslp_sdm_shape;

/* Bytes of device workspace sdm_forward / sdm_sparse_update need (0 on bad shape). */
size_t sdm_workspace_size(const sslp_sdm_shape* shape);

/*
 * sdm_forward -- product-key addressing for writes and reads, then the sparse
 * decay / delta update / read-after-write recurrence over T tokens.
 *
 * Slides: "Product keys select addresses without scoring every slot" (steps
 * 1-4: per-half top-k, k^2 candidate sums, top-W / top-R, softmax over the
 * selected scores) and "Selected slots decay and update; other slots
 * persist" Eqs. (3)-(5); residual per `residual_mode` (see above).
 * Per token t, head h:  M~[i] = alpha_t M[i] for i in I^w_t only;
 *   SHARED:   M[i_n] = M~[i_n] + beta_t wt_n (v_t - sum_m wt_m M~[i_m])
 *   PER_SLOT: M[i_n] = M~[i_n] + beta_t wt_n (v_t - M~[i_n])
 *   y_t = sum_m wt^r_m M[j_m]   (table after the write)
 * Rows outside I^w_t are never written.  Ranking is (fp32 score desc, index
 * asc) at both stages, the candidate score being the fp32 sum s1[a] + s2[b];
 * -0 and +0 tie.  Indices are returned in rank order.
 *
 *   sw1, sw2  [B,T,H,sqrtN] dtype  write-address score halves
 *   sr1, sr2  [B,T,H,sqrtN] dtype  read-address score halves (may alias sw1, sw2)
 *   v         [B,T,H,d_v]   dtype  values
 *   alpha     [B,T,H]       fp32   forget gate
 *   beta      [B,T,H]       fp32   input gate
 *   M         [B,H,N,d_v]   fp32   table, updated in place
 *   y         [B,T,H,d_v]   dtype  reads (out)
 *   idx_w, wt_w [B,T,H,W]   int32 / fp32  optional copies of the write addressing
 *   idx_r, wt_r [B,T,H,R]   int32 / fp32  optional copies of the read addressing
 *   workspace, ws_bytes     >= sdm_workspace_size(shape) bytes of device memory
 */
int sdm_forward(const sslp_sdm_shape* shape, int dtype, int residual_mode, const void* sw1,
                const void* sw2, const void* sr1, const void* sr2, const void* v,
                const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                float* wt_w, int32_t* idx_r, float* wt_r, void* workspace, size_t ws_bytes,
                void* stream);

/*
 * sdm_forward_noalloc -- sdm_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, semantics and kernels as sdm_forward,
 * minus the workspace: the scratch it needs (the addressing arrays and the
 * chunk plans) lives in a fixed array of SSLP_NOALLOC_SCRATCH_BYTES inside the
 * library, one copy per GPU, held until the process ends.  The call allocates
 * nothing and returns SSLP_ERR_WORKSPACE when sdm_workspace_size(shape)
 * exceeds that maximum.  Every call on a GPU uses that GPU's one array:
 * calls that overlap on the same GPU (other streams, other threads) race and
 * must be serialised by the caller.  The array keeps whatever the last call
 * left; nothing in it needs to start at zero.  sdm_noalloc_scratch_bytes()
 * returns the maximum.
 */
#define SSLP_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t sdm_noalloc_scratch_bytes(void);
int sdm_forward_noalloc(const sslp_sdm_shape* shape, int dtype, int residual_mode,
                        const void* sw1, const void* sw2, const void* sr1, const void* sr2,
                        const void* v, const float* alpha, const float* beta, float* M, void* y,
                        int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r, void* stream);

/*
 * sdm_decode_step -- one token for each of B independent sequences (shape->T
 * must be 1): addressing, update and read of each sequence's own table.  Same
 * arithmetic as sdm_forward with T = 1 (Sparse Delta Memory slides, same
 * passages; decode is the use named on slide "Sparse arithmetic still pays
 * for random memory access").
 *   sw1, sw2, sr1, sr2 [B,H,sqrtN] dtype;  v [B,H,d_v] dtype;  alpha, beta [B,H] fp32;
 *   M [B,H,N,d_v] fp32 in/out;  y [B,H,d_v] dtype out;
 *   idx_w, wt_w [B,H,W] and idx_r, wt_r [B,H,R] optional outputs.
 *   workspace, ws_bytes >= sdm_decode_workspace_size(shape) (may be NULL if that is 0).
 */
size_t sdm_decode_workspace_size(const sslp_sdm_shape* shape);
int sdm_decode_step(const sslp_sdm_shape* shape, int dtype, int residual_mode, const void* sw1,
                    const void* sw2, const void* sr1, const void* sr2, const void* v,
                    const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                    float* wt_w, int32_t* idx_r, float* wt_r, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * sdm_address -- the addressing step alone (slide "Product keys select
 * addresses without scoring every slot"), for B*T*H problems of the shape.
 *   s1, s2 [B,T,H,sqrtN] dtype;  k per-half top-k;  budget 1..min(k^2,128);
 *   idx [B,T,H,budget] int32 out (rank order);  wt [B,T,H,budget] fp32 out.
 * The shape's k_w/k_r/W/R fields are ignored.
 */
int sdm_address(const sslp_sdm_shape* shape, int dtype, const void* s1, const void* s2, int k,
                int budget, int32_t* idx, float* wt, void* stream);

/*
 * sdm_sparse_update -- the recurrence alone, given caller-supplied addressing
 * (slides "Selected slots decay and update; other slots persist" Eqs.
 * (3)-(5) and "A v1 inconsistency ...").  Weights are used as given (any
 * sign, no normalisation), so with W = R = N, wt_w = k_t, wt_r = q_t and the
 * shared residual it computes the dense gated delta rule.
 *   idx_w [B,T,H,W] int32 slots in [0,N), DISTINCT within each token
 *         (duplicates give unspecified results);  wt_w [B,T,H,W] fp32;
 *   idx_r [B,T,H,R] int32 in [0,N);  wt_r [B,T,H,R] fp32;
 *   v, alpha, beta, M, y as in sdm_forward;  shape->k_w, k_r are ignored and
 *   W, R may be up to 128 regardless of k.
 *   workspace, ws_bytes >= sdm_workspace_size(shape).
 * Indices are not range-checked on the host; one outside [0,N) is contained
 * on the device and reported by sslp_device_error.  Execution: with T >= 64
 * and W = R = 32 or W = R = 64 the recurrence runs chunk-parallel (chunks of
 * 16 or 8 tokens; its plans take the workspace after the addressing), other
 * shapes one token at a time.
 */
int sdm_sparse_update(const sslp_sdm_shape* shape, int dtype, int residual_mode,
                      const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                      const float* wt_r, const void* v, const float* alpha, const float* beta,
                      float* M, void* y, void* workspace, size_t ws_bytes, void* stream);

/* output gate activation of sdm_norm_gate */
#define SSLP_GATE_NONE 0
#define SSLP_GATE_SILU 1    /* g * sigmoid(g) */
#define SSLP_GATE_SIGMOID 2 /* 1 / (1 + exp(-g)) */

/*
 * sdm_norm_gate -- the layer output after the read (Sparse Delta Memory
 * slides, "Selected slots decay and update; other slots persist": the read is
 * followed by RMS-Norm, output gating and head mixing), RMS-Norm and gate in
 * one pass over each row of d values:
 *   o = y / sqrt(mean(y^2) + eps) * gamma * act(gate)
 * Head mixing (the dense output projection) follows outside the library.
 *   rows   number of rows (B*T*H for a [B,T,H,d] read), >= 0
 *   d      row width (d_v), a multiple of 4, <= 4096
 *   y      [rows, d] dtype;  gate [rows, d] dtype (NULL allowed with SSLP_GATE_NONE)
 *   gamma  [d] fp32, shared by all rows;  eps >= 0
 *   o      [rows, d] dtype out; may alias y (in place)
 * The sum of squares, the scale and the gate are fp32.
 */
int sdm_norm_gate(long long rows, int d, int dtype, const void* y, const void* gate,
                  const float* gamma, float eps, int act, void* o, void* stream);

/* ------------------------------------------------------------------------ */
/* Sparse Delta Memory training: backward by undoing writes                 */
/* ------------------------------------------------------------------------ */

/*
 * sdm_forward_train -- sdm_forward that also keeps what the backward needs:
 * the addressing (idx_w, wt_w, idx_r, wt_r, now required) and, per token, the
 * write rows as they were before the token (Sparse Delta Memory slides, backup
 * "Backup: undoing writes avoids repeated full-table snapshots": the forward
 * updates the table in place and retains the sparse update information).
 *   saved [B,T,H,W,d_v] fp32 out: saved[b,t,h,n,:] = M_{t-1}[idx_w[b,t,h,n], :]
 *   (T W d_v values per head, instead of one table per chunk).
 *   workspace, ws_bytes >= sdm_train_workspace_size(shape) (may be 0 / NULL
 *   when that is 0), 256-byte aligned, owned by the caller.
 * Other arguments as sdm_forward.  The recurrence runs as in sdm_forward: in
 * chunks (slides "Training parallelizes within chunks and recurs across
 * chunks") for T >= 64 and W = R = 32 or 64, each chunk's pre-write rows
 * coming out of the walk over every slot's visits; one token at a time
 * otherwise.  Errors: as sdm_forward, SSLP_ERR_WORKSPACE for a short workspace.
 */
int sdm_forward_train(const sslp_sdm_shape* shape, int dtype, int residual_mode, const void* sw1,
                      const void* sw2, const void* sr1, const void* sr2, const void* v,
                      const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                      float* wt_w, int32_t* idx_r, float* wt_r, float* saved, void* workspace,
                      size_t ws_bytes, void* stream);

/*
 * sdm_sparse_update_train -- sdm_sparse_update that also writes `saved` as
 * sdm_forward_train does (addressing given by the caller; W, R up to 128;
 * workspace as sdm_forward_train).
 */
int sdm_sparse_update_train(const sslp_sdm_shape* shape, int dtype, int residual_mode,
                            const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                            const float* wt_r, const void* v, const float* alpha,
                            const float* beta, float* M, void* y, float* saved, void* workspace,
                            size_t ws_bytes, void* stream);

/* Workspace bytes of sdm_forward_train and sdm_sparse_update_train: the
 * per-chunk plans of the chunk-parallel recurrence (0 for shapes that run one
 * token at a time, and for an invalid shape). */
size_t sdm_train_workspace_size(const sslp_sdm_shape* shape);

/* Workspace bytes of sdm_backward: per-token partial sums of the scalar
 * gradients for each slice of d_v (8 columns on the chunk-parallel path, 16
 * otherwise), the weight gradients when the caller does not ask for them, and
 * on the chunk-parallel path the per-chunk plans of both directions.  0 for an
 * invalid shape. */
size_t sdm_backward_workspace_size(const sslp_sdm_shape* shape);

/*
 * sdm_backward -- gradient of the SDM forward (Eqs. (3)-(5), either residual
 * form) by undoing writes (backup "Backup: undoing writes avoids repeated
 * full-table snapshots"): the tokens are walked in reverse with the table at
 * M_t; each token's saved rows step it back to M_{t-1}.  With G the gradient
 * of the table, per token t (reverse):
 *   G[j_m] += wt^r_m dy_t and dwt_r_m = <M_t[j_m], dy_t> for the read slots;
 *   then through the write with P_n = saved rows, M~_n = alpha_t P_n:
 *   SHARED:   r = v_t - sum_n wt_n M~_n;  dv_t = dr = sum_n beta_t wt_n G[i_n];
 *             dbeta_t = sum_n wt_n <G[i_n], r>;  dwt_n = beta_t <G[i_n], r> - <M~_n, dr>;
 *             dM~_n = G[i_n] - wt_n dr
 *   PER_SLOT: dv_t = sum_n beta_t wt_n G[i_n];  dbeta_t = sum_n wt_n <G[i_n], v_t - M~_n>;
 *             dwt_n = beta_t <G[i_n], v_t - M~_n>;  dM~_n = (1 - beta_t wt_n) G[i_n]
 *   dalpha_t = sum_n <P_n, dM~_n>;  G[i_n] = alpha_t dM~_n;  M[i_n] = P_n.
 * The score-half gradients follow from the softmax of the selected scores
 * s1[a] + s2[b] with the selection held fixed (slide "Product keys select
 * addresses without scoring every slot"): ds_m = wt_m (dwt_m - sum_j wt_j dwt_j),
 * added into ds1[a_m] and ds2[b_m]; halves in no selected pair get 0.
 *
 *   idx_w, wt_w, idx_r, wt_r  the forward's addressing (read slots, like write
 *                             slots, distinct within a token);
 *   v, alpha, beta            the forward's inputs;
 *   M      [B,H,N,d_v] fp32   in: the table after the forward; out: the table
 *                             before it (every write undone);
 *   saved  [B,T,H,W,d_v] fp32 from sdm_forward_train / sdm_sparse_update_train;
 *   dy     [B,T,H,d_v] dtype  gradient of y;
 *   dM     [B,H,N,d_v] fp32   in: gradient of the final table (zeros if none);
 *                             out: gradient of the initial table;
 *   dv     [B,T,H,d_v] dtype out;  dalpha, dbeta [B,T,H] fp32 out;
 *   dwt_w [B,T,H,W], dwt_r [B,T,H,R] fp32 optional out;
 *   dsw1, dsw2 / dsr1, dsr2 [B,T,H,sqrtN] fp32 optional out, each pair both or
 *                             neither (NULL skips that addressing backward);
 *   workspace, ws_bytes >= sdm_backward_workspace_size(shape).
 * The scalar gradients are added over d_v in a fixed order (deterministic).
 * Execution: with T >= 64 and W = R = 32 or 64 (the shapes whose forward is
 * chunk-parallel) the same gradients are formed chunk by chunk in reverse
 * (slides "Training parallelizes within chunks and recurs across chunks"): the
 * transpose of the chunk's linear map gives every token's dr at once, and each
 * slot's gradient row is carried backwards through its events in the chunk;
 * other shapes take the per-token sweep above.  A chunk holding a slot index
 * outside [0, N) is skipped (its gradients are 0, the tables keep their rows)
 * and reported through sslp_device_error.
 */
int sdm_backward(const sslp_sdm_shape* shape, int dtype, int residual_mode, const int32_t* idx_w,
                 const float* wt_w, const int32_t* idx_r, const float* wt_r, const void* v,
                 const float* alpha, const float* beta, float* M, const float* saved,
                 const void* dy, float* dM, void* dv, float* dalpha, float* dbeta, float* dwt_w,
                 float* dwt_r, float* dsw1, float* dsw2, float* dsr1, float* dsr2, void* workspace,
                 size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Gated DeltaNet / Kimi Delta Attention (dense limit: every slot selected)  */
/* ------------------------------------------------------------------------ */

/*   B, T, H; d_k = d_v = 128 and chunk = 64 (other sizes SSLP_ERR_UNSUPPORTED);
 *   bf16 q/k/v (SSLP_FP32 is SSLP_ERR_UNSUPPORTED). */
typedef struct {
    int B, T, H, d_k, d_v, chunk;
} sslp_gdn_shape;

/* Workspace bytes of gdn_chunk_forward: one record per (batch, head, chunk of
 * 64 tokens) holding the state-independent part of the chunk (about 89 KB:
 * the triangular-solve products, decayed operands and intra-chunk scores).
 * 0 for an invalid shape or T = 0. */
size_t gdn_workspace_size(const sslp_gdn_shape* shape);

/*
 * gdn_chunk_forward -- chunked forward of the gated delta rule (slides "GDN
 * and KDA change the granularity of forgetting", Eqs. 15-20, and "DeltaNet
 * writes a correction to the current association", Eq. 14).  With the state
 * S = W^T of shape [d_k, d_v] (row = key channel), per token:
 *   S~ = alpha_t S (SCALAR) or Diag(alpha_t) S (CHANNEL);
 *   S  = S~ + beta_t k_t (v_t - S~^T k_t)^T;   o_t = S^T q_t (after the write).
 * No query scaling and no key normalisation inside (the caller normalises).
 *   q, k  [B,T,H,d_k] dtype;  v [B,T,H,d_v] dtype;
 *   alpha [B,T,H] fp32 (SCALAR) or [B,T,H,d_k] fp32 (CHANNEL), in (0,1];
 *         CHANNEL: the chunked form factors each key channel's decay inside
 *         16-token blocks, exact (to rounding) for alpha in [2^-4, 1]; smaller
 *         per-channel decays give finite but less accurate results;
 *   beta  [B,T,H] fp32;
 *   S0    [B,H,d_k,d_v] fp32 initial state, or NULL for zeros;
 *   S_out [B,H,d_k,d_v] fp32 final state (may alias S0);
 *   o     [B,T,H,d_v] dtype out.
 *   workspace, ws_bytes >= gdn_workspace_size(shape) (may be NULL if that is 0),
 *   else SSLP_ERR_WORKSPACE.  All chunks are prepared in parallel first, then
 *   one pass over the chunks carries the state.
 */
int gdn_chunk_forward(const sslp_gdn_shape* shape, int dtype, int decay_mode, const void* q,
                      const void* k, const void* v, const float* alpha, const float* beta,
                      const float* S0, float* S_out, void* o, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * gdn2_chunk_forward -- GDN2 (slides "Linear Attention Architectures", "GDN2
 * separates key-side erase and value-side write", Eqs. 21-24), chunked like
 * gdn_chunk_forward with the per-channel (KDA) decay.  In the transposed
 * state S = W^T [d_k, d_v], per token:
 *   S~ = Diag(alpha_t) S;  r = (w_t (.) v_t) - S~^T (b_t (.) k_t);
 *   S = S~ + k_t r^T;      o_t = S^T q_t.
 * b = w = beta 1 is KDA.
 *   q, k [B,T,H,d_k] dtype; v [B,T,H,d_v] dtype;
 *   alpha, erase (b) [B,T,H,d_k] fp32; write (w) [B,T,H,d_v] fp32; alpha as
 *   gdn_chunk_forward's CHANNEL mode (exact for alpha in [2^-4, 1]);
 *   S0, S_out, o, workspace (gdn_workspace_size), errors: as gdn_chunk_forward.
 */
int gdn2_chunk_forward(const sslp_gdn_shape* shape, int dtype, const void* q, const void* k,
                       const void* v, const float* alpha, const float* erase, const float* write,
                       const float* S0, float* S_out, void* o, void* workspace, size_t ws_bytes,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Sparse State Expansion                                                    */
/* ------------------------------------------------------------------------ */

/*   B, T, H; N routed partitions 1..8 plus one shared; topk 1..min(N,4);
 *   c = d = 128 and chunk = 64 (other sizes SSLP_ERR_UNSUPPORTED); bf16 q/k/v. */
typedef struct {
    int B, T, H, N, topk, c, d, chunk;
} sslp_sse_shape;

/* Workspace bytes of sse_forward and sse_forward_masking: the routing of
 * every token (B*T*H*topk partition indices and gates, used when the caller
 * passes sel or e_sel as NULL), every routed partition's visit list
 * (B*H*N*T int32) and the token's contributions by slot before they are summed
 * (B*T*H*(topk+1)*d bf16).  0 for an invalid shape. */
size_t sse_workspace_size(const sslp_sse_shape* shape);

/*
 * sse_forward -- gated top-k partition routing, then the GLA recurrence of
 * each visited partition with decay advancing only on visits, plus the
 * always-active shared partition (slides "One gate controls both writes and
 * reads" Eqs. (9)-(14), "A memory decays only when its partition is
 * visited", "Varlen groups tokens while preserving causal order", backup
 * "Selected gate mass is usually below one").  Per token:
 *   e = softmax(logits_t) over N;  T_t = top-k of the logits (ties -> lowest index);
 *   S^i = Diag(lambda_t) S^i + e_i k_t^T v_t  for i in T_t (others untouched);
 *   S^N = Diag(lambda_t) S^N + k_sh_t^T v_t   (shared partition, every token);
 *   o_t = sum_{i in T_t, rank order} e_i q_t S^i + q_sh_t S^N.
 * The selected gate values are not renormalised.
 *   gate_logits [B,T,H,N] fp32;
 *   q, k [B,T,H,c] dtype (k already softmax-normalised over c by the caller);
 *   v [B,T,H,d] dtype;  lambda [B,T,H,c] fp32 in (0,1];
 *   q_sh, k_sh [B,T,H,c] dtype or NULL (then q, k are used);
 *   S [B,H,N+1,c,d] fp32 states in/out (index N = shared partition);
 *   o [B,T,H,d] dtype out;  sel [B,T,H,topk] int32 and e_sel [B,T,H,topk] fp32 optional.
 *   workspace, ws_bytes >= sse_workspace_size(shape) (may be NULL when T = 0);
 *   SSLP_ERR_WORKSPACE if too small.
 * Execution follows the varlen layout: the routing of all tokens, then every
 * routed partition's visits grouped in time order, one chunked pass over every
 * partition sequence (shared included), and the sum of each token's
 * contributions in rank order, then shared.
 */
int sse_forward(const sslp_sse_shape* shape, int dtype, const float* gate_logits, const void* q,
                const void* k, const void* v, const float* lambda, const void* q_sh,
                const void* k_sh, float* S, void* o, int32_t* sel, float* e_sel, void* workspace,
                size_t ws_bytes, void* stream);

/*
 * sse_forward_masking -- the same operation as sse_forward, run as the masking
 * execution that the SSE slides contrast with varlen grouping ("Varlen groups
 * tokens while preserving causal order"): every routed partition steps over
 * every token of the sequence; a token that does not select partition i
 * writes nothing to S^i, reads nothing from it, and leaves its decay at 1, so
 * S^i still decays only on its visits.  In exact arithmetic the results equal
 * sse_forward's; the work grows by N / topk on the routed partitions.
 * Arguments, layouts, workspace and errors as sse_forward.
 */
int sse_forward_masking(const sslp_sse_shape* shape, int dtype, const float* gate_logits,
                        const void* q, const void* k, const void* v, const float* lambda,
                        const void* q_sh, const void* k_sh, float* S, void* o, int32_t* sel,
                        float* e_sel, void* workspace, size_t ws_bytes, void* stream);

/*
 * sse_decode_step -- one token of every sequence (shape->T must be 1): the same
 * operation as sse_forward with T = 1, reading and writing only the topk
 * selected states and the shared one (the SSE slides' note on decoding under
 * "Varlen groups tokens while preserving causal order": only the selected
 * recurrent states are updated).  Layouts as in sse_forward with T = 1:
 *   gate_logits [B,1,H,N] fp32; q, k, q_sh, k_sh [B,1,H,c] dtype; v [B,1,H,d];
 *   lambda [B,1,H,c] fp32; S [B,H,N+1,c,d] fp32 in/out; o [B,1,H,d] dtype out;
 *   sel [B,1,H,topk] int32 and e_sel [B,1,H,topk] fp32 optional (written when
 *   given).  No workspace.  Errors: SSLP_ERR_INVALID_ARG when T != 1, else as
 *   sse_forward.  Steps of one sequence must be issued in order on one stream.
 */
int sse_decode_step(const sslp_sse_shape* shape, int dtype, const float* gate_logits,
                    const void* q, const void* k, const void* v, const float* lambda,
                    const void* q_sh, const void* k_sh, float* S, void* o, int32_t* sel,
                    float* e_sel, void* stream);

/* ------------------------------------------------------------------------ */
/* utilities                                                                 */
/* ------------------------------------------------------------------------ */

/* Description of the last failure on the calling thread ("" if none). */
const char* sslp_last_error(void);

/*
 * sslp_device_error -- whether a kernel met a caller-supplied SDM slot index
 * outside [0, N) (sdm_sparse_update, sdm_sparse_update_train, sdm_backward)
 * since the last query on this device: 1 if so, 0 if not, or a negative
 * status.  Such a call leaves its results undefined but touches no memory
 * outside the given tensors: a token's out-of-range slot is replaced by slot
 * 0 (per-token kernels), and a chunk (16 or 8 tokens) holding one is skipped
 * (y = 0, the table unchanged; chunk-parallel kernel).  The query synchronises
 * `stream` and clears the flag; it is the only entry point that synchronises.
 */
int sslp_device_error(void* stream);

/* SSLP_VERSION of the built library. */
int sslp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSLP_H */
