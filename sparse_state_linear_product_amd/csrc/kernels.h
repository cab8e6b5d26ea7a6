// Host-side launchers of the libsslp kernels (one per .hip file).  Each
// enqueues on `st` and returns the launch status; argument validation is done
// by the C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sslp {

// ---- Sparse Delta Memory ----
// number of pairs (i,j), i,j < k, with (i+1)(j+1) <= budget
int address_set_size(int k, int budget);

hipError_t launch_sdm_address(int P, int sqrtN, int dtype, const void* s1, const void* s2, int k,
                              int budget, int32_t* idx, float* wt, hipStream_t st);
// write and read addressing of the same problems (one launch for small batches)
hipError_t launch_sdm_address_pair(int P, int sqrtN, int dtype, const void* sw1, const void* sw2,
                                   int k_w, int W, int32_t* iw, float* ww, const void* sr1,
                                   const void* sr2, int k_r, int R, int32_t* ir, float* wr,
                                   hipStream_t st);

struct SdmUpdateArgs {
    int B, T, H, N, dv, W, R;
    int dtype;          // 0 fp32, 1 bf16 for v and y
    int residual_mode;  // 0 shared, 1 per-slot
    const int32_t* idx_w;
    const float* wt_w;
    const int32_t* idx_r;
    const float* wt_r;
    const void* v;
    const float* alpha;
    const float* beta;
    float* M;
    void* y;
    // [B,T,H,W,dv] fp32 or null: when set, each token's write rows as they were
    // before the token (what a backward sweep restores); only the per-token
    // kernel writes it
    float* saved;
    // device word set to 1 when a slot index outside [0, N) is met (such a
    // slot is replaced by slot 0, or the chunk holding it is skipped, so no
    // access leaves the table); may be null
    unsigned* err;
};
hipError_t launch_sdm_update(const SdmUpdateArgs& a, hipStream_t st);

// ---- SDM decode step in one launch (sdm_decode.hip): addressing of both sets
//      and the update / read of one token per (sequence, head) ----
struct SdmDecodeArgs {
    int P;  // B * H problems (one token each)
    int sqrtN, N, dv;
    int dtype;          // 0 fp32, 1 bf16 for the score halves, v and y
    int residual_mode;  // 0 shared, 1 per-slot
    const void* s1[2];  // [P, sqrtN] halves of the write (0) and read (1) scores
    const void* s2[2];
    int32_t* idx[2];    // [P, W] / [P, R] optional copies of the selections
    float* wt[2];
    int k[2], budget[2], nD[2];  // nD is filled in by the launcher
    const void* v;      // [P, dv]
    const float* alpha;  // [P]
    const float* beta;
    float* M;           // [P, N, dv]
    void* y;            // [P, dv]
};
bool sdm_decode_fused_fits(int sqrtN, int dv, int k_w, int W, int k_r, int R);
hipError_t launch_sdm_decode_fused(SdmDecodeArgs a, hipStream_t st);

// ---- SDM backward (sdm_backward.hip) ----
struct SdmBwdArgs {
    int B, T, H, N, dv, W, R;
    int dtype;          // 0 fp32, 1 bf16 for v, dy and dv
    int residual_mode;  // 0 shared, 1 per-slot
    const int32_t* idx_w;
    const float* wt_w;
    const int32_t* idx_r;
    const float* wt_r;
    const void* v;
    const float* alpha;
    const float* beta;
    float* M;            // [B,H,N,dv] in: M_T; out: M_0 (writes undone)
    const float* saved;  // [B,T,H,W,dv] pre-write rows
    const void* dy;      // [B,T,H,dv]
    float* dM;           // [B,H,N,dv] in: dL/dM_T; out: dL/dM_0
    void* dv_out;        // [B,T,H,dv]
    float* part;         // [B,T,H, nslice, 2 + W + R] per-slice partial sums
    float* dalpha;       // [B,T,H]
    float* dbeta;        // [B,T,H]
    float* dwt_w;        // [B,T,H,W]
    float* dwt_r;        // [B,T,H,R]
    unsigned* err;       // as SdmUpdateArgs::err
};
// per-token partial sums of the scalar gradients, one set per slice of
// slice_cols columns of d_v, and their sum over the slices (in slice order)
size_t sdm_bwd_part_bytes(int B, int T, int H, int dv, int W, int R, int slice_cols);
hipError_t launch_sdm_bwd_reduce(const SdmBwdArgs& a, int slice_cols, hipStream_t st);
// per-token reverse sweep (16-column slices) + the reduction
hipError_t launch_sdm_update_backward(const SdmBwdArgs& a, hipStream_t st);
// gradient of the addressing softmax onto the score halves, P problems
hipError_t launch_sdm_address_backward(int P, int sqrtN, int budget, const int32_t* idx,
                                       const float* wt, const float* dwt, float* ds1, float* ds2,
                                       hipStream_t st);
// the same for the write and the read sets of a step, in one launch where they fit
hipError_t launch_sdm_address_backward_pair(int P, int sqrtN, int W, const int32_t* idx_w,
                                            const float* wt_w, const float* dwt_w, float* dsw1,
                                            float* dsw2, int R, const int32_t* idx_r,
                                            const float* wt_r, const float* dwt_r, float* dsr1,
                                            float* dsr2, hipStream_t st);

// chunk-parallel recurrence (sdm_chunk.hip): supported shapes, workspace for
// its per-chunk plans, and the launcher (plan kernel + apply kernel)
bool sdm_chunked_supported(int B, int T, int H, int W, int R, int dv, long long N);
size_t sdm_chunk_plan_bytes(int B, int T, int H, int W);
hipError_t launch_sdm_update_chunked(const SdmUpdateArgs& a, void* plan, hipStream_t st);
// the plan kernel alone (the backward reuses the forward's plans)
hipError_t launch_sdm_chunk_plans(const SdmUpdateArgs& a, void* plan, hipStream_t st);
// chunk-parallel backward (sdm_chunk_bwd.hip), same shapes as the forward:
// its own per-chunk plans, and the launcher (forward plans, backward plans,
// the reverse sweep over chunks with 8-column slices, the slice reduction)
size_t sdm_chunk_bwd_plan_bytes(int B, int T, int H, int W);
constexpr int kChunkBwdSliceCols = 8;
hipError_t launch_sdm_backward_chunked(const SdmBwdArgs& a, void* fplan, void* bplan,
                                       hipStream_t st);

// RMS-Norm and output gate after the read (norm_gate.hip): rows x d, act 0 none,
// 1 SiLU, 2 sigmoid; d a multiple of 4 up to 4096; o may alias y
hipError_t launch_norm_gate(long long rows, int d, int dtype, const void* y, const void* g,
                            const float* gamma, float eps, int act, void* o, hipStream_t st);

// ---- Gated DeltaNet / KDA ----
// per-chunk records of the state-independent part (workspace), and the
// launcher (prep kernel over all chunks + state kernel over the chunk sequence)
size_t gdn_record_bytes(int B, int T, int H);
// kda: 0 GDN (alpha [B,T,H]), 1 KDA (alpha [B,T,H,dk]), 2 GDN2 (KDA decay, erase
// vector bvec [B,T,H,dk] and write vector wvec [B,T,H,dv] in place of beta)
hipError_t launch_gdn_chunk(int B, int T, int H, int dv, int dtype, int kda, const void* q,
                            const void* k, const void* v, const float* alpha, const float* beta,
                            const float* S0, float* S_out, void* o, void* rec, hipStream_t st,
                            const float* bvec = nullptr, const float* wvec = nullptr);

// ---- Sparse State Expansion ----
// scratch of launch_sse: the visit lists and counts of every routed partition
// and the per-slot contributions of every token
size_t sse_scratch_bytes(int B, int T, int H, int N, int topk, int dv);
// masking = 1: the masked execution (every routed partition over every token,
// unselected tokens with gate 0 and decay 1) instead of the grouped visits
hipError_t launch_sse(int B, int T, int H, int N, int topk, int dv, int dtype,
                      const float* logits, const void* q, const void* k, const void* v,
                      const float* lam, const void* q_sh, const void* k_sh, float* S, void* o,
                      int32_t* sel, float* e_sel, void* scratch, hipStream_t st, int masking = 0);
// one decode step (one token per sequence), touching only the selected states
hipError_t launch_sse_decode(int B, int H, int N, int topk, int dv, const float* logits,
                             const void* q, const void* k, const void* v, const float* lam,
                             const void* q_sh, const void* k_sh, float* S, void* o, int32_t* sel,
                             float* e_sel, hipStream_t st);

}  // namespace sslp
