// K5 + K6 for one token per sequence: the Sparse State Expansion decode step.
//
// Slides "Scaling Linear Attention with Sparse State Expansion": "One gate
// controls both writes and reads" (Eqs. (9)-(14)) for a single token, and
// "Varlen groups tokens while preserving causal order", whose note on decoding
// is that only the selected recurrent states are updated.  For each
// (sequence, head) with states S^0..S^{N-1} (routed) and S^N (shared):
//   e = softmax(logits) over N (fp32), T = top-k of the logits (ties -> lowest);
//   S^i = Diag(lambda) S^i + e_i k^T v           for i in T (others untouched);
//   S^N = Diag(lambda) S^N + k_sh^T v;
//   o   = sum_{i in T, rank order} e_i q S^i + q_sh S^N.
// The same operation as the chunked prefill kernel with T = 1, but it reads
// and writes only the k + 1 touched states, which is all the traffic a decode
// step must move: 2 (k + 1) c d 4 bytes per (sequence, head).
//
// One workgroup of 256 threads per (sequence, head, 32 columns of d): thread
// (row group g = t / 32, column n = t % 32) owns rows 16 g .. 16 g + 15 of
// column n of every touched state slice, so a wave's loads and stores of a
// state row are 128-byte contiguous.  All touched slices are loaded before any
// is used.
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

constexpr int CR = 128;      // state rows (key width c)
constexpr int DB = 32;       // columns of d per workgroup
constexpr int RPT = 16;      // rows per thread
constexpr int NG = CR / RPT;  // row groups
constexpr int MAXN = 8;
constexpr int MAXK = 4;

struct SseDecodeArgs {
    int B, H, N, topk, dv;
    const float* logits;  // [B, H, N]
    const uint16_t* q;    // [B, H, c] bf16
    const uint16_t* k;
    const uint16_t* v;    // [B, H, d]
    const float* lam;     // [B, H, c]
    const uint16_t* q_sh;
    const uint16_t* k_sh;
    float* S;             // [B, H, N + 1, c, d]
    uint16_t* o;          // [B, H, d]
    int32_t* sel;         // [B, H, topk] or null
    float* e_sel;
};

SSLP_DEVICE float bfl(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

__global__ __launch_bounds__(256) void sse_decode_kernel(SseDecodeArgs a) {
    __shared__ float s_q[CR], s_k[CR], s_qs[CR], s_ks[CR], s_lam[CR];
    __shared__ float s_part[MAXK + 1][NG][DB];
    const int tid = threadIdx.x;
    const int nblk = a.dv / DB;
    const int cb = blockIdx.x % nblk, bh = blockIdx.x / nblk;
    const int n = tid % DB, g = tid / DB;
    const int N = a.N, topk = a.topk;
    const size_t row0 = (size_t)bh * CR;

    // ---- routing (every thread, the same fp32 arithmetic as the prefill router) ----
    const float* lg = a.logits + (size_t)bh * N;
    float lv[MAXN];
    float mx = lg[0];
#pragma unroll
    for (int i = 0; i < MAXN; ++i) {
        lv[i] = i < N ? lg[i] : 0.f;
        if (i < N && lv[i] > mx) mx = lv[i];
    }
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < MAXN; ++i)
        if (i < N) z += __expf(lv[i] - mx);
    int sel[MAXK + 1];
    float gsel[MAXK + 1];
    unsigned taken = 0;
#pragma unroll
    for (int r = 0; r < MAXK; ++r) {
        sel[r] = -1;
        gsel[r] = 0.f;
        if (r < topk) {
            int best = -1;
#pragma unroll
            for (int i = 0; i < MAXN; ++i)
                if (i < N && !((taken >> i) & 1u) && (best < 0 || lv[i] > lv[best])) best = i;
            taken |= 1u << best;
            sel[r] = best;
            gsel[r] = __expf(lv[best] - mx) / z;
        }
    }
    if (cb == 0 && tid < topk) {
        int sr = 0;
        float gr = 0.f;
#pragma unroll
        for (int r = 0; r < MAXK; ++r)
            if (r == tid) {
                sr = sel[r];
                gr = gsel[r];
            }
        if (a.sel) a.sel[(size_t)bh * topk + tid] = sr;
        if (a.e_sel) a.e_sel[(size_t)bh * topk + tid] = gr;
    }

    // ---- the token's vectors ----
    if (tid < CR) {
        s_q[tid] = bfl(a.q[row0 + tid]);
        s_k[tid] = bfl(a.k[row0 + tid]);
        s_qs[tid] = bfl((a.q_sh ? a.q_sh : a.q)[row0 + tid]);
        s_ks[tid] = bfl((a.k_sh ? a.k_sh : a.k)[row0 + tid]);
        s_lam[tid] = a.lam[row0 + tid];
    }
    const int col = cb * DB + n;
    const float vn = bfl(a.v[(size_t)bh * a.dv + col]);
    __syncthreads();

    // ---- touched state slices: ranks 0..topk-1, then the shared partition ----
    const int nt = topk + 1;
    float st[MAXK + 1][RPT];
    auto slice = [&](int r) {
        const int part = r < topk ? sel[r] : N;
        return a.S + (((size_t)bh * (N + 1) + part) * CR + RPT * g) * a.dv + col;
    };
#pragma unroll
    for (int r = 0; r <= MAXK; ++r)
        if (r < nt) {
            const float* p = slice(r);
#pragma unroll
            for (int i = 0; i < RPT; ++i) st[r][i] = p[(size_t)i * a.dv];
        }
#pragma unroll
    for (int r = 0; r <= MAXK; ++r)
        if (r < nt) {
            const bool shared = r == topk;
            const float e = shared ? 1.f : gsel[r];
            const float* kk = shared ? s_ks : s_k;
            const float* qq = shared ? s_qs : s_q;
            float* p = slice(r);
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = RPT * g + i;
                const float s = fmaf(s_lam[row], st[r][i], e * kk[row] * vn);
                p[(size_t)i * a.dv] = s;
                acc = fmaf(qq[row], s, acc);
            }
            s_part[r][g][n] = acc;
        }
    __syncthreads();

    // ---- o = sum over ranks of e_r q S^r, then the shared q_sh S^N ----
    if (g == 0) {
        float o = 0.f;
#pragma unroll
        for (int r = 0; r <= MAXK; ++r)
            if (r < nt) {
                float t = 0.f;
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) t += s_part[r][gg][n];
                o += (r == topk ? 1.f : gsel[r]) * t;
            }
        a.o[(size_t)bh * a.dv + col] = f32_to_bf16(o).bits;
    }
}

}  // namespace

hipError_t launch_sse_decode(int B, int H, int N, int topk, int dv, const float* logits,
                             const void* q, const void* k, const void* v, const float* lam,
                             const void* q_sh, const void* k_sh, float* S, void* o, int32_t* sel,
                             float* e_sel, hipStream_t st) {
    if (N < 1 || N > MAXN || topk < 1 || topk > MAXK || topk > N || dv % DB != 0)
        return hipErrorInvalidValue;
    SseDecodeArgs a{B,
                    H,
                    N,
                    topk,
                    dv,
                    logits,
                    static_cast<const uint16_t*>(q),
                    static_cast<const uint16_t*>(k),
                    static_cast<const uint16_t*>(v),
                    lam,
                    static_cast<const uint16_t*>(q_sh),
                    static_cast<const uint16_t*>(k_sh),
                    S,
                    static_cast<uint16_t*>(o),
                    sel,
                    e_sel};
    const long long grid = (long long)B * H * (dv / DB);
    if (grid == 0) return hipSuccess;
    sse_decode_kernel<<<(unsigned)grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace sslp
