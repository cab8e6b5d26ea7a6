// Backward of the Sparse Delta Memory recurrence by undoing writes, and of the
// addressing softmax.
//
// Sparse Delta Memory slides: "Selected slots decay and update; other slots
// persist" (Eqs. (3)-(5)), "A v1 inconsistency matters for reproducing the
// update" (shared or per-slot residual) and the backup "Backup: undoing writes
// avoids repeated full-table snapshots": the forward keeps each token's write
// rows as they were before the token (T W d_v values per head instead of a
// table per chunk); the backward walks the tokens in reverse with the table
// at M_t and steps it back to M_{t-1} by restoring those rows, so on return
// the table holds M_0 again.
//
// Per token t, in reverse, with G the running gradient of the table:
//   read   y = sum_m e_m M_t[j_m]:  de_m = <M_t[j_m], dy>;  G[j_m] += e_m dy
//   write  P_n = M_{t-1}[i_n] (saved), Mt_n = alpha P_n, G_n = G[i_n]:
//     shared    r = v - sum_n w_n Mt_n;  dr = sum_n beta w_n G_n = dv;
//               dbeta = sum_n w_n <G_n, r>;  dw_n = beta <G_n, r> - <Mt_n, dr>;
//               dMt_n = G_n - w_n dr
//     per-slot  dv = sum_n beta w_n G_n;  dbeta = sum_n w_n <G_n, v - Mt_n>;
//               dw_n = beta <G_n, v - Mt_n>;  dMt_n = (1 - beta w_n) G_n
//     dalpha = sum_n <P_n, dMt_n>;  G[i_n] = alpha dMt_n;  M[i_n] = P_n.
//
// Every operation on a d_v column is independent of the other columns except
// the scalar gradients (dalpha, dbeta, dw, de), which are sums over d_v.  So
// the sweep runs as in the per-token forward kernel: one wavefront per
// 16-column slice of a (batch, head), lane (g, c) = (lane / 16, lane % 16)
// owning column c of rows g, g + 4, ...; each wavefront writes its slice's
// partial sums per token, and a second kernel adds the slices in a fixed order
// (deterministic, no atomics).
//
// Ordering: all loads and stores of table and gradient rows are issued by the
// one wavefront that owns the columns, in program order, so each token sees
// the restores and gradient updates of the tokens after it.  Each token makes
// one trip for its rows (M_t and G at the read slots, G at the write slots,
// all requested together, with the next token's indices, weights and saved
// rows already in flight); a write slot that the same token also reads gets
// the read's contribution added in registers.  Read slots must be distinct
// within a token (the addressing guarantees it), as write slots are.
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

constexpr int kCols = 16;  // columns per wavefront

SSLP_DEVICE int nslices(int dv) { return (dv + kCols - 1) / kCols; }

// Everything a token needs that does not depend on the table (gates, indices,
// weights, the saved rows, v and dy).  It is loaded one token ahead, from
// clamped (always valid) addresses; out-of-range rows and columns are masked
// where the values are used, so no load waits on a condition.
template <int NL>
struct BwdMeta {
    float al, be, dyc, vc;
    int sw[NL], sr[NL];
    float w[NL], e[NL], P[NL];
};

template <typename io_t, int NL>
SSLP_DEVICE void load_meta(BwdMeta<NL>& m, const SdmBwdArgs& a, size_t bth, int g, int colc) {
    const io_t* vin = static_cast<const io_t*>(a.v);
    const io_t* dyin = static_cast<const io_t*>(a.dy);
    m.al = a.alpha[bth];
    m.be = a.beta[bth];
    m.dyc = to_f32(dyin[bth * a.dv + colc]);
    m.vc = to_f32(vin[bth * a.dv + colc]);
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int nw = min(g + 4 * r, a.W - 1), nr = min(g + 4 * r, a.R - 1);
        m.sw[r] = a.idx_w[bth * a.W + nw];  // range-checked where used (keep_slot)
        m.w[r] = a.wt_w[bth * a.W + nw];
        m.P[r] = a.saved[(bth * a.W + nw) * a.dv + colc];
        m.sr[r] = a.idx_r[bth * a.R + nr];
        m.e[r] = a.wt_r[bth * a.R + nr];
    }
}

template <typename io_t, int NL>
__global__ __launch_bounds__(64) void sdm_update_bwd_kernel(SdmBwdArgs a) {
    __shared__ int s_rs[4 * NL];
    __shared__ float s_re[4 * NL];
    const int nslice = nslices(a.dv);
    const int slice = blockIdx.x % nslice;
    const int bh = blockIdx.x / nslice;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int lane = threadIdx.x;
    const int g = lane >> 4, c = lane & 15;
    const int col = slice * kCols + c;
    const bool colok = col < a.dv;
    const int colc = colok ? col : a.dv - 1;
    const int W = a.W, R = a.R;
    const int NP = 2 + W + R;
    const size_t tab0 = ((size_t)b * a.H + h) * (size_t)a.N * a.dv;
    float* tab = a.M + tab0;
    float* G = a.dM + tab0;
    io_t* dvout = static_cast<io_t*>(a.dv_out);
    const bool shared = a.residual_mode == 0;

    BwdMeta<NL> cur;
    bool bad = false;  // a slot index outside [0, N) was seen (and replaced by 0)
    if (a.T > 0) load_meta<io_t, NL>(cur, a, ((size_t)b * a.T + (a.T - 1)) * a.H + h, g, colc);
    for (int t = a.T - 1; t >= 0; --t) {
        const size_t bth = ((size_t)b * a.T + t) * a.H + h;
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            cur.sw[r] = keep_slot(cur.sw[r], a.N, bad);
            cur.sr[r] = keep_slot(cur.sr[r], a.N, bad);
        }
        // ---- one trip for every row the token touches: M_t and G at the read
        //      slots, G at the write slots ----
        float mr[NL], gr[NL], gw[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            mr[r] = tab[(size_t)cur.sr[r] * a.dv + colc];
            gr[r] = G[(size_t)cur.sr[r] * a.dv + colc];
            gw[r] = G[(size_t)cur.sw[r] * a.dv + colc];
        }
        // the next token's table-independent data, in flight meanwhile
        BwdMeta<NL> nxt;
        load_meta<io_t, NL>(nxt, a, ((size_t)b * a.T + (t > 0 ? t - 1 : 0)) * a.H + h, g, colc);
        // ---- a write slot that is also read by this token: its G must include
        //      the read's e dy.  Lane (g, c) checks its write rows against read
        //      rows c, c + 16, ...; the 16 lanes of the row group add up ----
        if (c == 0) {
#pragma unroll
            for (int r = 0; r < NL; ++r)
                if (g + 4 * r < R) {
                    s_rs[g + 4 * r] = cur.sr[r];
                    s_re[g + 4 * r] = cur.e[r];
                }
        }
        wave_sync();
        float fix[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) fix[r] = 0.f;
#pragma unroll
        for (int j = 0; j < (4 * NL + 15) / 16; ++j) {
            const int m = c + 16 * j;
            if (m < R) {
                const int sm = s_rs[m];
                const float em = s_re[m];
#pragma unroll
                for (int r = 0; r < NL; ++r) fix[r] += sm == cur.sw[r] ? em : 0.f;
            }
        }
#pragma unroll
        for (int s = 1; s < 16; s <<= 1)
#pragma unroll
            for (int r = 0; r < NL; ++r) fix[r] += xor_lane_f(fix[r], s, lane_id());
        const float dyc = colok ? cur.dyc : 0.f, vc = colok ? cur.vc : 0.f;
        const float al = cur.al, be = cur.be;
        // ---- read after writing: de and the read contribution to G ----
        float pe[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const bool ok = g + 4 * r < R && colok;
            pe[r] = ok ? mr[r] * dyc : 0.f;
            if (ok) G[(size_t)cur.sr[r] * a.dv + col] = gr[r] + cur.e[r] * dyc;
        }
        // ---- the write, from the saved rows ----
        float P[NL], mt[NL], gn[NL], w[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const bool live = g + 4 * r < W && colok;
            w[r] = g + 4 * r < W ? cur.w[r] : 0.f;
            P[r] = live ? cur.P[r] : 0.f;
            gn[r] = live ? gw[r] + fix[r] * dyc : 0.f;
            mt[r] = al * P[r];
        }
        float vh = 0.f, dr = 0.f;
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            vh = fmaf(w[r], mt[r], vh);
            dr = fmaf(be * w[r], gn[r], dr);
        }
        vh += xor_lane_f(vh, 16, lane_id());
        vh += xor_lane_f(vh, 32, lane_id());
        dr += xor_lane_f(dr, 16, lane_id());
        dr += xor_lane_f(dr, 32, lane_id());
        const float rres = vc - vh;
        float pw[NL];
        float pa = 0.f, pb = 0.f;
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const float res = shared ? rres : vc - mt[r];
            const float gres = gn[r] * res;
            pw[r] = shared ? be * gres - mt[r] * dr : be * gres;
            pb = fmaf(w[r], gres, pb);
            const float dmt = shared ? gn[r] - w[r] * dr : (1.f - be * w[r]) * gn[r];
            pa = fmaf(P[r], dmt, pa);
            if (g + 4 * r < W && colok) {
                const size_t off = (size_t)cur.sw[r] * a.dv + col;
                G[off] = al * dmt;
                tab[off] = P[r];
            }
        }
        if (g == 0 && colok) dvout[bth * a.dv + col] = from_f32<io_t>(dr);
        // ---- partial sums over this slice's 16 columns ----
#pragma unroll
        for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                pe[r] += xor_lane_f(pe[r], s, lane_id());
                pw[r] += xor_lane_f(pw[r], s, lane_id());
            }
            pa += xor_lane_f(pa, s, lane_id());
            pb += xor_lane_f(pb, s, lane_id());
        }
        pa += xor_lane_f(pa, 16, lane_id());
        pa += xor_lane_f(pa, 32, lane_id());
        pb += xor_lane_f(pb, 16, lane_id());
        pb += xor_lane_f(pb, 32, lane_id());
        float* pp = a.part + (bth * nslice + slice) * NP;
        if (c == 0) {
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                if (g + 4 * r < W) pp[2 + g + 4 * r] = pw[r];
                if (g + 4 * r < R) pp[2 + W + g + 4 * r] = pe[r];
            }
        }
        if (lane == 0) {
            pp[0] = pa;
            pp[1] = pb;
        }
        wave_sync();
        cur = nxt;
    }
    report_slot_error(bad, a.err);
}

// Adds the slices' partial sums in slice order: one thread per (token, head, j).
__global__ __launch_bounds__(256) void sdm_bwd_reduce_kernel(SdmBwdArgs a, long long total,
                                                             int nslice) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int W = a.W, R = a.R, NP = 2 + W + R;
    const long long bth = i / NP;
    const int j = (int)(i - bth * NP);
    const float* pp = a.part + (size_t)bth * nslice * NP + j;
    // slices added in order; their loads are issued 16 at a time (a loop of
    // single loads waited for one memory round trip per slice)
    float s = 0.f;
    int k = 0;
    for (; k + 16 <= nslice; k += 16) {
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = pp[(size_t)(k + u) * NP];
#pragma unroll
        for (int u = 0; u < 16; ++u) s += x[u];
    }
    for (; k < nslice; ++k) s += pp[(size_t)k * NP];
    if (j == 0) a.dalpha[bth] = s;
    else if (j == 1) a.dbeta[bth] = s;
    else if (j < 2 + W) a.dwt_w[bth * W + (j - 2)] = s;
    else a.dwt_r[bth * R + (j - 2 - W)] = s;
}

// Softmax gradient with the selection fixed (slide "Product keys select
// addresses without scoring every slot": weights are a softmax of the selected
// candidate scores s1[a] + s2[b]):
//   ds_m = wt_m (dwt_m - sum_j wt_j dwt_j);  ds1[a_m] += ds_m;  ds2[b_m] += ds_m.
// One wavefront per problem; each output element adds its terms in rank order.
constexpr int kAbWaves = 4;
constexpr int kMaxBudget = 128;

__global__ __launch_bounds__(64 * kAbWaves) void sdm_address_bwd_kernel(
    int P, int sqrtN, int budget, const int32_t* __restrict__ idx, const float* __restrict__ wt,
    const float* __restrict__ dwt, float* __restrict__ ds1, float* __restrict__ ds2) {
    __shared__ float s_ds[kAbWaves][kMaxBudget];
    __shared__ int s_a[kAbWaves][kMaxBudget], s_b[kAbWaves][kMaxBudget];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long p = (long long)blockIdx.x * kAbWaves + wv;
    if (p >= P) return;  // whole wavefronts leave together; no block barrier below
    const int32_t* ip = idx + (size_t)p * budget;
    const float* w = wt + (size_t)p * budget;
    const float* dw = dwt + (size_t)p * budget;
    float dot = 0.f;
    for (int m = lane; m < budget; m += 64) dot = fmaf(w[m], dw[m], dot);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) dot += xor_lane_f(dot, s, lane_id());
    for (int m = lane; m < budget; m += 64) {
        const int n = ip[m];
        s_ds[wv][m] = w[m] * (dw[m] - dot);
        s_a[wv][m] = n / sqrtN;
        s_b[wv][m] = n - (n / sqrtN) * sqrtN;
    }
    wave_sync();
    for (int x = lane; x < sqrtN; x += 64) {
        float g1 = 0.f, g2 = 0.f;
        for (int m = 0; m < budget; ++m) {
            const float d = s_ds[wv][m];
            if (s_a[wv][m] == x) g1 += d;
            if (s_b[wv][m] == x) g2 += d;
        }
        ds1[(size_t)p * sqrtN + x] = g1;
        ds2[(size_t)p * sqrtN + x] = g2;
    }
}

// The same gradients for sqrtN <= 256: lane m (entry m < budget <= 64) sums
// the d of every entry of its row a_m (and of its column b_m) in entry order,
// so each sum is the one the loop above forms; the first entry of a row
// writes it into the wavefront's zeroed LDS copy of ds1 (ds2), which is then
// stored whole.  About a fifth of the instructions of the loop above.
// The write and read sets of a step go in one launch: workgroups below nblk0
// take set 0, the others set 1.
constexpr int kAbMaxN = 256;
struct AbSet {
    const int32_t* idx;
    const float* wt;
    const float* dwt;
    float* ds1;
    float* ds2;
    int budget;
};
struct AbPair {
    AbSet set[2];
    int P, sqrtN, nblk0;
};
__global__ __launch_bounds__(64 * kAbWaves) void sdm_address_bwd_small_kernel(AbPair ab) {
    __shared__ float s_g[kAbWaves][2][kAbMaxN];
    __shared__ float s_ds[kAbWaves][64];
    __shared__ int s_ab[kAbWaves][64];  // a_m | b_m << 16
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int si = (int)blockIdx.x >= ab.nblk0 ? 1 : 0;
    const AbSet& S = ab.set[si];
    const int P = ab.P, sqrtN = ab.sqrtN, budget = S.budget;
    const int32_t* __restrict__ idx = S.idx;
    const float* __restrict__ wt = S.wt;
    const float* __restrict__ dwt = S.dwt;
    float* __restrict__ ds1 = S.ds1;
    float* __restrict__ ds2 = S.ds2;
    const long long p = (long long)((int)blockIdx.x - si * ab.nblk0) * kAbWaves + wv;
    if (p >= P) return;  // whole wavefronts leave together; no block barrier below
    const bool on = lane < budget;
    const int m = on ? lane : 0;
    const int n = idx[(size_t)p * budget + m];
    const float w = wt[(size_t)p * budget + m], dw = dwt[(size_t)p * budget + m];
    float dot = on ? w * dw : 0.f;  // the first fmaf of the loop above is this product
    // (the wave sum in the same lane pattern as the loop above: one term per lane)
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) dot += xor_lane_f(dot, s, lane);
    // an entry whose slot lies outside [0, sqrtN^2) joins no row or column
    const bool ok = on && (unsigned)n < (unsigned)(sqrtN * sqrtN);
    const int am = ok ? n / sqrtN : 0, bm = ok ? n - am * sqrtN : 0;
    const float d = w * (dw - dot);
    s_ds[wv][lane] = on ? d : 0.f;
    s_ab[wv][lane] = ok ? (am | (bm << 16)) : -1;
    for (int x = lane; x < sqrtN; x += 64) {
        s_g[wv][0][x] = 0.f;
        s_g[wv][1][x] = 0.f;
    }
    wave_sync();
    float g1 = 0.f, g2 = 0.f;
    bool first1 = true, first2 = true;
    for (int q = 0; q < budget; ++q) {
        const int ab = s_ab[wv][q];
        const float dq = s_ds[wv][q];
        const bool same1 = (ab & 0xFFFF) == am, same2 = (ab >> 16) == bm;
        g1 += same1 ? dq : 0.f;
        g2 += same2 ? dq : 0.f;
        first1 = first1 && !(same1 && q < lane);
        first2 = first2 && !(same2 && q < lane);
    }
    if (ok && first1) s_g[wv][0][am] = g1;
    if (ok && first2) s_g[wv][1][bm] = g2;
    wave_sync();
    for (int x = lane; x < sqrtN; x += 64) {
        ds1[(size_t)p * sqrtN + x] = s_g[wv][0][x];
        ds2[(size_t)p * sqrtN + x] = s_g[wv][1][x];
    }
}

template <typename io_t>
hipError_t dispatch_bwd(int NL, dim3 grid, hipStream_t st, const SdmBwdArgs& a) {
    switch (NL) {
        case 1: sdm_update_bwd_kernel<io_t, 1><<<grid, 64, 0, st>>>(a); break;
        case 2: sdm_update_bwd_kernel<io_t, 2><<<grid, 64, 0, st>>>(a); break;
        case 4: sdm_update_bwd_kernel<io_t, 4><<<grid, 64, 0, st>>>(a); break;
        case 8: sdm_update_bwd_kernel<io_t, 8><<<grid, 64, 0, st>>>(a); break;
        case 16: sdm_update_bwd_kernel<io_t, 16><<<grid, 64, 0, st>>>(a); break;
        case 32: sdm_update_bwd_kernel<io_t, 32><<<grid, 64, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

size_t sdm_bwd_part_bytes(int B, int T, int H, int dv, int W, int R, int slice_cols) {
    return (size_t)B * T * H * ((dv + slice_cols - 1) / slice_cols) * (2 + W + R) * sizeof(float);
}

hipError_t launch_sdm_bwd_reduce(const SdmBwdArgs& a, int slice_cols, hipStream_t st) {
    const long long total = (long long)a.B * a.T * a.H * (2 + a.W + a.R);
    const int nslice = (a.dv + slice_cols - 1) / slice_cols;
    sdm_bwd_reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(a, total, nslice);
    return hipGetLastError();
}

hipError_t launch_sdm_update_backward(const SdmBwdArgs& a, hipStream_t st) {
    if (a.T <= 0 || a.B <= 0) return hipSuccess;
    const int rows = a.W > a.R ? a.W : a.R;
    int NL = 1;
    while (4 * NL < rows) NL <<= 1;
    const int nslice = (a.dv + kCols - 1) / kCols;
    dim3 grid((unsigned)(a.B * a.H * nslice));
    hipError_t e = a.dtype == 0 ? dispatch_bwd<float>(NL, grid, st, a)
                                : dispatch_bwd<bf16_t>(NL, grid, st, a);
    if (e != hipSuccess) return e;
    return launch_sdm_bwd_reduce(a, kCols, st);
}

hipError_t launch_sdm_address_backward(int P, int sqrtN, int budget, const int32_t* idx,
                                       const float* wt, const float* dwt, float* ds1, float* ds2,
                                       hipStream_t st) {
    if (P <= 0) return hipSuccess;
    if (budget < 1 || budget > kMaxBudget || sqrtN < 1) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((P + kAbWaves - 1) / kAbWaves);
    if (sqrtN <= kAbMaxN && budget <= 64) {
        const AbSet one{idx, wt, dwt, ds1, ds2, budget};
        sdm_address_bwd_small_kernel<<<grid, 64 * kAbWaves, 0, st>>>(AbPair{{one, one}, P, sqrtN, (int)grid});
    } else
        sdm_address_bwd_kernel<<<grid, 64 * kAbWaves, 0, st>>>(P, sqrtN, budget, idx, wt, dwt, ds1,
                                                               ds2);
    return hipGetLastError();
}

hipError_t launch_sdm_address_backward_pair(int P, int sqrtN, int W, const int32_t* idx_w,
                                            const float* wt_w, const float* dwt_w, float* dsw1,
                                            float* dsw2, int R, const int32_t* idx_r,
                                            const float* wt_r, const float* dwt_r, float* dsr1,
                                            float* dsr2, hipStream_t st) {
    if (P <= 0) return hipSuccess;
    if (sqrtN > kAbMaxN || W > 64 || R > 64) {  // the looped kernel, one launch per set
        const hipError_t e =
            launch_sdm_address_backward(P, sqrtN, W, idx_w, wt_w, dwt_w, dsw1, dsw2, st);
        if (e != hipSuccess) return e;
        return launch_sdm_address_backward(P, sqrtN, R, idx_r, wt_r, dwt_r, dsr1, dsr2, st);
    }
    if (W < 1 || R < 1 || sqrtN < 1) return hipErrorInvalidValue;
    const int nblk = (P + kAbWaves - 1) / kAbWaves;
    const AbPair ab{{AbSet{idx_w, wt_w, dwt_w, dsw1, dsw2, W}, AbSet{idx_r, wt_r, dwt_r, dsr1, dsr2, R}},
                    P, sqrtN, nblk};
    sdm_address_bwd_small_kernel<<<(unsigned)(2 * nblk), 64 * kAbWaves, 0, st>>>(ab);
    return hipGetLastError();
}

}  // namespace sslp
