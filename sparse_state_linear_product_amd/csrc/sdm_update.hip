// K2: the Sparse Delta Memory recurrence given the addressing.
//
// Slides "Sparse Delta Memory: Scaling the State of Linear RNNs through
// Sparsity": "Selected slots decay and update; other slots persist"
// (Eqs. (3)-(5): decay only the selected write slots, delta update, read y_t
// from the updated table) and "A v1 inconsistency matters for reproducing the
// update" (shared prediction v_hat = sum_i k^(i) M~[i] vs Eq. (4)'s per-slot
// residual).
//
// Given the addressing every operation acts on one value column at a time, so
// the d_v columns are independent recurrences.  One wavefront owns a
// 16-column slice (64 B row segments) of one (batch, head) table and walks
// the tokens in order.  Lane (g, c), g = lane / 16, c = lane % 16, handles
// column c of the write rows n = g, g+4, ... and read rows m = g, g+4, ...;
// row sums are reduced across the four lane groups with two shuffles.
//
// Each token makes one trip to the table: its write and read rows are
// requested together, while the next token's gates, indices and weights are
// already in flight.  A read slot that the token also writes takes the
// updated value from LDS (write slots are distinct within a token).
// Ordering: every store to the table and every later load of the same row
// are issued by the same wavefront, whose memory operations complete in
// program order, so token t+1 observes token t's writes without a wait.
//
// For training, the kernel can also store each token's write rows as they were
// before the token (the sparse update information from which a backward sweep
// undoes the writes, Sparse Delta Memory slides, backup "Backup: undoing
// writes avoids repeated full-table snapshots").
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

constexpr int kCols = 16;  // columns per wavefront

// What a token needs that does not depend on the table (gates, v, indices and
// weights), loaded one token ahead from clamped (always valid) addresses;
// rows past W or R and columns past d_v are masked where the values are used,
// so no load waits on a condition.
template <int NL>
struct FwdMeta {
    float al, be, vc;
    int sw[NL], sr[NL];
    float w[NL], e[NL];
};

template <typename io_t, int NL>
SSLP_DEVICE void load_fwd_meta(FwdMeta<NL>& m, const SdmUpdateArgs& a, size_t bth, int g,
                               int colc) {
    m.al = a.alpha[bth];
    m.be = a.beta[bth];
    m.vc = to_f32(static_cast<const io_t*>(a.v)[bth * a.dv + colc]);
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int nw = min(g + 4 * r, a.W - 1), nr = min(g + 4 * r, a.R - 1);
        m.sw[r] = a.idx_w[bth * a.W + nw];  // range-checked where used (keep_slot)
        m.w[r] = a.wt_w[bth * a.W + nw];
        m.sr[r] = a.idx_r[bth * a.R + nr];
        m.e[r] = a.wt_r[bth * a.R + nr];
    }
}

template <typename io_t, int NL>
__global__ __launch_bounds__(64) void sdm_update_kernel(SdmUpdateArgs a) {
    __shared__ int s_ws[4 * NL];             // the token's write slots
    __shared__ float s_new[4 * NL][kCols];   // their updated values, this slice's columns
    const int nslice = (a.dv + kCols - 1) / kCols;
    const int slice = blockIdx.x % nslice;
    const int bh = blockIdx.x / nslice;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int lane = threadIdx.x;
    const int g = lane >> 4, c = lane & 15;
    const int col = slice * kCols + c;
    const bool colok = col < a.dv;
    const int colc = colok ? col : a.dv - 1;
    const int W = a.W, R = a.R;
    float* tab = a.M + ((size_t)b * a.H + h) * (size_t)a.N * a.dv;
    io_t* yout = static_cast<io_t*>(a.y);

    FwdMeta<NL> cur;
    bool bad = false;  // a slot index outside [0, N) was seen (and replaced by 0)
    if (a.T > 0) load_fwd_meta<io_t, NL>(cur, a, ((size_t)b * a.T) * a.H + h, g, colc);
    for (int t = 0; t < a.T; ++t) {
        const size_t bth = ((size_t)b * a.T + t) * a.H + h;
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            cur.sw[r] = keep_slot(cur.sw[r], a.N, bad);
            cur.sr[r] = keep_slot(cur.sr[r], a.N, bad);
        }
        // ---- one trip for the write and the read rows ----
        float m0[NL], mr[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            m0[r] = tab[(size_t)cur.sw[r] * a.dv + colc];
            mr[r] = tab[(size_t)cur.sr[r] * a.dv + colc];
        }
        FwdMeta<NL> nxt;
        load_fwd_meta<io_t, NL>(nxt, a, ((size_t)b * a.T + (t + 1 < a.T ? t + 1 : t)) * a.H + h,
                                g, colc);
        const float al = cur.al, be = cur.be, vc = colok ? cur.vc : 0.f;
        // ---- decay the write rows (Eq. 3) and update them (Eq. 4 / figure form) ----
        float mt[NL], w[NL], nv[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const bool live = g + 4 * r < W && colok;
            w[r] = g + 4 * r < W ? cur.w[r] : 0.f;
            if (a.saved != nullptr && live) a.saved[(bth * W + g + 4 * r) * a.dv + col] = m0[r];
            mt[r] = live ? al * m0[r] : 0.f;
        }
        if (a.residual_mode == 0) {
            // shared prediction v_hat = sum_n wt_n M~[i_n]
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < NL; ++r) acc = fmaf(w[r], mt[r], acc);
            acc += xor_lane_f(acc, 16, lane_id());
            acc += xor_lane_f(acc, 32, lane_id());
            const float res = vc - acc;
#pragma unroll
            for (int r = 0; r < NL; ++r) nv[r] = fmaf(be * w[r], res, mt[r]);
        } else {
            // per-slot residual v - M~[i] (Eq. 4 as printed)
#pragma unroll
            for (int r = 0; r < NL; ++r) nv[r] = fmaf(be * w[r], vc - mt[r], mt[r]);
        }
#pragma unroll
        for (int r = 0; r < NL; ++r)
            if (g + 4 * r < W && colok) tab[(size_t)cur.sw[r] * a.dv + col] = nv[r];
        // ---- read after writing (Eq. 5): a read slot that this token writes
        //      takes the updated value.  Lane (g, c) checks its read rows
        //      against write rows c, c + 16, ...; the row group combines ----
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            if (g + 4 * r < W) s_new[g + 4 * r][c] = nv[r];
            if (c == 0 && g + 4 * r < W) s_ws[g + 4 * r] = cur.sw[r];
        }
        wave_sync();
        int hit[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) hit[r] = 0;
#pragma unroll
        for (int j = 0; j < (4 * NL + 15) / 16; ++j) {
            const int n = c + 16 * j;
            if (n < W) {
                const int sn = s_ws[n];
#pragma unroll
                for (int r = 0; r < NL; ++r) hit[r] = sn == cur.sr[r] ? n + 1 : hit[r];
            }
        }
#pragma unroll
        for (int s = 1; s < 16; s <<= 1)
#pragma unroll
            for (int r = 0; r < NL; ++r) hit[r] = max(hit[r], xor_lane_i(hit[r], s, lane_id()));
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            if (g + 4 * r < R) {
                const float m = hit[r] > 0 ? s_new[hit[r] - 1][c] : mr[r];
                acc = fmaf(cur.e[r], m, acc);
            }
        }
        acc += xor_lane_f(acc, 16, lane_id());
        acc += xor_lane_f(acc, 32, lane_id());
        if (g == 0 && colok) yout[bth * a.dv + col] = from_f32<io_t>(acc);
        wave_sync();
        cur = nxt;
    }
    report_slot_error(bad, a.err);
}

// ---------------------------------------------------------------------------
// One token per sequence (a decode step).  One workgroup of 4 wavefronts per
// (batch, head, 256 columns): lane l holds columns 4l .. 4l+3 of a row, so a
// wavefront moves a row piece of up to 1 KB in one contiguous access.  Wave w
// takes write rows w, w+4, ... and read rows w, w+4, ...; all of them are
// loaded at once.  The read-after-write needs no second trip to memory: a read
// slot that this token writes takes its updated value from LDS (write slots
// are distinct within a token), any other read slot its loaded value.
// ---------------------------------------------------------------------------
constexpr int kDecCols = 256;  // columns per workgroup
constexpr int kDecMaxRows = 64;  // W, R <= 64

template <typename io_t, int NL>
__global__ __launch_bounds__(256) void sdm_decode_update_kernel(SdmUpdateArgs a) {
    __shared__ float4 s_new[kDecMaxRows][64];  // updated write rows (this workgroup's columns)
    __shared__ float4 s_part[4][64];           // per-wave partial sums
    __shared__ int s_wslot[kDecMaxRows];
    const int nslice = (a.dv + kDecCols - 1) / kDecCols;
    const int slice = blockIdx.x % nslice;
    const int bh = blockIdx.x / nslice;  // = b * H + h (T = 1)
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = slice * kDecCols + 4 * lane;
    const bool colok = col < a.dv;  // dv % 4 == 0: a lane's 4 columns are all in or all out
    const int W = a.W, R = a.R;
    const float* tab = a.M + (size_t)bh * (size_t)a.N * a.dv;
    float* tabw = a.M + (size_t)bh * (size_t)a.N * a.dv;
    const float al = a.alpha[bh], be = a.beta[bh];

    // gather the write rows and the read rows of this wave
    bool bad = false;  // a slot index outside [0, N) was seen (and replaced by 0)
    int ws[NL], rs[NL];
    float ww[NL], wr[NL];
    float4 mw[NL], mr[NL];
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + 4 * r;
        const bool okw = n < W, okr = n < R;
        ws[r] = okw ? keep_slot(a.idx_w[(size_t)bh * W + n], a.N, bad) : 0;
        ww[r] = okw ? a.wt_w[(size_t)bh * W + n] : 0.f;
        rs[r] = okr ? keep_slot(a.idx_r[(size_t)bh * R + n], a.N, bad) : -1;
        wr[r] = okr ? a.wt_r[(size_t)bh * R + n] : 0.f;
        if (okw && threadIdx.x % 64 == 0) s_wslot[n] = ws[r];
    }
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + 4 * r;
        mw[r] = (n < W && colok) ? *reinterpret_cast<const float4*>(tab + (size_t)ws[r] * a.dv + col) : z4;
        mr[r] = (n < R && colok) ? *reinterpret_cast<const float4*>(tab + (size_t)rs[r] * a.dv + col) : z4;
    }
    float4 vc = z4;
    if (colok) {
        const io_t* vin = static_cast<const io_t*>(a.v) + (size_t)bh * a.dv + col;
        vc = make_float4(to_f32(vin[0]), to_f32(vin[1]), to_f32(vin[2]), to_f32(vin[3]));
    }
    // decay (Eq. 3) and the shared prediction v_hat = sum_n wt_n M~[i_n]
    float4 acc = z4;
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        mw[r].x *= al;
        mw[r].y *= al;
        mw[r].z *= al;
        mw[r].w *= al;
        acc.x = fmaf(ww[r], mw[r].x, acc.x);
        acc.y = fmaf(ww[r], mw[r].y, acc.y);
        acc.z = fmaf(ww[r], mw[r].z, acc.z);
        acc.w = fmaf(ww[r], mw[r].w, acc.w);
    }
    s_part[w][lane] = acc;
    __syncthreads();
    float4 vh = z4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float4 pu = s_part[u][lane];
        vh.x += pu.x;
        vh.y += pu.y;
        vh.z += pu.z;
        vh.w += pu.w;
    }
    // delta update of the write rows (shared residual, or Eq. 4's per-slot one)
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + 4 * r;
        if (n < W) {
            float4 res;
            if (a.residual_mode == 0) {
                res = make_float4(vc.x - vh.x, vc.y - vh.y, vc.z - vh.z, vc.w - vh.w);
            } else {
                res = make_float4(vc.x - mw[r].x, vc.y - mw[r].y, vc.z - mw[r].z, vc.w - mw[r].w);
            }
            const float c = be * ww[r];
            float4 nv;
            nv.x = fmaf(c, res.x, mw[r].x);
            nv.y = fmaf(c, res.y, mw[r].y);
            nv.z = fmaf(c, res.z, mw[r].z);
            nv.w = fmaf(c, res.w, mw[r].w);
            s_new[n][lane] = nv;
            if (colok) *reinterpret_cast<float4*>(tabw + (size_t)ws[r] * a.dv + col) = nv;
        }
    }
    __syncthreads();
    // read after writing (Eq. 5); lane q < W compares write slot q with the read
    // slot, so each read row finds the write row holding its slot in one step
    const int myw = lane < W ? s_wslot[lane] : -2;
    float4 y = z4;
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + 4 * r;
        if (n < R) {
            float4 m = mr[r];
            const unsigned long long hit = __ballot(myw == rs[r]);
            if (hit) m = s_new[__ffsll((long long)hit) - 1][lane];
            y.x = fmaf(wr[r], m.x, y.x);
            y.y = fmaf(wr[r], m.y, y.y);
            y.z = fmaf(wr[r], m.z, y.z);
            y.w = fmaf(wr[r], m.w, y.w);
        }
    }
    s_part[w][lane] = y;
    __syncthreads();
    if (w == 0 && colok) {
        float4 t = z4;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 pu = s_part[u][lane];
            t.x += pu.x;
            t.y += pu.y;
            t.z += pu.z;
            t.w += pu.w;
        }
        io_t* yo = static_cast<io_t*>(a.y) + (size_t)bh * a.dv + col;
        yo[0] = from_f32<io_t>(t.x);
        yo[1] = from_f32<io_t>(t.y);
        yo[2] = from_f32<io_t>(t.z);
        yo[3] = from_f32<io_t>(t.w);
    }
    report_slot_error(bad, a.err);
}

template <typename io_t>
hipError_t dispatch_nl(int NL, dim3 grid, hipStream_t st, const SdmUpdateArgs& a) {
    switch (NL) {
        case 1: sdm_update_kernel<io_t, 1><<<grid, 64, 0, st>>>(a); break;
        case 2: sdm_update_kernel<io_t, 2><<<grid, 64, 0, st>>>(a); break;
        case 4: sdm_update_kernel<io_t, 4><<<grid, 64, 0, st>>>(a); break;
        case 8: sdm_update_kernel<io_t, 8><<<grid, 64, 0, st>>>(a); break;
        case 16: sdm_update_kernel<io_t, 16><<<grid, 64, 0, st>>>(a); break;
        case 32: sdm_update_kernel<io_t, 32><<<grid, 64, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sdm_update(const SdmUpdateArgs& a, hipStream_t st) {
    if (a.T <= 0 || a.B <= 0) return hipSuccess;
    if (a.T == 1 && a.saved == nullptr && a.dv % 4 == 0 && a.W <= kDecMaxRows &&
        a.R <= kDecMaxRows) {
        const int nslice = (a.dv + kDecCols - 1) / kDecCols;
        dim3 grid((unsigned)(a.B * a.H * nslice));
        const int rows = a.W > a.R ? a.W : a.R;
        const bool f32 = a.dtype == 0;
        if (rows <= 16) {
            if (f32) sdm_decode_update_kernel<float, 4><<<grid, 256, 0, st>>>(a);
            else sdm_decode_update_kernel<bf16_t, 4><<<grid, 256, 0, st>>>(a);
        } else if (rows <= 32) {
            if (f32) sdm_decode_update_kernel<float, 8><<<grid, 256, 0, st>>>(a);
            else sdm_decode_update_kernel<bf16_t, 8><<<grid, 256, 0, st>>>(a);
        } else {
            if (f32) sdm_decode_update_kernel<float, 16><<<grid, 256, 0, st>>>(a);
            else sdm_decode_update_kernel<bf16_t, 16><<<grid, 256, 0, st>>>(a);
        }
        return hipGetLastError();
    }
    const int rows = (a.W > a.R ? a.W : a.R);
    int NL = 1;
    while (4 * NL < rows) NL <<= 1;
    const int nslice = (a.dv + kCols - 1) / kCols;
    dim3 grid((unsigned)(a.B * a.H * nslice));
    if (a.dtype == 0) return dispatch_nl<float>(NL, grid, st, a);
    return dispatch_nl<bf16_t>(NL, grid, st, a);
}

}  // namespace sslp
