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
// Ordering: every store to the table and every later load of the same row
// are issued by the same wavefront, whose memory operations complete in
// program order, so token t+1 (and the read-after-write of token t) observe
// token t's writes without a wait.
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

template <typename io_t, int NL>
__global__ __launch_bounds__(64) void sdm_update_kernel(SdmUpdateArgs a) {
    const int nslice = (a.dv + kCols - 1) / kCols;
    const int slice = blockIdx.x % nslice;
    const int bh = blockIdx.x / nslice;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int lane = threadIdx.x;
    const int g = lane >> 4;
    const int col = slice * kCols + (lane & 15);
    const bool colok = col < a.dv;
    const int W = a.W, R = a.R;
    float* tab = a.M + ((size_t)b * a.H + h) * (size_t)a.N * a.dv;
    const io_t* vin = static_cast<const io_t*>(a.v);
    io_t* yout = static_cast<io_t*>(a.y);

    for (int t = 0; t < a.T; ++t) {
        const size_t bth = ((size_t)b * a.T + t) * a.H + h;
        const float al = a.alpha[bth];
        const float be = a.beta[bth];
        // gather the write rows and decay them (Eq. 3)
        float mt[NL], w[NL];
        int slot[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const int n = g + 4 * r;
            const bool ok = n < W;
            slot[r] = ok ? a.idx_w[bth * W + n] : 0;
            w[r] = ok ? a.wt_w[bth * W + n] : 0.f;
            const float m0 = (ok && colok) ? tab[(size_t)slot[r] * a.dv + col] : 0.f;
            if (a.saved != nullptr && ok && colok) a.saved[(bth * W + n) * a.dv + col] = m0;
            mt[r] = al * m0;
        }
        const float vc = colok ? to_f32(vin[bth * a.dv + col]) : 0.f;
        if (a.residual_mode == 0) {
            // shared prediction v_hat = sum_n wt_n M~[i_n]
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < NL; ++r) acc = fmaf(w[r], mt[r], acc);
            acc += __shfl_xor(acc, 16, 64);
            acc += __shfl_xor(acc, 32, 64);
            const float res = vc - acc;
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                const int n = g + 4 * r;
                if (n < W && colok)
                    tab[(size_t)slot[r] * a.dv + col] = fmaf(be * w[r], res, mt[r]);
            }
        } else {
            // per-slot residual v - M~[i] (Eq. 4 as printed)
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                const int n = g + 4 * r;
                if (n < W && colok)
                    tab[(size_t)slot[r] * a.dv + col] = fmaf(be * w[r], vc - mt[r], mt[r]);
            }
        }
        wave_sync();
        // read after writing (Eq. 5)
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const int m = g + 4 * r;
            if (m < R) {
                const int s = a.idx_r[bth * R + m];
                const float wr = a.wt_r[bth * R + m];
                if (colok) acc = fmaf(wr, tab[(size_t)s * a.dv + col], acc);
            }
        }
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        if (g == 0 && colok) yout[bth * a.dv + col] = from_f32<io_t>(acc);
        wave_sync();
    }
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
    int ws[NL], rs[NL];
    float ww[NL], wr[NL];
    float4 mw[NL], mr[NL];
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + 4 * r;
        const bool okw = n < W, okr = n < R;
        ws[r] = okw ? a.idx_w[(size_t)bh * W + n] : 0;
        ww[r] = okw ? a.wt_w[(size_t)bh * W + n] : 0.f;
        rs[r] = okr ? a.idx_r[(size_t)bh * R + n] : -1;
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
