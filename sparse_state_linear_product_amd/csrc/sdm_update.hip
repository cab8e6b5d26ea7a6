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
            mt[r] = (ok && colok) ? al * tab[(size_t)slot[r] * a.dv + col] : 0.f;
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
    const int rows = (a.W > a.R ? a.W : a.R);
    int NL = 1;
    while (4 * NL < rows) NL <<= 1;
    const int nslice = (a.dv + kCols - 1) / kCols;
    dim3 grid((unsigned)(a.B * a.H * nslice));
    if (a.dtype == 0) return dispatch_nl<float>(NL, grid, st, a);
    return dispatch_nl<bf16_t>(NL, grid, st, a);
}

}  // namespace sslp
