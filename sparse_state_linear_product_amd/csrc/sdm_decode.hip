// The SDM decode step in one launch: product-key addressing of the token's
// write and read sets, then the sparse decay / delta update / read of its
// sequence's table (slides "Sparse Delta Memory: Scaling the State of Linear
// RNNs through Sparsity": "Product keys select addresses without scoring every
// slot", "Selected slots decay and update; other slots persist" Eqs. (3)-(5),
// and the figure-form or per-slot residual of "A v1 inconsistency matters for
// reproducing the update").
//
// One workgroup of 512 threads per (sequence, head, 256 columns of d_v).  The
// first 256 threads address the write set and the other 256 the read set (the
// steps of addr_wg.h, both groups in step at every barrier); every workgroup
// of a (sequence, head) repeats this small computation, which costs less than
// a second launch and a round trip of the indices through memory.  The
// selected slots and weights stay in LDS, and the 8 wavefronts then gather
// the write and read rows of their 256 columns (lane l: columns 4l .. 4l+3, so
// a wavefront moves a 1 KB row piece in one access), update the write rows and
// read the read rows after the write; a read slot that the token writes takes
// its updated value from LDS (write slots are distinct within a token).  The
// barriers wait for LDS operations only, so the table stores stay in flight.
#include "addr_wg.h"
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

typedef float f32v4 __attribute__((ext_vector_type(4)));

constexpr int kCols = 256;    // columns per workgroup
constexpr int kWaves = 8;     // wavefronts per workgroup
constexpr int kMaxRows = 64;  // W, R <= 64

// LDS of one workgroup, sized for at most 8 NL rows per set and a per-half
// top-k of at most KMAX (the rare path ranks all k^2 candidates): 41 KB at
// the 1.4B-layer shape (k = W = R = 32)
template <int NL, int KMAX>
struct DecSmem {
    static constexpr int kRows = kWaves * NL;
    static constexpr int kCand = KMAX * KMAX > kAddrGroup ? KMAX * KMAX : kAddrGroup;
    struct Upd {
        float4 nw[kRows][64];     // updated write rows, this workgroup's columns
        float4 part[kWaves][64];  // per-wave partial sums
    };
    // the addressing scratch of both sets, reused by the update once the
    // selections sit in idx / wt
    union {
        WgAddrSmemT<kCand> addr[2];
        Upd upd;
    };
    int idx[2][kRows];
    float wt[2][kRows];
};

template <typename io_t, int NL, int KMAX>
__global__ __launch_bounds__(64 * kWaves) void sdm_decode_fused_kernel(SdmDecodeArgs a) {
    __shared__ DecSmem<NL, KMAX> sm;
    auto& s_idx = sm.idx;
    auto& s_wt = sm.wt;
    const int t = threadIdx.x, grp = t >> 8, tt = t & 255;
    const int nblk = (a.dv + kCols - 1) / kCols;
    const int slice = blockIdx.x % nblk;
    const int p = blockIdx.x / nblk;  // = b * H + h

    // ---- addressing: group 0 the write set, group 1 the read set ----
    auto* sma = sm.addr;
    const size_t soff = (size_t)p * a.sqrtN;
    const WgAddrProblem pr{static_cast<const io_t*>(a.s1[grp]) + soff,
                           static_cast<const io_t*>(a.s2[grp]) + soff, a.sqrtN, a.k[grp],
                           a.budget[grp], a.nD[grp]};
    const bool first = slice == 0;
    int32_t* gi = first && a.idx[grp] ? a.idx[grp] + (size_t)p * pr.budget : nullptr;
    float* gw = first && a.wt[grp] ? a.wt[grp] + (size_t)p * pr.budget : nullptr;
    wg_addr_select<io_t>(pr, tt, sma[grp], s_idx[grp], s_wt[grp], gi, gw);
    // both groups take the rare path together, so their barriers stay matched
    // (a group whose common path already wrote its selection writes it again)
    if (sma[0].F != a.budget[0] || sma[1].F != a.budget[1]) {
        wg_addr_rank_all(pr, tt, sma[grp]);
        wg_addr_softmax(pr, tt, sma[grp], s_idx[grp], s_wt[grp], gi, gw);
        block_sync_lds();
    }

    // ---- the update and the read of this workgroup's columns ----
    auto& su = sm.upd;
    const int lane = t & 63, w = t >> 6;
    const int col = slice * kCols + 4 * lane;
    const bool colok = col < a.dv;  // dv % 4 == 0: a lane's 4 columns are all in or all out
    const int W = a.budget[0], R = a.budget[1];
    float* tab = a.M + (size_t)p * (size_t)a.N * a.dv;
    const float al = a.alpha[p], be = a.beta[p];
    int ws[NL], rs[NL];
    float ww[NL], wr[NL];
    float4 mw[NL], mr[NL];
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + kWaves * r;
        const bool okw = n < W, okr = n < R;
        ws[r] = okw ? s_idx[0][n] : 0;
        ww[r] = okw ? s_wt[0][n] : 0.f;
        rs[r] = okr ? s_idx[1][n] : -1;
        wr[r] = okr ? s_wt[1][n] : 0.f;
    }
    // every load is issued from a valid address (row 0, the last 4 columns)
    // and masked afterwards, so that none of them waits on a condition
    const int cc = colok ? col : a.dv - 4;
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        mw[r] = *reinterpret_cast<const float4*>(tab + (size_t)ws[r] * a.dv + cc);
        mr[r] = *reinterpret_cast<const float4*>(tab + (size_t)(rs[r] < 0 ? 0 : rs[r]) * a.dv + cc);
    }
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + kWaves * r;
        if (!(n < W && colok)) mw[r] = z4;
        if (!(n < R && colok)) mr[r] = z4;
    }
    float4 vc = z4;
    if (colok) {
        const io_t* vin = static_cast<const io_t*>(a.v) + (size_t)p * a.dv + col;
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
    su.part[w][lane] = acc;
    block_sync_lds();
    float4 vh = z4;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
        const float4 pu = su.part[u][lane];
        vh.x += pu.x;
        vh.y += pu.y;
        vh.z += pu.z;
        vh.w += pu.w;
    }
    // delta update of the write rows (shared residual, or Eq. 4's per-slot one)
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + kWaves * r;
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
            su.nw[n][lane] = nv;
            // a streaming store: the step does not read the row from memory again
            if (colok)
                __builtin_nontemporal_store(f32v4{nv.x, nv.y, nv.z, nv.w},
                                            reinterpret_cast<f32v4*>(tab + (size_t)ws[r] * a.dv + col));
        }
    }
    block_sync_lds();
    // read after writing (Eq. 5): lane q < W holds write slot q, so each read
    // row finds the write row holding its slot with one ballot
    const int myw = lane < W ? s_idx[0][lane] : -2;
    float4 y = z4;
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int n = w + kWaves * r;
        if (n < R) {
            float4 m = mr[r];
            const unsigned long long hit = __ballot(myw == rs[r]);
            if (hit) m = su.nw[__ffsll((long long)hit) - 1][lane];
            y.x = fmaf(wr[r], m.x, y.x);
            y.y = fmaf(wr[r], m.y, y.y);
            y.z = fmaf(wr[r], m.z, y.z);
            y.w = fmaf(wr[r], m.w, y.w);
        }
    }
    su.part[w][lane] = y;  // every wave read v_hat from su.part before the last barrier
    block_sync_lds();
    if (w == 0 && colok) {
        float4 s = z4;
#pragma unroll
        for (int u = 0; u < kWaves; ++u) {
            const float4 pu = su.part[u][lane];
            s.x += pu.x;
            s.y += pu.y;
            s.z += pu.z;
            s.w += pu.w;
        }
        io_t* yo = static_cast<io_t*>(a.y) + (size_t)p * a.dv + col;
        yo[0] = from_f32<io_t>(s.x);
        yo[1] = from_f32<io_t>(s.y);
        yo[2] = from_f32<io_t>(s.z);
        yo[3] = from_f32<io_t>(s.w);
    }
}

template <typename io_t, int KMAX>
hipError_t dispatch_rows(int rows, unsigned grid, hipStream_t st, const SdmDecodeArgs& a) {
    if (rows <= 8) sdm_decode_fused_kernel<io_t, 1, KMAX><<<grid, 64 * kWaves, 0, st>>>(a);
    else if (rows <= 16) sdm_decode_fused_kernel<io_t, 2, KMAX><<<grid, 64 * kWaves, 0, st>>>(a);
    else if (rows <= 32) sdm_decode_fused_kernel<io_t, 4, KMAX><<<grid, 64 * kWaves, 0, st>>>(a);
    else sdm_decode_fused_kernel<io_t, 8, KMAX><<<grid, 64 * kWaves, 0, st>>>(a);
    return hipGetLastError();
}

template <typename io_t>
hipError_t dispatch_k(int kmax, int rows, unsigned grid, hipStream_t st, const SdmDecodeArgs& a) {
    if (kmax <= 32) return dispatch_rows<io_t, 32>(rows, grid, st, a);
    return dispatch_rows<io_t, 64>(rows, grid, st, a);
}

}  // namespace

bool sdm_decode_fused_fits(int sqrtN, int dv, int k_w, int W, int k_r, int R) {
    return dv % 4 == 0 && W <= kMaxRows && R <= kMaxRows && wg_address_fits(sqrtN, k_w, W) &&
           wg_address_fits(sqrtN, k_r, R);
}

hipError_t launch_sdm_decode_fused(SdmDecodeArgs a, hipStream_t st) {
    if (a.P <= 0) return hipSuccess;
    if (a.sqrtN < 1 || a.dv < 4 || a.dv % 4 != 0 || a.budget[0] > kMaxRows ||
        a.budget[1] > kMaxRows)
        return hipErrorInvalidValue;
    a.nD[0] = address_set_size_host(a.k[0], a.budget[0]);
    a.nD[1] = address_set_size_host(a.k[1], a.budget[1]);
    const long long grid = (long long)a.P * ((a.dv + kCols - 1) / kCols);
    if (grid > 0x7fffffffll) return hipErrorInvalidValue;
    const int rows = a.budget[0] > a.budget[1] ? a.budget[0] : a.budget[1];
    const int kmax = a.k[0] > a.k[1] ? a.k[0] : a.k[1];
    if (a.dtype == 0) return dispatch_k<float>(kmax, rows, (unsigned)grid, st, a);
    return dispatch_k<bf16_t>(kmax, rows, (unsigned)grid, st, a);
}

}  // namespace sslp
