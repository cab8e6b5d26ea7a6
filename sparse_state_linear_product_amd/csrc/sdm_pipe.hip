// K2 (pipelined): the Sparse Delta Memory recurrence given the addressing,
// with the table rows of future tokens prefetched far ahead of their use.
//
// Same arithmetic as the per-token kernel in sdm_update.hip (slides "Sparse
// Delta Memory: Scaling the State of Linear RNNs through Sparsity", Eqs.
// (3)-(5) and the shared-prediction figure form); only the schedule differs.
//
// Why: the recurrence of one value column is a chain over all T tokens, so the
// table traffic of a wavefront is latency-bound unless the rows of token t+D
// are in flight while token t is computed.  The addressing of every token is
// known before the recurrence starts, so the rows can be requested early; a
// row requested early is stale only if a token in between writes it.
//
// Two kernels:
//  * sdm_records_kernel (one wavefront per token): packs, per token, the byte
//    offsets, weights and a FORWARD code of each selected row into a record.
//    The forward code names the latest writer (t', n') of the same slot among
//    the D-1 preceding tokens (and the token itself for reads), i.e. the
//    writes a load issued D tokens early cannot have observed; -1 otherwise.
//  * sdm_update_pipe_kernel (one wavefront per 8-column slice of a head): walks
//    the tokens; rows of token t+D are loaded into registers right after token
//    t has stored its writes; forwarded rows are taken from an LDS ring that
//    holds the values written by the last D tokens.  Records reach LDS two
//    blocks of D tokens ahead of use.
// Lane (g, c), g = lane/8, c = lane%8, owns column c of write rows n = g + 8r
// and read rows m = g + 8r; row sums are reduced over the 8 lane groups.
// Eight-column slices use 32-byte row segments; workgroups are mapped so that
// the 16 slices sharing 512 bytes of a row run on the same XCD (its L2 merges
// the segments).
//
// Ordering: all table stores and loads of a column slice come from one
// wavefront, whose memory operations complete in program order, so a load
// issued after a store to the same address observes it.
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

constexpr int CW = 8;  // columns per wavefront
constexpr int G = 8;   // lane groups (rows are dealt round-robin to them)

// record layout, in 32-bit words, for one token: for each lane group g the
// block [woff x NWG][wwt x NWG][wfwd x NWG][roff x NRG][rwt x NRG][rfwd x NRG],
// then a 4-word header (alpha, beta, flags, pad)
template <int NWG, int NRG>
struct Rec {
    static constexpr int GW = 3 * NWG + 3 * NRG;  // words per group
    static constexpr int HDR = G * GW;            // header offset
    static constexpr int WORDS = HDR + 4;
};
constexpr uint32_t FLAG_WFWD = 1u, FLAG_RFWD = 2u;

struct RecArgs {
    int B, T, H, N, dv, W, R, D;
    const int32_t* idx_w;
    const float* wt_w;
    const int32_t* idx_r;
    const float* wt_r;
    const float* alpha;
    const float* beta;
    uint32_t* rec;  // [B, H, T, WORDS]
};

template <int NWG, int NRG>
__global__ __launch_bounds__(256) void sdm_records_kernel(RecArgs a) {
    using RC = Rec<NWG, NRG>;
    constexpr int W = NWG * G, R = NRG * G;
    constexpr int MAXD = 16;
    __shared__ int32_t win[4][MAXD][W];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long p = (long long)blockIdx.x * 4 + wv;  // (b, t, h) in [B,T,H] order
    if (p >= (long long)a.B * a.T * a.H) return;
    const int h = (int)(p % a.H);
    const int t = (int)((p / a.H) % a.T);
    const int b = (int)(p / ((long long)a.H * a.T));
    const int D = a.D;
    const int tlo = t - D + 1 > 0 ? t - D + 1 : 0;
    const int nt = t - tlo + 1;  // window tokens tlo..t
    for (int e = lane; e < nt * W; e += 64) {
        const int tt = tlo + e / W, n = e - (e / W) * W;
        win[wv][e / W][n] = a.idx_w[(((size_t)b * a.T + tt) * a.H + h) * W + n];
    }
    wave_sync();
    const size_t bth = ((size_t)b * a.T + t) * a.H + h;
    uint32_t* out = a.rec + (((size_t)b * a.H + h) * a.T + t) * RC::WORDS;
    bool wf = false, rf = false;
    for (int x = lane; x < W + R; x += 64) {
        const bool isw = x < W;
        const int n = isw ? x : x - W;
        const int slot = isw ? a.idx_w[bth * W + n] : a.idx_r[bth * R + n];
        const float wt = isw ? a.wt_w[bth * W + n] : a.wt_r[bth * R + n];
        int fwd = -1;
        for (int tt = isw ? t - 1 : t; tt >= tlo && fwd < 0; --tt) {
            for (int n2 = 0; n2 < W; ++n2)
                if (win[wv][tt - tlo][n2] == slot) {
                    fwd = (tt % D) * W + n2;
                    break;
                }
        }
        const int g = n % G, r = n / G;
        uint32_t* grp = out + g * RC::GW;
        const uint32_t off = (uint32_t)slot * (uint32_t)a.dv * 4u;
        if (isw) {
            grp[r] = off;
            grp[NWG + r] = __float_as_uint(wt);
            grp[2 * NWG + r] = (uint32_t)fwd;
            wf |= fwd >= 0;
        } else {
            grp[3 * NWG + r] = off;
            grp[3 * NWG + NRG + r] = __float_as_uint(wt);
            grp[3 * NWG + 2 * NRG + r] = (uint32_t)fwd;
            rf |= fwd >= 0;
        }
    }
    const bool anyw = __ballot(wf) != 0ull, anyr = __ballot(rf) != 0ull;
    if (lane == 0) {
        out[RC::HDR + 0] = __float_as_uint(a.alpha[bth]);
        out[RC::HDR + 1] = __float_as_uint(a.beta[bth]);
        out[RC::HDR + 2] = (anyw ? FLAG_WFWD : 0u) | (anyr ? FLAG_RFWD : 0u);
        out[RC::HDR + 3] = 0u;
    }
}

template <typename io_t, int NWG, int NRG, int D>
__global__ __launch_bounds__(64) void sdm_update_pipe_kernel(SdmUpdateArgs a,
                                                             const uint32_t* __restrict__ rec,
                                                             int nslice, int total) {
    using RC = Rec<NWG, NRG>;
    constexpr int W = NWG * G;
    constexpr int WORDS = RC::WORDS;
    constexpr int BLKW = D * WORDS;                 // words per block of D records
    constexpr int SEGS = (BLKW + 4 * 64 - 1) / (4 * 64);  // dwordx4 loads per lane per block
    __shared__ __align__(16) uint32_t meta[2][BLKW + 4];
    __shared__ float ring[D * W][CW];

    // XCD-aware placement: the 16 slices of a 128-column group share an XCD
    const int id = blockIdx.x;
    const int xcd = id & 7, k = id >> 3;
    const int L = (k >> 4) * 128 + xcd * 16 + (k & 15);
    if (L >= total) return;
    const int bh = L / nslice, slice = L - (L / nslice) * nslice;
    const int lane = threadIdx.x, g = lane >> 3, c = lane & 7;
    const int col = slice * CW + c;
    const int T = a.T;
    const io_t* vin = static_cast<const io_t*>(a.v);
    io_t* yout = static_cast<io_t*>(a.y);
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    float* tab = a.M + (size_t)bh * a.N * a.dv;
    const char* tabc = reinterpret_cast<const char*>(tab);
    const uint32_t* recb = rec + (size_t)bh * T * WORDS;
    const int nblk = (T + D - 1) / D;

    auto load_block = [&](int blk, uint4 (&st)[SEGS]) {
        const uint4* src = reinterpret_cast<const uint4*>(recb + (size_t)blk * BLKW);
        const int nwords = ((T - blk * D) < D ? (T - blk * D) : D) * WORDS;
#pragma unroll
        for (int s = 0; s < SEGS; ++s) {
            const int q = lane + 64 * s;
            st[s] = (blk < nblk && 4 * q < nwords) ? src[q] : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_block = [&](int buf, const uint4 (&st)[SEGS]) {
        uint4* dst = reinterpret_cast<uint4*>(&meta[buf][0]);
#pragma unroll
        for (int s = 0; s < SEGS; ++s) {
            const int q = lane + 64 * s;
            if (4 * q < BLKW) dst[q] = st[s];
        }
    };

    // rows in flight: token t's rows live in pre*[t % D]
    float prew[D][NWG], prer[D][NRG], prev[D];
    auto issue = [&](int tn, int u, const uint32_t* r) {
        // r = record of token tn in LDS
        const uint32_t* grp = r + g * RC::GW;
#pragma unroll
        for (int j = 0; j < NWG; ++j)
            prew[u][j] = *reinterpret_cast<const float*>(tabc + grp[j] + 4u * col);
#pragma unroll
        for (int j = 0; j < NRG; ++j)
            prer[u][j] = *reinterpret_cast<const float*>(tabc + grp[3 * NWG + j] + 4u * col);
        prev[u] = to_f32(vin[(((size_t)b * T + tn) * a.H + h) * a.dv + col]);
    };

    uint4 st[SEGS];
    load_block(0, st);
    store_block(0, st);
    load_block(1, st);
    store_block(1, st);
    wave_sync();
#pragma unroll
    for (int u = 0; u < D; ++u)
        if (u < T) issue(u, u, &meta[0][u * WORDS]);
    load_block(2, st);

    for (int blk = 0; blk < nblk; ++blk) {
        const uint32_t* cur = &meta[blk & 1][0];
        const uint32_t* nxt = &meta[(blk + 1) & 1][0];
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int t = blk * D + u;
            if (t < T) {
                const uint32_t* r = cur + u * WORDS;
                const uint32_t* grp = r + g * RC::GW;
                const float al = __uint_as_float(r[RC::HDR + 0]);
                const float be = __uint_as_float(r[RC::HDR + 1]);
                const uint32_t flags = r[RC::HDR + 2];
                float wv[NWG], wt[NWG];
                uint32_t woff[NWG];
#pragma unroll
                for (int j = 0; j < NWG; ++j) {
                    woff[j] = grp[j];
                    wt[j] = __uint_as_float(grp[NWG + j]);
                    wv[j] = prew[u][j];
                }
                if (flags & FLAG_WFWD) {
#pragma unroll
                    for (int j = 0; j < NWG; ++j) {
                        const int fw = (int)grp[2 * NWG + j];
                        if (fw >= 0) wv[j] = ring[fw][c];
                    }
                }
                float mt[NWG];
#pragma unroll
                for (int j = 0; j < NWG; ++j) mt[j] = al * wv[j];
                const float vc = prev[u];
                float nw[NWG];
                if (a.residual_mode == 0) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < NWG; ++j) acc = fmaf(wt[j], mt[j], acc);
                    acc += __shfl_xor(acc, 8, 64);
                    acc += __shfl_xor(acc, 16, 64);
                    acc += __shfl_xor(acc, 32, 64);
                    const float res = vc - acc;
#pragma unroll
                    for (int j = 0; j < NWG; ++j) nw[j] = fmaf(be * wt[j], res, mt[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < NWG; ++j) nw[j] = fmaf(be * wt[j], vc - mt[j], mt[j]);
                }
                const int ring0 = (t % D) * W;
#pragma unroll
                for (int j = 0; j < NWG; ++j) {
                    *reinterpret_cast<float*>(const_cast<char*>(tabc) + woff[j] + 4u * col) = nw[j];
                    ring[ring0 + g + G * j][c] = nw[j];
                }
                // read after writing
                float rv[NRG];
#pragma unroll
                for (int j = 0; j < NRG; ++j) rv[j] = prer[u][j];
                if (flags & FLAG_RFWD) {
                    wave_sync();  // this token's ring writes before its reads
#pragma unroll
                    for (int j = 0; j < NRG; ++j) {
                        const int fw = (int)grp[3 * NWG + 2 * NRG + j];
                        if (fw >= 0) rv[j] = ring[fw][c];
                    }
                }
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < NRG; ++j)
                    acc = fmaf(__uint_as_float(grp[3 * NWG + NRG + j]), rv[j], acc);
                acc += __shfl_xor(acc, 8, 64);
                acc += __shfl_xor(acc, 16, 64);
                acc += __shfl_xor(acc, 32, 64);
                if (g == 0) yout[(((size_t)b * T + t) * a.H + h) * a.dv + col] = from_f32<io_t>(acc);
            }
            // rows of token t + D, requested after token t's stores
            const int tn = t + D;
            if (tn < T) {
                wave_sync();
                issue(tn, u, nxt + u * WORDS);
            }
        }
        // records of block blk+2 replace block blk's; then request block blk+3
        wave_sync();
        store_block(blk & 1, st);
        wave_sync();
        load_block(blk + 3, st);
    }
}

template <typename io_t, int NWG, int NRG, int D>
hipError_t launch_pipe(const SdmUpdateArgs& a, uint32_t* rec, hipStream_t st) {
    RecArgs ra{a.B, a.T, a.H, a.N, a.dv, a.W, a.R, D, a.idx_w, a.wt_w, a.idx_r, a.wt_r,
               a.alpha, a.beta, rec};
    const long long P = (long long)a.B * a.T * a.H;
    sdm_records_kernel<NWG, NRG><<<(unsigned)((P + 3) / 4), 256, 0, st>>>(ra);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslice = a.dv / CW;
    const int total = a.B * a.H * nslice;
    const int grid = ((total + 127) / 128) * 128;
    sdm_update_pipe_kernel<io_t, NWG, NRG, D><<<grid, 64, 0, st>>>(a, rec, nslice, total);
    return hipGetLastError();
}

}  // namespace

bool sdm_pipe_supported(int W, int R, int dv, long long N) {
    if (dv % CW != 0) return false;
    if ((unsigned long long)N * (unsigned long long)dv * 4ull >= (1ull << 32)) return false;
    return (W == 32 && R == 32) || (W == 16 && R == 16) || (W == 64 && R == 64);
}

size_t sdm_pipe_record_bytes(int B, int T, int H, int W, int R) {
    const int words = G * (3 * (W / G) + 3 * (R / G)) + 4;
    return (size_t)B * H * T * words * 4;
}

hipError_t launch_sdm_update_pipe(const SdmUpdateArgs& a, void* rec, hipStream_t st) {
    uint32_t* r = static_cast<uint32_t*>(rec);
    const bool bf = a.dtype != 0;
    if (a.W == 32 && a.R == 32)
        return bf ? launch_pipe<bf16_t, 4, 4, 16>(a, r, st) : launch_pipe<float, 4, 4, 16>(a, r, st);
    if (a.W == 16 && a.R == 16)
        return bf ? launch_pipe<bf16_t, 2, 2, 16>(a, r, st) : launch_pipe<float, 2, 2, 16>(a, r, st);
    if (a.W == 64 && a.R == 64)
        return bf ? launch_pipe<bf16_t, 8, 8, 8>(a, r, st) : launch_pipe<float, 8, 8, 8>(a, r, st);
    return hipErrorInvalidValue;
}

}  // namespace sslp
