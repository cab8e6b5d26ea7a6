// K2 (pipelined): the Sparse Delta Memory recurrence given the addressing,
// with the table rows of future tokens streamed into LDS far ahead of use.
//
// Same arithmetic as the per-token kernel in sdm_update.hip (slides "Sparse
// Delta Memory: Scaling the State of Linear RNNs through Sparsity", Eqs.
// (3)-(5) and the shared-prediction figure form); only the schedule differs.
//
// Why: the recurrence of one value column is a chain over all T tokens, so a
// wavefront's table traffic is latency-bound unless the rows of token t+D are
// in flight while token t is computed.  Every token's addressing is known
// before the recurrence starts, so rows can be requested early; a row
// requested early is stale only if a token in between writes it.
//
// Two kernels:
//  * sdm_records_kernel (one wavefront per token) packs, per token and per
//    selected row, the byte offset of the row, its weight and a FORWARD code:
//    the latest writer (t', n') of the same slot among the D-1 preceding
//    tokens (and the token itself, for reads), i.e. a write that a load issued
//    D tokens early cannot have observed; -1 otherwise.
//  * sdm_update_pipe_kernel (one wavefront per 8-column slice of a head) walks
//    the tokens.  All global->LDS traffic (rows of token t+D, values, records)
//    uses the gfx950 LDS-DMA loads (global_load_lds_dwordx4 / _dword), which
//    need no registers, so D tokens of rows (D x 2 KB at W=R=32) stay in
//    flight.  The vector-memory counter is waited on explicitly before a
//    DMA'd buffer is read: the loop issues a fixed sequence of vector memory
//    instructions per token, so "at most 3(D-1) newer instructions
//    outstanding" implies that token t's rows (and its value group, requested
//    at least 15 tokens earlier) have landed.  Forwarded rows come from an LDS
//    ring holding the values written by the last D tokens; writes are stored
//    from that ring as 16-byte segments, and y is stored once per 16 tokens.
// Lane (g, c), g = lane/8, c = lane%8, owns column c of write rows n = g + 8j
// and read rows m = g + 8j; row sums are reduced over the 8 lane groups.
// Workgroups are placed so that the 16 slices sharing 512 bytes of a row run
// on the same XCD, whose L2 merges their 32-byte segments.
//
// Ordering: every table store and every later load of a column slice is issued
// by the same wavefront, whose vector memory operations are performed in
// order, so a load issued after a store to the same address observes it.
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

constexpr int CW = 8;   // columns per wavefront
constexpr int G = 8;    // lane groups (rows are dealt round-robin to them)
constexpr int VG = 16;  // tokens per value / output group

// record of one token, 32-bit words: [W+R rows][off, wt, fwd] then
// [alpha, beta, flags, pad]; rows are the write rows then the read rows
template <int W, int R>
struct Rec {
    static constexpr int HDR = 3 * (W + R);
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

template <int W, int R>
__global__ __launch_bounds__(256) void sdm_records_kernel(RecArgs a) {
    using RC = Rec<W, R>;
    constexpr int MAXD = 32;
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
        out[3 * x + 0] = (uint32_t)slot * (uint32_t)a.dv * 4u;
        out[3 * x + 1] = __float_as_uint(wt);
        out[3 * x + 2] = (uint32_t)fwd;
        if (isw) wf |= fwd >= 0;
        else rf |= fwd >= 0;
    }
    const bool anyw = __ballot(wf) != 0ull, anyr = __ballot(rf) != 0ull;
    if (lane == 0) {
        out[RC::HDR + 0] = __float_as_uint(a.alpha[bth]);
        out[RC::HDR + 1] = __float_as_uint(a.beta[bth]);
        out[RC::HDR + 2] = (anyw ? FLAG_WFWD : 0u) | (anyr ? FLAG_RFWD : 0u);
        out[RC::HDR + 3] = 0u;
    }
}

typedef void __attribute__((address_space(3))) * lds_ptr_t;

SSLP_DEVICE void dma16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 16, 0, 0);
}
SSLP_DEVICE void dma4(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 4, 0, 0);
}

// wait until at most N vector memory instructions are outstanding
template <int N>
SSLP_DEVICE void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_sched_barrier(0);
}

template <typename io_t, int W, int R, int D>
__global__ __launch_bounds__(64) void sdm_update_pipe_kernel(SdmUpdateArgs a,
                                                             const uint32_t* __restrict__ rec,
                                                             int nslice, int total) {
    using RC = Rec<W, R>;
    constexpr int WORDS = RC::WORDS;
    constexpr int NWG = W / G, NRG = R / G;
    constexpr int ROWS = W + R;
    constexpr int RDMA = ROWS / 32;                      // 16-byte DMA instructions per token
    constexpr int BLKW = D * WORDS;                      // words of D records
    constexpr int RECDMA = (BLKW + 255) / 256;           // DMA instructions per record block
    constexpr int VB = CW * (int)sizeof(io_t);           // value bytes per token
    constexpr int VDMA = (VG * VB + 255) / 256;          // dword DMA instructions per value group
    // per token the loop issues one 16-byte store and RDMA row DMAs (plus, once
    // per value group, a y store and the value DMA): at least 1 + RDMA = 3
    // vector memory instructions
    constexpr int PER_TOK = 1 + RDMA;
    constexpr int WAIT_ROWS = PER_TOK * (D - 1);
    constexpr int WAIT_REC = PER_TOK * D;
    static_assert(W == 32 && ROWS % 32 == 0, "store path assumes 32 write rows");
    static_assert(D <= VG, "value groups are requested one group ahead");
    static_assert(WAIT_ROWS <= 63 && WAIT_REC <= 63, "vmcnt range");

    __shared__ __align__(16) float rowbuf[D][ROWS][CW];
    __shared__ __align__(16) float ring[D * W][CW];
    __shared__ __align__(16) uint32_t meta[3][RECDMA * 256];
    __shared__ __align__(16) uint32_t vbuf[2][VDMA * 64];
    __shared__ __align__(16) io_t ybuf[VG][CW];

    // XCD-aware placement: the 16 slices of a 128-column group share an XCD
    const int id = blockIdx.x;
    const int xcd = id & 7, k = id >> 3;
    const int L = (k >> 4) * 128 + xcd * 16 + (k & 15);
    if (L >= total) return;
    const int bh = L / nslice, slice = L - (L / nslice) * nslice;
    const int lane = threadIdx.x, g = lane >> 3, c = lane & 7;
    const int col0 = slice * CW;
    const int T = a.T, H = a.H, dv = a.dv;
    const int b = bh / H, h = bh - (bh / H) * H;
    const char* tabc = reinterpret_cast<const char*>(a.M + (size_t)bh * a.N * dv);
    char* tabw = reinterpret_cast<char*>(a.M + (size_t)bh * a.N * dv);
    const char* vin = static_cast<const char*>(a.v);
    io_t* yout = static_cast<io_t*>(a.y);
    const uint32_t* recb = rec + (size_t)bh * T * WORDS;
    const int nblk = (T + D - 1) / D;
    const int ngrp = (T + VG - 1) / VG;
    // this lane's 16-byte piece of a row segment: row 32q + lane/2, half lane%2
    const uint32_t colbyte = 4u * (uint32_t)(col0 + 4 * (lane & 1));

    // -- DMA helpers; each issues a fixed number of vector memory instructions,
    //    out-of-range pieces read a valid dummy address and are never used --
    auto rec_dma = [&](int blk) {  // records of block blk -> meta[blk % 3]
        const int ntok = (T - blk * D) < D ? (T - blk * D) : D;
        const int nwords = blk < nblk ? ntok * WORDS : 0;
        const char* src = reinterpret_cast<const char*>(recb + (size_t)blk * BLKW);
        uint32_t* dst = &meta[blk % 3][0];
#pragma unroll
        for (int s = 0; s < RECDMA; ++s) {
            const int w0 = s * 256 + 4 * lane;
            const bool ok = w0 < nwords;
            dma16(ok ? (const void*)(src + 4 * w0) : (const void*)recb, dst + s * 256);
        }
    };
    auto val_dma = [&](int grp) {  // values of tokens [16 grp, 16 grp + 16) -> vbuf[grp & 1]
#pragma unroll
        for (int s = 0; s < VDMA; ++s) {
            const int byte = (s * 64 + lane) * 4;  // within the group's VG*VB bytes
            const int tt = grp * VG + byte / VB;
            const bool ok = grp < ngrp && byte < VG * VB && tt < T;
            const char* src = ok ? vin + ((((size_t)b * T + tt) * H + h) * dv + col0) * sizeof(io_t) +
                                       (byte % VB)
                                 : vin;
            dma4(src, &vbuf[grp & 1][s * 64]);
        }
    };
    auto row_dma = [&](int tn, const uint32_t* r) {  // rows of token tn -> rowbuf[tn % D]
        const int u = tn % D;
#pragma unroll
        for (int q = 0; q < RDMA; ++q) {
            const int row = 32 * q + (lane >> 1);
            const uint32_t off = tn < T ? r[3 * row] : 0u;
            dma16(tabc + off + colbyte, &rowbuf[u][32 * q][0]);
        }
    };

    // -- prologue: records of blocks 0..2, values of groups 0..1, rows of
    //    tokens 0..D-1, all complete before the loop --
    rec_dma(0);
    rec_dma(1);
    rec_dma(2);
    val_dma(0);
    val_dma(1);
    wait_vm<0>();
#pragma unroll
    for (int u = 0; u < D; ++u) row_dma(u, &meta[0][u * WORDS]);
    wait_vm<0>();

    for (int blk = 0; blk < nblk; ++blk) {
        const uint32_t* cur = &meta[blk % 3][0];
        const uint32_t* nxt = &meta[(blk + 1) % 3][0];
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int t = blk * D + u;
            if (t < T) {
                wait_vm<WAIT_ROWS>();  // rows of t (and its value group) have landed
                const uint32_t* r = cur + u * WORDS;
                const float al = __uint_as_float(r[RC::HDR + 0]);
                const float be = __uint_as_float(r[RC::HDR + 1]);
                const uint32_t flags = r[RC::HDR + 2];
                float wv[NWG], wt[NWG];
#pragma unroll
                for (int j = 0; j < NWG; ++j) {
                    const int n = g + G * j;
                    wt[j] = __uint_as_float(r[3 * n + 1]);
                    wv[j] = rowbuf[u][n][c];
                }
                if (flags & FLAG_WFWD) {
#pragma unroll
                    for (int j = 0; j < NWG; ++j) {
                        const int fw = (int)r[3 * (g + G * j) + 2];
                        if (fw >= 0) wv[j] = ring[fw][c];
                    }
                }
                const int vt = t % VG;
                const io_t vraw = reinterpret_cast<const io_t*>(&vbuf[(t / VG) & 1][0])[vt * CW + c];
                const float vc = to_f32(vraw);
                float mt[NWG], nw[NWG];
#pragma unroll
                for (int j = 0; j < NWG; ++j) mt[j] = al * wv[j];
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
                const int ring0 = u * W;
#pragma unroll
                for (int j = 0; j < NWG; ++j) ring[ring0 + g + G * j][c] = nw[j];
                // read after writing
                float rv[NRG];
#pragma unroll
                for (int j = 0; j < NRG; ++j) rv[j] = rowbuf[u][W + g + G * j][c];
                if (flags & FLAG_RFWD) {
#pragma unroll
                    for (int j = 0; j < NRG; ++j) {
                        const int fw = (int)r[3 * (W + g + G * j) + 2];
                        if (fw >= 0) rv[j] = ring[fw][c];
                    }
                }
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < NRG; ++j)
                    acc = fmaf(__uint_as_float(r[3 * (W + g + G * j) + 1]), rv[j], acc);
                acc += __shfl_xor(acc, 8, 64);
                acc += __shfl_xor(acc, 16, 64);
                acc += __shfl_xor(acc, 32, 64);
                if (g == 0) ybuf[vt][c] = from_f32<io_t>(acc);
                // the token's writes, 16 bytes per lane: row lane/2, columns 4(lane%2)..+3
                const int wrow = lane >> 1;
                const float4 seg =
                    *reinterpret_cast<const float4*>(&ring[ring0 + wrow][4 * (lane & 1)]);
                *reinterpret_cast<float4*>(tabw + r[3 * wrow] + colbyte) = seg;
                // outputs and values once per group of 16 tokens
                if (vt == VG - 1 || t == T - 1) {
                    const int gt0 = t - vt;
                    // (vt + 1) tokens of VB bytes, 4 bytes per lane and pass
                    for (int bb = lane * 4; bb < (vt + 1) * VB; bb += 256) {
                        const int tt = gt0 + bb / VB;
                        const int cb = bb % VB;
                        char* dst = reinterpret_cast<char*>(yout) +
                                    ((((size_t)b * T + tt) * H + h) * dv + col0) * sizeof(io_t) + cb;
                        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(
                            reinterpret_cast<const char*>(&ybuf[0][0]) + bb);
                    }
                    val_dma(t / VG + 2);
                }
            }
            // rows of token t + D (after token t's stores)
            row_dma(t + D, nxt + u * WORDS);
        }
        // records of block blk+2 (requested one block ago) must be in LDS before
        // block blk+1 requests rows of block blk+2; then request block blk+3
        // into the buffer block blk no longer needs
        wait_vm<WAIT_REC>();
        rec_dma(blk + 3);
    }
    wait_vm<0>();
}

template <typename io_t, int W, int R, int D>
hipError_t launch_pipe(const SdmUpdateArgs& a, uint32_t* rec, hipStream_t st) {
    RecArgs ra{a.B, a.T, a.H, a.N, a.dv, a.W, a.R, D, a.idx_w, a.wt_w, a.idx_r, a.wt_r,
               a.alpha, a.beta, rec};
    const long long P = (long long)a.B * a.T * a.H;
    sdm_records_kernel<W, R><<<(unsigned)((P + 3) / 4), 256, 0, st>>>(ra);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslice = a.dv / CW;
    const int total = a.B * a.H * nslice;
    const int grid = ((total + 127) / 128) * 128;
    sdm_update_pipe_kernel<io_t, W, R, D><<<grid, 64, 0, st>>>(a, rec, nslice, total);
    return hipGetLastError();
}

}  // namespace

// The pipelined kernel holds one workgroup per CU (its LDS footprint), so it pays
// off for long sequences spread over few column slices; short sequences (decode)
// and many-slice batches are left to the per-token kernel, whose occupancy hides
// the latency instead.
bool sdm_pipe_supported(int B, int T, int H, int W, int R, int dv, long long N) {
    if (dv % CW != 0) return false;
    if ((unsigned long long)N * (unsigned long long)dv * 4ull >= (1ull << 31)) return false;
    if (T < 64 || (long long)B * H * (dv / CW) > 1024) return false;
    return W == 32 && R == 32;
}

size_t sdm_pipe_record_bytes(int B, int T, int H, int W, int R) {
    const int words = 3 * (W + R) + 4;
    // + one block of slack: record DMAs read whole 1 KB pieces
    return ((size_t)B * H * T + 64) * words * 4;
}

hipError_t launch_sdm_update_pipe(const SdmUpdateArgs& a, void* rec, hipStream_t st) {
    uint32_t* r = static_cast<uint32_t*>(rec);
    if (a.W == 32 && a.R == 32)
        return a.dtype != 0 ? launch_pipe<bf16_t, 32, 32, 16>(a, r, st)
                            : launch_pipe<float, 32, 32, 16>(a, r, st);
    return hipErrorInvalidValue;
}

}  // namespace sslp
