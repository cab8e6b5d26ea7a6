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
//    selected row, the byte offset of the row, its weight and its SOURCE: the
//    LDS row that will hold the slot's current value when the token runs --
//    the staging slot the row is DMA'd into, or, when one of the preceding D
//    tokens (or the token itself, for reads) wrote the slot, the ring row
//    holding that newer value.
//  * sdm_update_pipe_kernel (one wavefront per 8-column slice of a head) walks
//    the tokens.  All global->LDS traffic (rows of token t+D, values, records)
//    uses the gfx950 LDS-DMA loads (global_load_lds_dwordx4 / _dword), which
//    need no registers, so D tokens of rows (D x 2 KB at W=R=32) stay in
//    flight.  The vector-memory counter is waited on explicitly before a
//    DMA'd buffer is read: the loop issues a fixed sequence of vector memory
//    instructions per token, so "at most 3(D-1) newer instructions
//    outstanding" implies that token t's rows (and its value group, requested
//    at least 32 tokens earlier) have landed.
// The per-token critical path is kept to one LDS round trip: the token's
// weights and row sources are loaded into registers one token ahead, every
// row value is read from its source in one batch, row sums are DPP octet
// reductions, and the token's 16-byte write-back segments are stored one
// token later from the ring.  y is stored once per 32 tokens.
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
constexpr int VG = 32;  // tokens per value / output group

// tokens of table rows in flight per wavefront
#ifndef SSLP_SDM_PIPE_D
#define SSLP_SDM_PIPE_D 16
#endif
constexpr int PIPE_D = SSLP_SDM_PIPE_D;

// Record of one token, 32-bit words:
//   [0, W+R)            byte offset of each row in the head's table (write rows, then read rows)
//   [W+R, 3(W+R))       (weight, source) pairs, ordered so that lane group g finds its
//                       rows g, g+8, g+16, ... as consecutive pairs: write row n at pair
//                       (n % 8) * (W/8) + n / 8, read row m at W + (m % 8) * (R/8) + m / 8
//   [3(W+R), +4)        alpha, beta, flags, 0
template <int W, int R>
struct Rec {
    static constexpr int ROWS = W + R;
    static constexpr int PAIR = ROWS;
    static constexpr int HDR = 3 * ROWS;
    static constexpr int WORDS = HDR + 4;
};
constexpr uint32_t FLAG_RSELF = 1u;  // a read row was written by the same token

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

// One wavefront per token.  A row DMA'd for token t is requested D tokens
// early and table stores trail their token by one, so the latest value of a
// slot written by any of tokens t-D .. t-1 (and t itself, for reads) is not in
// the table when the row is fetched: such rows are sourced from the ring,
// which keeps the written rows of the last D+1 tokens (ring slot t % (D+1)).
template <int W, int R>
__global__ __launch_bounds__(256) void sdm_records_kernel(RecArgs a) {
    using RC = Rec<W, R>;
    constexpr int MAXD = 32;
    __shared__ int32_t win[4][MAXD + 1][W];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long p = (long long)blockIdx.x * 4 + wv;  // (b, t, h) in [B,T,H] order
    if (p >= (long long)a.B * a.T * a.H) return;
    const int h = (int)(p % a.H);
    const int t = (int)((p / a.H) % a.T);
    const int b = (int)(p / ((long long)a.H * a.T));
    const int D = a.D;
    const int tlo = t - D > 0 ? t - D : 0;
    const int nt = t - tlo + 1;  // window tokens tlo..t
    for (int e = lane; e < nt * W; e += 64) {
        const int tt = tlo + e / W, n = e - (e / W) * W;
        win[wv][e / W][n] = a.idx_w[(((size_t)b * a.T + tt) * a.H + h) * W + n];
    }
    wave_sync();
    const size_t bth = ((size_t)b * a.T + t) * a.H + h;
    uint32_t* out = a.rec + (((size_t)b * a.H + h) * a.T + t) * RC::WORDS;
    const int ring0 = D * RC::ROWS;  // first ring row among the update kernel's LDS rows
    bool self = false;
    for (int x = lane; x < RC::ROWS; x += 64) {
        const bool isw = x < W;
        const int n = isw ? x : x - W;
        const int slot = isw ? a.idx_w[bth * W + n] : a.idx_r[bth * R + n];
        const float wt = isw ? a.wt_w[bth * W + n] : a.wt_r[bth * R + n];
        int src = (t % D) * RC::ROWS + x;
        for (int tt = isw ? t - 1 : t; tt >= tlo; --tt) {
            int hit = -1;
            for (int n2 = 0; n2 < W; ++n2)
                if (win[wv][tt - tlo][n2] == slot) {
                    hit = n2;
                    break;
                }
            if (hit >= 0) {
                src = ring0 + (tt % (D + 1)) * W + hit;
                self |= !isw && tt == t;
                break;
            }
        }
        const int pr = isw ? (n % G) * (W / G) + n / G : W + (n % G) * (R / G) + n / G;
        out[x] = (uint32_t)slot * (uint32_t)a.dv * 4u;
        out[RC::PAIR + 2 * pr + 0] = __float_as_uint(wt);
        out[RC::PAIR + 2 * pr + 1] = (uint32_t)src;
    }
    const bool anyself = __ballot(self) != 0ull;
    if (lane == 0) {
        out[RC::HDR + 0] = __float_as_uint(a.alpha[bth]);
        out[RC::HDR + 1] = __float_as_uint(a.beta[bth]);
        out[RC::HDR + 2] = anyself ? FLAG_RSELF : 0u;
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

// sum over the 8 lanes of an aligned lane octet, left in all 8 (DPP, no LDS):
// swap neighbours, swap pairs, then mirror within the octet
SSLP_DEVICE float octet_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

// LDS reads on the per-token path are issued as inline asm.  The compiler
// cannot tell a read of a DMA'd row at a data-dependent address from one that
// aliases an LDS-DMA still in flight, and would drain the whole vector memory
// queue before it; it would also wait for the next token's records as soon as
// they are loaded.  The rows were DMA'd long before (ordered by the explicit
// vmcnt waits), so the reads are issued directly and their results are tied to
// an explicit "lgkmcnt(0)" wait placed where they are first needed.  The
// "memory" clobbers keep them in program order with the ring and staging writes.
typedef float __attribute__((address_space(3))) * lds_f32_ptr_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
SSLP_DEVICE uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_f32_ptr_t)p; }
SSLP_DEVICE float lds_f32(uint32_t addr) {
    float v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
SSLP_DEVICE uint32_t lds_u32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
SSLP_DEVICE uint32_t lds_u16(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
SSLP_DEVICE u32x4 lds_u32x4(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
SSLP_DEVICE f32x4 lds_f32x4(uint32_t addr) {
    f32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// per-token values a lane needs, loaded one token ahead (raw record words)
struct TokRegs {
    u32x4 pw[2], pr[2];   // (weight, source) of write rows g+8j, read rows g+8j
    uint32_t al, be, fl;  // alpha, beta, flags
    uint32_t st;          // table byte offset of write row lane/2 (write-back)
};

// issue the loads of a record at LDS byte address ra (no wait)
template <int W, int R>
SSLP_DEVICE void load_tok(TokRegs& k, uint32_t ra, int g, int lane) {
    using RC = Rec<W, R>;
    const uint32_t pw = ra + 4u * (RC::PAIR + 2 * g * (W / G));
    const uint32_t pr = ra + 4u * (RC::PAIR + 2 * (W + g * (R / G)));
    k.pw[0] = lds_u32x4(pw);
    k.pw[1] = lds_u32x4(pw + 16);
    k.pr[0] = lds_u32x4(pr);
    k.pr[1] = lds_u32x4(pr + 16);
    k.al = lds_u32(ra + 4u * RC::HDR);
    k.be = lds_u32(ra + 4u * (RC::HDR + 1));
    k.fl = lds_u32(ra + 4u * (RC::HDR + 2));
    k.st = lds_u32(ra + 4u * (uint32_t)(lane >> 1));
}
SSLP_DEVICE void wait_tok(TokRegs& k) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(k.pw[0]), "+v"(k.pw[1]), "+v"(k.pr[0]), "+v"(k.pr[1]), "+v"(k.al),
                   "+v"(k.be), "+v"(k.fl), "+v"(k.st)
                 :
                 : "memory");
}

// Lane (c, g), c = lane/8, g = lane%8, owns column c of write rows g + 8j and
// read rows g + 8j; row sums are octet sums.  LDS rows (8 floats each):
//   [0, D*(W+R))            staging: rows of token t at slot t % D
//   [D*(W+R), +(D+1)*W)     ring: rows written by token t at slot t % (D+1)
template <typename io_t, int W, int R, int D>
__global__ __launch_bounds__(64) void sdm_update_pipe_kernel(SdmUpdateArgs a,
                                                             const uint32_t* __restrict__ rec,
                                                             int nslice, int total) {
    using RC = Rec<W, R>;
    constexpr int WORDS = RC::WORDS;
    constexpr int ROWS = RC::ROWS;
    constexpr int RING0 = D * ROWS;
    constexpr int NLROWS = RING0 + (D + 1) * W;
    constexpr int RDMA = ROWS / 32;              // 16-byte DMA instructions per token
    constexpr int BLKW = D * WORDS;              // words of D records
    constexpr int RECDMA = (BLKW + 255) / 256;   // DMA instructions per record block
    constexpr int VB = CW * (int)sizeof(io_t);   // value bytes per token
    constexpr int VDMA = (VG * VB + 255) / 256;  // dword DMA instructions per value group
    // every token issues one 16-byte store (the previous token's writes) and RDMA
    // row DMAs; value, output and record traffic only adds instructions
    constexpr int PER_TOK = 1 + RDMA;
    constexpr int WAIT_ROWS = PER_TOK * (D - 1);
    constexpr int WAIT_REC = PER_TOK * D;
    static_assert(W == 32 && R == 32, "row layout: 4 write and 4 read rows per lane");
    static_assert(RDMA == 2, "two row pieces per lane and token");
    static_assert(D <= VG + 1, "value groups are requested one group ahead");
    static_assert(WAIT_ROWS <= 63 && WAIT_REC <= 63, "vmcnt range");
    static_assert((WORDS * 4) % 16 == 0, "records are DMA'd in 16-byte pieces");

    __shared__ __align__(16) float rows[NLROWS][CW];
    __shared__ __align__(16) uint32_t meta[3][RECDMA * 256];
    __shared__ __align__(16) uint32_t vbuf[2][VDMA * 64];
    __shared__ __align__(16) io_t ybuf[VG][CW];

    // XCD-aware placement: the 16 slices of a 128-column group share an XCD
    const int id = blockIdx.x;
    const int xcd = id & 7, kq = id >> 3;
    const int L = (kq >> 4) * 128 + xcd * 16 + (kq & 15);
    if (L >= total) return;
    const int bh = L / nslice, slice = L - (L / nslice) * nslice;
    const int lane = threadIdx.x, c = lane >> 3, g = lane & 7;
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
    // this lane's 16-byte piece of a row: columns 4(lane%2) .. +3 of the slice
    const uint32_t colbyte = 4u * (uint32_t)(col0 + 4 * (lane & 1));
    // this lane's column of LDS row 0; row x is lbase + 32 x
    const uint32_t lbase = lds_addr(&rows[0][c]);
    const uint32_t mbase = lds_addr(&meta[0][0]);
    const uint32_t vbase = lds_addr(&vbuf[0][0]) + (uint32_t)(c * sizeof(io_t));

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
    auto val_dma = [&](int grp) {  // values of tokens [32 grp, 32 grp + 32) -> vbuf[grp & 1]
#pragma unroll
        for (int s = 0; s < VDMA; ++s) {
            const int byte = (s * 64 + lane) * 4;
            const int tt = grp * VG + byte / VB;
            const bool ok = grp < ngrp && byte < VG * VB && tt < T;
            const char* src = ok ? vin + ((((size_t)b * T + tt) * H + h) * dv + col0) * sizeof(io_t) +
                                       (byte % VB)
                                 : vin;
            dma4(src, &vbuf[grp & 1][s * 64]);
        }
    };
    // rows of token tn -> staging slot tn % D; off[q] = table offset of row 32q + lane/2
    auto row_dma = [&](int tn, const uint32_t (&off)[RDMA]) {
        const int u = tn % D;
#pragma unroll
        for (int q = 0; q < RDMA; ++q)
            dma16(tabc + (tn < T ? off[q] : 0u) + colbyte, &rows[u * ROWS + 32 * q][0]);
    };
    // LDS address of the 16-byte write-back piece of token tp (ring slot tp % (D+1))
    auto ring_piece = [&](int tp) {
        return lds_addr(&rows[RING0 + (tp % (D + 1)) * W + (lane >> 1)][4 * (lane & 1)]);
    };
    auto rec_addr = [&](int buf, int u) { return mbase + 4u * (uint32_t)(buf * RECDMA * 256 + u * WORDS); };

    // -- prologue: records of blocks 0..2, values of groups 0..1, rows of
    //    tokens 0..D-1, all complete before the loop --
    rec_dma(0);
    rec_dma(1);
    rec_dma(2);
    val_dma(0);
    val_dma(1);
    wait_vm<0>();
#pragma unroll
    for (int u = 0; u < D; ++u) {
        uint32_t off[RDMA];
#pragma unroll
        for (int q = 0; q < RDMA; ++q) off[q] = meta[0][u * WORDS + 32 * q + (lane >> 1)];
        row_dma(u, off);
    }
    TokRegs kn;
    load_tok<W, R>(kn, rec_addr(0, 0), g, lane);
    uint32_t prev_st = 0;
    wait_vm<0>();

    for (int blk = 0; blk < nblk; ++blk) {
        const int bc = blk % 3, bn = (blk + 1) % 3;
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int t = blk * D + u;
            uint32_t off[RDMA];  // table offsets for the rows of token t + D
            if (t < T) {
                wait_vm<WAIT_ROWS>();  // rows of t (and its value group) have landed
                wait_tok(kn);          // this token's record words (loaded a token ago)
                const TokRegs k = kn;
                const uint32_t fl = __builtin_amdgcn_readfirstlane(k.fl);
                const uint32_t sw[4] = {k.pw[0].y, k.pw[0].w, k.pw[1].y, k.pw[1].w};
                const uint32_t sr[4] = {k.pr[0].y, k.pr[0].w, k.pr[1].y, k.pr[1].w};
                const float ww[4] = {__uint_as_float(k.pw[0].x), __uint_as_float(k.pw[0].z),
                                     __uint_as_float(k.pw[1].x), __uint_as_float(k.pw[1].z)};
                const float wr[4] = {__uint_as_float(k.pr[0].x), __uint_as_float(k.pr[0].z),
                                     __uint_as_float(k.pr[1].x), __uint_as_float(k.pr[1].z)};
                const float al = __uint_as_float(k.al), be = __uint_as_float(k.be);
                // one batch of LDS reads: row values (staging or ring), the value,
                // the previous token's write-back piece, the rows of token t + D
                float wv[4], rv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) wv[j] = lds_f32(lbase + sw[j] * (CW * 4));
#pragma unroll
                for (int j = 0; j < 4; ++j) rv[j] = lds_f32(lbase + sr[j] * (CW * 4));
                const int vt = t % VG;
                const uint32_t va = vbase + (uint32_t)(((t / VG) & 1) * VDMA * 256 + vt * VB);
                uint32_t vraw = sizeof(io_t) == 2 ? lds_u16(va) : lds_u32(va);
                f32x4 seg = lds_f32x4(ring_piece(t > 0 ? t - 1 : 0));
                const uint32_t na = rec_addr(bn, u);  // record of token t + D
#pragma unroll
                for (int q = 0; q < RDMA; ++q) off[q] = lds_u32(na + 4u * (32 * q + (lane >> 1)));
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(wv[0]), "+v"(wv[1]), "+v"(wv[2]), "+v"(wv[3]), "+v"(rv[0]),
                               "+v"(rv[1]), "+v"(rv[2]), "+v"(rv[3]), "+v"(vraw), "+v"(seg),
                               "+v"(off[0]), "+v"(off[1])
                             :
                             : "memory");
                const float vc = sizeof(io_t) == 2 ? __uint_as_float(vraw << 16) : __uint_as_float(vraw);
                // previous token's write-back, then the next token's record
                if (t > 0)
                    *reinterpret_cast<f32x4*>(tabw + prev_st + colbyte) = seg;
                prev_st = k.st;
                load_tok<W, R>(kn, u + 1 < D ? rec_addr(bc, u + 1) : rec_addr(bn, 0), g, lane);

                float mt[4], nw[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) mt[j] = al * wv[j];
                if (a.residual_mode == 0) {
                    const float p0 = fmaf(ww[2], mt[2], ww[0] * mt[0]);
                    const float p1 = fmaf(ww[3], mt[3], ww[1] * mt[1]);
                    const float res = vc - octet_sum(p0 + p1);
#pragma unroll
                    for (int j = 0; j < 4; ++j) nw[j] = fmaf(be * ww[j], res, mt[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) nw[j] = fmaf(be * ww[j], vc - mt[j], mt[j]);
                }
                const int ring = RING0 + (t % (D + 1)) * W;
#pragma unroll
                for (int j = 0; j < 4; ++j) rows[ring + g + G * j][c] = nw[j];
                if (fl & FLAG_RSELF) {
                    // some read row is one this token just wrote: read again
#pragma unroll
                    for (int j = 0; j < 4; ++j) rv[j] = lds_f32(lbase + sr[j] * (CW * 4));
                    asm volatile("s_waitcnt lgkmcnt(0)"
                                 : "+v"(rv[0]), "+v"(rv[1]), "+v"(rv[2]), "+v"(rv[3])
                                 :
                                 : "memory");
                }
                const float q0 = fmaf(wr[2], rv[2], wr[0] * rv[0]);
                const float q1 = fmaf(wr[3], rv[3], wr[1] * rv[1]);
                const float yv = octet_sum(q0 + q1);
                if (g == 0) ybuf[vt][c] = from_f32<io_t>(yv);
                // outputs and values once per group of 32 tokens
                if (vt == VG - 1 || t == T - 1) {
                    const int gt0 = t - vt;
                    for (int bb = lane * 4; bb < (vt + 1) * VB; bb += 256) {
                        const int tt = gt0 + bb / VB;
                        char* dst = reinterpret_cast<char*>(yout) +
                                    ((((size_t)b * T + tt) * H + h) * dv + col0) * sizeof(io_t) +
                                    bb % VB;
                        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(
                            reinterpret_cast<const char*>(&ybuf[0][0]) + bb);
                    }
                    val_dma(t / VG + 2);
                }
            } else {
#pragma unroll
                for (int q = 0; q < RDMA; ++q) off[q] = 0u;
            }
            // rows of token t + D
            row_dma(t + D, off);
        }
        // records of block blk+2 (requested one block ago) must be in LDS before
        // block blk+1 requests rows of block blk+2; then request block blk+3
        // into the buffer block blk no longer needs
        wait_vm<WAIT_REC>();
        rec_dma(blk + 3);
    }
    if (T > 0) {
        const f32x4 seg = *reinterpret_cast<const f32x4*>(
            &rows[RING0 + ((T - 1) % (D + 1)) * W + (lane >> 1)][4 * (lane & 1)]);
        *reinterpret_cast<f32x4*>(tabw + prev_st + colbyte) = seg;
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
    // + slack: record DMAs read whole 1 KB pieces past the last token
    return ((size_t)B * H * T + 64) * words * 4;
}

hipError_t launch_sdm_update_pipe(const SdmUpdateArgs& a, void* rec, hipStream_t st) {
    uint32_t* r = static_cast<uint32_t*>(rec);
    if (a.W == 32 && a.R == 32)
        return a.dtype != 0 ? launch_pipe<bf16_t, 32, 32, PIPE_D>(a, r, st)
                            : launch_pipe<float, 32, 32, PIPE_D>(a, r, st);
    return hipErrorInvalidValue;
}

}  // namespace sslp
