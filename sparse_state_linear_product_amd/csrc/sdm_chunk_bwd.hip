// Backward of the chunk-parallel Sparse Delta Memory recurrence, chunk by chunk
// in reverse, by undoing writes.
//
// Sparse Delta Memory slides: "Training parallelizes within chunks and recurs
// across chunks", the backup "Backup: undoing writes avoids repeated
// full-table snapshots" and Eqs. (3)-(5) with the shared or per-slot residual
// ("A v1 inconsistency matters for reproducing the update").  Same operation
// and results (to rounding) as the per-token sweep in sdm_backward.hip.
//
// Within a chunk the forward is linear in the chunk-start table M0 and the
// residuals (sdm_chunk.hip): res = T (v - g), y = E M0 + Bm res,
// M_C = P M0 + F res.  Walking the tokens of the chunk backwards, the gradient
// of the residual of token t (which is also dv_t) satisfies
//   (I + A^T) dr = F^T dM_C + Bm^T dy,   i.e.   dr = T^T (u + Bm^T dy),
//   u_t = sum_i f_ti dM_C[n_ti],  f_ti = beta_t w_ti * (decays of the slot's
//   later visits in the chunk),
// with the forward plan's T = (I + A)^-1 and Bm (A = 0, T = I for the per-slot
// form).  Given dr, every slot's gradient row is carried backwards through its
// events in the chunk, in reverse token order (at a token, its read before its
// write): a read at t adds e_tk dy_t; a write visit (t, i) is where the
// per-token step of the sweep is taken with G = the carried row:
//   shared    dMt = G - w dr_t;  dbeta += w <G, r_t>;  dw = beta <G, r_t> - alpha <P, dr_t>
//   per-slot  dMt = (1 - beta w) G;  dbeta += w <G, v_t - alpha P>;  dw = beta <G, v_t - alpha P>
//   dalpha += <P, dMt>;  G <- alpha dMt
// (P = the visit's pre-write row, kept by the forward; r_t = v_t -
// alpha_t sum_i w_ti P_ti).  The row left at the chunk start is the slot's
// gradient before the chunk; the table row goes back to the pre-write row of
// the slot's first visit.  A read sees the row after the slot's last write at
// or before its token (d P + beta w res of that visit), else the chunk-start
// row (the pre-write row of the slot's first visit, or the table row for a
// slot the chunk does not write): de_tk = <that row, dy_t>.
//
// A plan kernel lists, per (b, h, chunk), every slot's events in token order,
// f for every write entry and the source of every read's row; the sweep kernel
// runs one workgroup per 8-column slice of a head through the chunks in
// reverse: it gathers the gradient-table rows of every entry and the table
// rows of the reads (LDS-DMA), forms r, u, dr (dv), then carries each slot's
// row through its events (two lanes per slot), writes the slot's gradient and
// restored table row once, and leaves per-token partial sums of the scalar
// gradients for the slice reduction.  The next chunk's plans, inputs and
// pre-write rows are loaded during the step's arithmetic.  Every store of a
// chunk completes before the next (earlier) chunk's gathers are issued.
#include "common.h"
#include "kernels.h"
#include "sdm_chunk.h"

namespace sslp {

namespace {

using namespace chunk;

// backward plan block of one (b, h, chunk), 32-bit words
constexpr int NEV = 2 * NE;               // events per chunk: C x (W + R) = 1024
constexpr int BPL_F = 0;                  // [t][i] f of write entry (t, i)
constexpr int BPL_Y = BPL_F + NE;         // [t][k] source of read entry (t, k)'s row
constexpr int BPL_EV = BPL_Y + NE;        // events sorted by (slot, token, kind)
constexpr int BPL_GS = BPL_EV + NEV;      // [g] first event of slot group g, [ng] = events
constexpr int BPL_NG = BPL_GS + NEV + 1;  // number of slot groups
constexpr int BPL_WORDS = (BPL_NG + 1 + 3) / 4 * 4;
static_assert(BPL_WORDS % 4 == 0 && BPL_F % 4 == 0 && BPL_EV % 4 == 0, "plan copies in 16 bytes");
// event word: token | kind << 5 (0 write, 1 read) | row index << 6
// read source: kind (0 table row, 1 pre-write row of entry (tok, i), 2 the row
// after write entry (tok, i)) | tok << 2 | i << 7

struct BwdPlanArgs {
    int B, T, H, N, nch, mode;
    const int32_t* idx_w;
    const float* wt_w;
    const int32_t* idx_r;
    const float* alpha;
    const float* beta;
    uint32_t* bplan;  // [B, H, nch, BPL_WORDS]
};

// ---------------------------------------------------------------------------
// plan kernel: one workgroup of 256 threads per (b, h, chunk)
// ---------------------------------------------------------------------------
template <class G>
__global__ __launch_bounds__(256) void sdm_chunk_bwd_plan_kernel(BwdPlanArgs a) {
    constexpr int CC = G::CC, NW = G::NW, NR = G::NR, LOGNW = G::LOGNW;
    __shared__ uint64_t key[NEV];  // (slot << 12 | token << 7 | kind << 6 | index), sorted
    __shared__ int s_scan[NEV];    // group starts, then their inclusive prefix count
    __shared__ uint64_t s_xbuf[NEV];  // the sort's exchange buffer
    __shared__ int s_tot[4 * (NEV / 256)];  // wavefront totals of the scan
    __shared__ float s_d[NE], s_bw[NE];  // decay and beta w of write entry t*NW + i
    __shared__ float s_al[CC], s_be[CC];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int nch = a.nch;
    const int c = blockIdx.x % nch, bh = blockIdx.x / nch;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int t0 = c * CC;
    const uint64_t NONE = ~0ull;
    // a chunk holding a slot outside [0, N) has no events (the forward plan of
    // the same chunk reports it)
    if (tid == 0) s_bad = 0;
    __syncthreads();
    const int nt = a.T - t0 < CC ? a.T - t0 : CC;
    // every load issued before any test (rows past the end load the last
    // token's indices and weights, then unused); the keys below reuse them
    static_assert(NE % 256 == 0, "whole passes of the 256 threads");
    unsigned sw[NE / 256], sr[NE / 256];
    float ww[NE / 256];
    {
#pragma unroll
        for (int r = 0; r < NE / 256; ++r) {
            const int e = tid + 256 * r;
            const int t = (e >> LOGNW) < nt ? (e >> LOGNW) : nt - 1;
            const size_t bth = ((size_t)b * a.T + t0 + t) * a.H + h;
            sw[r] = (unsigned)a.idx_w[bth * NW + (e & (NW - 1))];
            sr[r] = (unsigned)a.idx_r[bth * NR + (e & (NW - 1))];
            ww[r] = a.wt_w[bth * NW + (e & (NW - 1))];
        }
        bool bad = false;
#pragma unroll
        for (int r = 0; r < NE / 256; ++r)
            bad |= ((tid + 256 * r) >> LOGNW) < nt && (sw[r] >= (unsigned)a.N || sr[r] >= (unsigned)a.N);
        if (bad) s_bad = 1;
    }
    __syncthreads();
    const int ntok = s_bad ? 0 : nt;
    uint32_t* out = a.bplan + (size_t)blockIdx.x * BPL_WORDS;
    if (tid < CC) {
        const bool ok = tid < ntok;
        const size_t bth = ((size_t)b * a.T + t0 + (ok ? tid : 0)) * a.H + h;
        s_al[tid] = ok ? a.alpha[bth] : 1.f;
        s_be[tid] = ok ? a.beta[bth] : 0.f;
    }
    __syncthreads();

    // S1: one key per entry: writes (kind 0) at x < NE, reads (kind 1) above
    static_assert(NEV == 4 * 256 && NE == 2 * 256, "x = tid + 256 j: writes for j < 2");
#pragma unroll
    for (int jx = 0; jx < NEV / 256; ++jx) {
        const int x = tid + 256 * jx;
        const int rd = x >= NE ? 1 : 0;
        const int e = x - rd * NE;
        const int t = e >> LOGNW, i = e & (NW - 1);
        uint64_t k = NONE;
        float w = 0.f;
        if (t < ntok) {
            const uint32_t sl = rd ? sr[jx & 1] : sw[jx & 1];
            k = ((uint64_t)sl << 12) | ((uint64_t)t << 7) | ((uint64_t)rd << 6) | (uint64_t)i;
            if (!rd) w = ww[jx & 1];
        }
        key[x] = k;
        if (!rd) {
            s_bw[e] = s_be[t] * w;
            s_d[e] = a.mode == 0 ? s_al[t] : s_al[t] * (1.f - s_be[t] * w);
        }
    }
    __syncthreads();

    // S2: bitonic sort of the keys, ascending (invalid keys last)
    static_assert(NEV == 1024, "four keys per thread");
    {
        uint64_t kr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) kr[r] = key[tid + 256 * r];
        chunk::block_sort_asc<4>(kr, key, s_xbuf);
        __syncthreads();
    }

    // S3: slot groups (equal slot) and their inclusive prefix count
    const int nev = ntok * (NW + NR);
    for (int p = tid; p < NEV; p += 256)
        s_scan[p] = (p < nev && (p == 0 || (key[p - 1] >> 12) != (key[p] >> 12))) ? 1 : 0;
    __syncthreads();
    {
        int v[NEV / 256];
#pragma unroll
        for (int x = 0; x < NEV / 256; ++x) v[x] = s_scan[tid + 256 * x];
        chunk::block_scan<NEV / 256>(v, s_tot);
#pragma unroll
        for (int x = 0; x < NEV / 256; ++x) s_scan[tid + 256 * x] = v[x];
        __syncthreads();
    }
    const int ng = nev > 0 ? s_scan[nev - 1] : 0;

    // S4: the event list, group starts, f of the writes, sources of the reads
    for (int p = tid; p < nev; p += 256) {
        const uint64_t kp = key[p];
        const uint64_t sl = kp >> 12;
        const int t = (int)((kp >> 7) & 31u), rd = (int)((kp >> 6) & 1u), i = (int)(kp & 63u);
        out[BPL_EV + p] = (uint32_t)t | ((uint32_t)rd << 5) | ((uint32_t)i << 6);
        if (p == 0 || (key[p - 1] >> 12) != sl) out[BPL_GS + s_scan[p] - 1] = (uint32_t)p;
        if (!rd) {
            float f = s_bw[t * NW + i];
            for (int l = p + 1; l < nev && (key[l] >> 12) == sl; ++l)
                if (((key[l] >> 6) & 1u) == 0u)
                    f *= s_d[(int)((key[l] >> 7) & 31u) * NW + (int)(key[l] & 63u)];
            out[BPL_F + t * NW + i] = __float_as_uint(f);
        } else {
            // the slot's last write at or before t (a write at t sorts before
            // this read), else its first write in the chunk, else none
            uint32_t rec = 0u;
            int l = p - 1;
            while (l >= 0 && (key[l] >> 12) == sl && ((key[l] >> 6) & 1u) != 0u) --l;
            if (l >= 0 && (key[l] >> 12) == sl) {
                rec = 2u | ((uint32_t)((key[l] >> 7) & 31u) << 2) | ((uint32_t)(key[l] & 63u) << 7);
            } else {
                l = p + 1;
                while (l < nev && (key[l] >> 12) == sl && ((key[l] >> 6) & 1u) != 0u) ++l;
                if (l < nev && (key[l] >> 12) == sl)
                    rec = 1u | ((uint32_t)((key[l] >> 7) & 31u) << 2) |
                          ((uint32_t)(key[l] & 63u) << 7);
            }
            out[BPL_Y + t * NR + i] = rec;
        }
    }
    for (int e = tid; e < NE; e += 256)
        if ((e >> LOGNW) >= ntok) {
            out[BPL_F + e] = 0u;
            out[BPL_Y + e] = 0u;
        }
    if (tid == 0) {
        out[BPL_GS + ng] = (uint32_t)nev;
        out[BPL_NG] = (uint32_t)ng;
    }
}

// ---------------------------------------------------------------------------
// sweep kernel helpers
// ---------------------------------------------------------------------------
// The next chunk's plans and inputs are loaded a chunk ahead with loads written
// as inline assembly, so that the compiler cannot sink them down to the LDS
// stores that consume them at the end of the step; the compiler does not track
// their completion, so that consumer waits for them explicitly, with every
// register they fill tied to the wait.
SSLP_DEVICE u32x4 pinned_load16(const void* p) {
    u32x4 v;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
    return v;
}
SSLP_DEVICE uint32_t pinned_load4(const void* p) {
    uint32_t v;
    asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
    return v;
}
SSLP_DEVICE float dot4(f32x4 x, f32x4 y) {
    return fmaf(x.w, y.w, fmaf(x.z, y.z, fmaf(x.y, y.y, x.x * y.x)));
}
SSLP_DEVICE f32x4 axpy4(float s, f32x4 x, f32x4 y) {  // s x + y
    return f32x4{fmaf(s, x.x, y.x), fmaf(s, x.y, y.y), fmaf(s, x.z, y.z), fmaf(s, x.w, y.w)};
}
SSLP_DEVICE f32x4 scale4(float s, f32x4 x) { return f32x4{s * x.x, s * x.y, s * x.z, s * x.w}; }

// ---------------------------------------------------------------------------
// sweep kernel: one workgroup of NWAVE wavefronts per (b, h, 8-column slice),
// chunks in reverse.  Gathered rows sit in LDS at (q, t) -> q C + t as in the
// forward: q < W the write entries, q >= W the read entries.
// ---------------------------------------------------------------------------
template <typename io_t, class G>
__global__ __launch_bounds__(64 * NWAVE) void sdm_chunk_bwd_kernel(SdmBwdArgs a,
                                                                   const uint32_t* __restrict__ fplan,
                                                                   const uint32_t* __restrict__ bplan,
                                                                   int nslice, int total, int nch) {
    constexpr int CC = G::CC, NW = G::NW, NR = G::NR, NQ = G::NQ;
    constexpr int LPT = 64 / CC;   // compute lanes per token
    constexpr int CPL = CW / LPT;  // columns per compute lane
    // forward-plan words kept per chunk: the row offsets, then T and Bm
    constexpr int FOFF = 32 * G::OFFS_LD, FTM = FOFF, FBM = FOFF + CC * G::TB_LD;
    constexpr int FPC = FOFF + 2 * CC * G::TB_LD;
    constexpr int NP = 2 + NW + NR;
    constexpr int DWT = CW * (int)sizeof(io_t) / 4;  // dwords of a token's dy (or v) slice
    static_assert(FPC % 4 == 0 && FPC / 4 <= 64 * NWAVE && FOFF <= G::PL_COEF &&
                      G::PL_BM == G::PL_TM + CC * G::TB_LD && G::PL_TM % 4 == 0,
                  "forward-plan copy");
    static_assert(BPL_WORDS / 4 <= 2 * 64 * NWAVE && NE == 64 * NWAVE && CC * DWT <= 64 * NWAVE,
                  "one chunk's prefetch: two plan pieces, one weight of each kind per thread");
    static_assert(2 * NW * CC == 2 * 64 * NWAVE, "two 16-byte pieces of pre-write rows per thread");
    static_assert(JW == 4 && NW % NWAVE == 0, "sweep layout");

    __shared__ __align__(16) float gst[NQ * CC][CW];  // gradient-table rows of every entry
    __shared__ __align__(16) float mst[NR * CC][CW];  // table rows of the read entries
    __shared__ __align__(16) float pst[2][NW * CC][CW];  // pre-write rows of the writes, by chunk parity
    // plans and inputs, double-buffered by chunk parity
    __shared__ __align__(16) uint32_t fpl[2][FPC];
    __shared__ __align__(16) uint32_t bpl[2][BPL_WORDS];
    __shared__ float s_w[2][NE], s_e[2][NE];  // write / read weights [t][i]
    __shared__ float s_al[2][CC], s_be[2][CC];
    __shared__ __align__(16) float s_dy[2][CC][CW], s_v[2][CC][CW];
    __shared__ __align__(16) float s_res[CC][CW], s_dr[CC][CW];
    __shared__ __align__(16) float s_s[CC][CW];
    __shared__ __align__(16) float part[NWAVE][2][CC][CW];
    __shared__ float s_pa[NE][2], s_pb[NE][2], s_pw[NE][2], s_pe[NE][2];

    // XCD-aware placement as in the forward: 16 slices of a 128-column group per XCD
    const int id = blockIdx.x;
    const int xcd = id & 7, kq = id >> 3;
    const int L = (kq >> 4) * 128 + xcd * 16 + (kq & 15);
    if (L >= total) return;
    const int bh = L / nslice, slice = L - (L / nslice) * nslice;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col0 = slice * CW;
    const int T = a.T, H = a.H, dv = a.dv;
    const int b = bh / H, h = bh - (bh / H) * H;
    const bool shared = a.residual_mode == 0;
    const size_t tab0 = (size_t)bh * a.N * dv;
    const char* Mc = reinterpret_cast<const char*>(a.M + tab0);
    char* Mw = reinterpret_cast<char*>(a.M + tab0);
    const char* Gc = reinterpret_cast<const char*>(a.dM + tab0);
    char* Gw = reinterpret_cast<char*>(a.dM + tab0);
    const io_t* dyin = static_cast<const io_t*>(a.dy);
    const io_t* vin = static_cast<const io_t*>(a.v);
    io_t* dvout = static_cast<io_t*>(a.dv_out);

    // DMA lane mapping: lane l covers 16 bytes (half l%2) of row
    // (q = G::RPD j + (l/2) / C, t = (l/2) % C) of DMA j
    const int dh = lane & 1;
    const uint32_t colbyte = 4u * (uint32_t)(col0 + 4 * dh);
    // compute mapping: lane (t, qt) owns columns CPL qt .. CPL qt + CPL - 1 of token t
    const int ct = lane / LPT, qt = lane % LPT;
    const uint32_t row_end = (uint32_t)a.N * (uint32_t)dv * 4u;  // < 2^31 on this path

    // one chunk's plans and inputs: loaded by every thread (clamped, always
    // valid addresses), kept by the threads that own a piece
    struct Pref {
        u32x4 f, b0, b1, p0, p1;
        uint32_t w, e, al, be, dy, v;
    };
    // piece x of the pre-write rows: row x / 2 = i C + t, half x % 2
    auto saved_piece = [&](int t0n, int ntn, int x) -> const float* {
        const int row = x >> 1, i = row / CC, t = row - (row / CC) * CC;
        const int tc = t < ntn ? t : ntn - 1;
        return a.saved + ((((size_t)b * T + t0n + tc) * H + h) * NW + i) * dv + col0 + 4 * (x & 1);
    };
    auto prefetch = [&](int cn, Pref& r) {
        const int t0n = cn * CC;
        const int ntn = T - t0n < CC ? T - t0n : CC;
        const uint32_t* fp = fplan + ((size_t)bh * nch + cn) * PL_WORDS;
        const uint32_t* bp = bplan + ((size_t)bh * nch + cn) * BPL_WORDS;
        const int u = tid < FPC / 4 ? tid : FPC / 4 - 1;
        r.f = pinned_load16(u < FOFF / 4 ? fp + 4 * u : fp + G::PL_TM + 4 * (u - FOFF / 4));
        r.b0 = pinned_load16(bp + 4 * (tid < BPL_WORDS / 4 ? tid : BPL_WORDS / 4 - 1));
        r.b1 = pinned_load16(bp + 4 * (tid + 64 * NWAVE < BPL_WORDS / 4 ? tid + 64 * NWAVE
                                                                          : BPL_WORDS / 4 - 1));
        const int te = tid / NW < ntn ? tid / NW : ntn - 1, ie = tid % NW;
        const size_t bte = ((size_t)b * T + t0n + te) * H + h;
        r.w = pinned_load4(a.wt_w + bte * NW + ie);
        r.e = pinned_load4(a.wt_r + bte * NR + ie);
        const size_t btg = ((size_t)b * T + t0n + (tid < ntn ? tid : ntn - 1)) * H + h;
        r.al = pinned_load4(a.alpha + btg);
        r.be = pinned_load4(a.beta + btg);
        const int d = tid < CC * DWT ? tid : CC * DWT - 1;
        const int td = d / DWT < ntn ? d / DWT : ntn - 1;
        const size_t btd = ((size_t)b * T + t0n + td) * H + h;
        r.dy = pinned_load4(reinterpret_cast<const uint32_t*>(dyin + btd * dv + col0) + d % DWT);
        r.v = pinned_load4(reinterpret_cast<const uint32_t*>(vin + btd * dv + col0) + d % DWT);
        r.p0 = pinned_load16(saved_piece(t0n, ntn, tid));
        r.p1 = pinned_load16(saved_piece(t0n, ntn, tid + 64 * NWAVE));
    };
    auto commit = [&](int cn, Pref& r) {
        asm volatile("s_waitcnt vmcnt(0)"
                     : "+v"(r.f), "+v"(r.b0), "+v"(r.b1), "+v"(r.p0), "+v"(r.p1), "+v"(r.w),
                       "+v"(r.e), "+v"(r.al), "+v"(r.be), "+v"(r.dy), "+v"(r.v)
                     :
                     : "memory");
        const int nb = cn & 1;
        *reinterpret_cast<u32x4*>(&pst[nb][tid >> 1][4 * (tid & 1)]) = r.p0;
        *reinterpret_cast<u32x4*>(&pst[nb][(tid + 64 * NWAVE) >> 1][4 * (tid & 1)]) = r.p1;
        const int ntn = T - cn * CC < CC ? T - cn * CC : CC;
        if (tid < FPC / 4) *reinterpret_cast<u32x4*>(&fpl[nb][4 * tid]) = r.f;
        if (tid < BPL_WORDS / 4) *reinterpret_cast<u32x4*>(&bpl[nb][4 * tid]) = r.b0;
        if (tid + 64 * NWAVE < BPL_WORDS / 4)
            *reinterpret_cast<u32x4*>(&bpl[nb][4 * (tid + 64 * NWAVE)]) = r.b1;
        const bool okw = tid / NW < ntn;
        s_w[nb][tid] = okw ? __uint_as_float(r.w) : 0.f;
        s_e[nb][tid] = okw ? __uint_as_float(r.e) : 0.f;
        if (tid < CC) {
            s_al[nb][tid] = tid < ntn ? __uint_as_float(r.al) : 1.f;
            s_be[nb][tid] = tid < ntn ? __uint_as_float(r.be) : 0.f;
        }
        if (tid < CC * DWT) {
            const int t = tid / DWT, o = tid % DWT;
            const bool ok = t < ntn;
            if constexpr (sizeof(io_t) == 2) {
                s_dy[nb][t][2 * o] = ok ? bf16lo(r.dy) : 0.f;
                s_dy[nb][t][2 * o + 1] = ok ? bf16hi(r.dy) : 0.f;
                s_v[nb][t][2 * o] = ok ? bf16lo(r.v) : 0.f;
                s_v[nb][t][2 * o + 1] = ok ? bf16hi(r.v) : 0.f;
            } else {
                s_dy[nb][t][o] = ok ? __uint_as_float(r.dy) : 0.f;
                s_v[nb][t][o] = ok ? __uint_as_float(r.v) : 0.f;
            }
        }
    };
    {
        Pref r;
        prefetch(nch - 1, r);
        commit(nch - 1, r);
        __syncthreads();
    }

    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * CC;
        const int ntok = T - t0 < CC ? T - t0 : CC;
        const int cb = c & 1;

        // ---- row DMAs: gradient rows of all entries, table rows of the reads
        //      (DMAs j >= 16); the pre-write rows came with the prefetch ----
        {
            const uint32_t* ow = &fpl[cb][G::PL_OFFS + (lane >> 1) * G::OFFS_LD + wave * JW];
            const uint4 o = *reinterpret_cast<const uint4*>(ow);
            const uint32_t om[JW] = {o.x, o.y, o.z, o.w};
#pragma unroll
            for (int m = 0; m < JW; ++m) {
                const int j = wave + NWAVE * m;
                dma16(Gc + om[m] + colbyte, &gst[j * 32][0]);
                if (NWAVE * m >= 16) dma16(Mc + om[m] + colbyte, &mst[(j - 16) * 32][0]);
            }
        }
        wait_vm0();
        block_sync_lds();
        // the earlier chunk's plans, inputs and pre-write rows: in flight during
        // this step's arithmetic (issued after the wait above, so that no wait
        // of the compiler's, which does not see them, covers them)
        Pref pre;
        if (c > 0) prefetch(c - 1, pre);

        // ---- partial sums over this wave's write rows i = wave + NWAVE m:
        //      alpha w P (shared residual) and f G (u) ----
        {
            float rs[CPL], us[CPL];
#pragma unroll
            for (int k = 0; k < CPL; ++k) rs[k] = us[k] = 0.f;
            const float al = s_al[cb][ct];
#pragma unroll
            for (int m = 0; m < NW / NWAVE; ++m) {
                const int i = wave + NWAVE * m;
                const float aw = shared ? al * s_w[cb][ct * NW + i] : 0.f;
                const float f = __uint_as_float(bpl[cb][BPL_F + ct * NW + i]);
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    rs[k] = fmaf(aw, pst[cb][i * CC + ct][CPL * qt + k], rs[k]);
                    us[k] = fmaf(f, gst[i * CC + ct][CPL * qt + k], us[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                part[wave][0][ct][CPL * qt + k] = rs[k];
                part[wave][1][ct][CPL * qt + k] = us[k];
            }
        }
        __syncthreads();

        // ---- wave 0: residuals, u + Bm^T dy, dr = T^T (u + Bm^T dy) = dv ----
        if (wave == 0) {
            const bool ok = ct < ntok;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int cc = CPL * qt + k;
                float rsum = 0.f, usum = 0.f;
#pragma unroll
                for (int w = 0; w < NWAVE; ++w) {
                    rsum += part[w][0][ct][cc];
                    usum += part[w][1][ct][cc];
                }
                s_res[ct][cc] = ok ? (shared ? s_v[cb][ct][cc] - rsum : s_v[cb][ct][cc]) : 0.f;
                // Bm[tau][t] is zero for tau < t: the loop runs over every tau
                float z = usum;
#pragma unroll
                for (int tau = 0; tau < CC; ++tau)
                    z = fmaf(__uint_as_float(fpl[cb][FBM + tau * G::TB_LD + ct]), s_dy[cb][tau][cc], z);
                s_s[ct][cc] = z;
            }
            wave_sync();
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int cc = CPL * qt + k;
                float dr = 0.f;  // T lower triangular: T[tau][t] = 0 for tau < t
#pragma unroll
                for (int tau = 0; tau < CC; ++tau)
                    dr = fmaf(__uint_as_float(fpl[cb][FTM + tau * G::TB_LD + ct]), s_s[tau][cc], dr);
                s_dr[ct][cc] = dr;
                if (ok)
                    dvout[(((size_t)b * T + t0 + ct) * H + h) * dv + col0 + cc] = from_f32<io_t>(dr);
            }
        }
        __syncthreads();

        // ---- every slot's gradient row through its events (two lanes per
        //      slot), then each read's row value ----
        const int ng = (int)bpl[cb][BPL_NG];
        for (int task = tid; task < 2 * ng; task += 64 * NWAVE) {
            const int g = task >> 1, hf = task & 1;
            const int gs = (int)bpl[cb][BPL_GS + g], ge = (int)bpl[cb][BPL_GS + g + 1];
            const uint32_t ev0 = bpl[cb][BPL_EV + gs];
            const int q0 = ((ev0 >> 5) & 1u) ? NW + (int)(ev0 >> 6) : (int)(ev0 >> 6);
            const int r0 = q0 * CC + (int)(ev0 & 31u);
            f32x4 gr = *reinterpret_cast<const f32x4*>(&gst[r0][4 * hf]);
            const uint32_t off = fpl[cb][G::offs_word(q0, (int)(ev0 & 31u))];
            int firstw = -1;  // row of the slot's earliest write in the chunk
            for (int p = ge - 1; p >= gs; --p) {
                const uint32_t ev = bpl[cb][BPL_EV + p];
                const int t = (int)(ev & 31u), i = (int)(ev >> 6);
                const f32x4 dy4 = *reinterpret_cast<const f32x4*>(&s_dy[cb][t][4 * hf]);
                if ((ev >> 5) & 1u) {
                    gr = axpy4(s_e[cb][t * NR + i], dy4, gr);
                    continue;
                }
                const f32x4 P = *reinterpret_cast<const f32x4*>(&pst[cb][i * CC + t][4 * hf]);
                const f32x4 x = *reinterpret_cast<const f32x4*>(&s_res[t][4 * hf]);
                const f32x4 drt = *reinterpret_cast<const f32x4*>(&s_dr[t][4 * hf]);
                const float al = s_al[cb][t], be = s_be[cb][t], w = s_w[cb][t * NW + i];
                f32x4 dmt;
                float pb, pw;
                if (shared) {
                    dmt = axpy4(-w, drt, gr);
                    const float gx = dot4(gr, x);
                    pb = w * gx;
                    pw = be * gx - al * dot4(P, drt);
                } else {
                    dmt = scale4(1.f - be * w, gr);
                    const float gx = dot4(gr, axpy4(-al, P, x));
                    pb = w * gx;
                    pw = be * gx;
                }
                const int e = t * NW + i;
                s_pa[e][hf] = dot4(P, dmt);
                s_pb[e][hf] = pb;
                s_pw[e][hf] = pw;
                gr = scale4(al, dmt);
                firstw = i * CC + t;
            }
            if (off < row_end) {  // always, for a plan of this chunk; a guard on the stores
                *reinterpret_cast<f32x4*>(Gw + off + 16u * hf + 4u * col0) = gr;
                if (firstw >= 0)
                    *reinterpret_cast<f32x4*>(Mw + off + 16u * hf + 4u * col0) =
                        *reinterpret_cast<const f32x4*>(&pst[cb][firstw][4 * hf]);
            }
        }
        for (int task = tid; task < 2 * CC * NR; task += 64 * NWAVE) {
            const int er = task >> 1, hf = task & 1;
            const int t = er / NR, k = er - (er / NR) * NR;
            if (t >= ntok) continue;
            const uint32_t rec = bpl[cb][BPL_Y + er];
            const int tt = (int)((rec >> 2) & 31u), ii = (int)(rec >> 7);
            f32x4 y;
            if ((rec & 3u) == 0u) {
                y = *reinterpret_cast<const f32x4*>(&mst[k * CC + t][4 * hf]);
            } else {
                const f32x4 P = *reinterpret_cast<const f32x4*>(&pst[cb][ii * CC + tt][4 * hf]);
                if ((rec & 3u) == 1u) {
                    y = P;
                } else {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(&s_res[tt][4 * hf]);
                    const float al = s_al[cb][tt], bw = s_be[cb][tt] * s_w[cb][tt * NW + ii];
                    const float d = shared ? al : al * (1.f - bw);
                    y = axpy4(bw, x, scale4(d, P));
                }
            }
            s_pe[er][hf] = dot4(y, *reinterpret_cast<const f32x4*>(&s_dy[cb][t][4 * hf]));
        }
        __syncthreads();

        // ---- this slice's per-token partial sums (fixed order); a chunk without
        //      events (one holding an out-of-range slot) leaves zeros.  dalpha and
        //      dbeta: one wavefront per token adds its 2 W entry halves (lane l
        //      takes values l, l + 64, ..., then a butterfly over the lanes) ----
        for (int t = wave; t < ntok; t += NWAVE) {
            const float* fa = &s_pa[t * NW][0];
            const float* fb = &s_pb[t * NW][0];
            float sa = 0.f, sb = 0.f;
#pragma unroll
            for (int r = 0; r < 2 * NW / 64; ++r) {
                sa += fa[lane + 64 * r];
                sb += fb[lane + 64 * r];
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                sa += xor_lane_f(sa, m, lane);
                sb += xor_lane_f(sb, m, lane);
            }
            float* pp = a.part + ((((size_t)b * T + t0 + t) * H + h) * nslice + slice) * NP;
            if (lane == 0) {
                pp[0] = ng > 0 ? sa : 0.f;
                pp[1] = ng > 0 ? sb : 0.f;
            }
        }
        for (int x = tid; x < ntok * (NW + NR); x += 64 * NWAVE) {
            const int t = x / (NW + NR), j = x - (x / (NW + NR)) * (NW + NR);
            float s = 0.f;
            if (ng == 0) {
            } else if (j < NW) {
                s = s_pw[t * NW + j][0] + s_pw[t * NW + j][1];
            } else {
                s = s_pe[t * NR + j - NW][0] + s_pe[t * NR + j - NW][1];
            }
            a.part[((((size_t)b * T + t0 + t) * H + h) * nslice + slice) * NP + 2 + j] = s;
        }
        // the earlier chunk's plans and inputs into the other buffers; this
        // chunk's table and gradient stores land before its gathers are issued
        if (c > 0) commit(c - 1, pre);
        wait_vm0();
        __syncthreads();
    }
}

template <class G>
hipError_t launch_bwd(const SdmBwdArgs& a, uint32_t* fplan, uint32_t* bplan, hipStream_t st) {
    SdmUpdateArgs u{};
    u.B = a.B;
    u.T = a.T;
    u.H = a.H;
    u.N = a.N;
    u.dv = a.dv;
    u.W = a.W;
    u.R = a.R;
    u.dtype = a.dtype;
    u.residual_mode = a.residual_mode;
    u.idx_w = a.idx_w;
    u.wt_w = a.wt_w;
    u.idx_r = a.idx_r;
    u.wt_r = a.wt_r;
    u.alpha = a.alpha;
    u.beta = a.beta;
    u.err = a.err;
    hipError_t e = launch_sdm_chunk_plans(u, fplan, st);
    if (e != hipSuccess) return e;
    const int nch = (a.T + G::CC - 1) / G::CC;
    BwdPlanArgs pa{a.B, a.T, a.H, a.N, nch, a.residual_mode, a.idx_w, a.wt_w, a.idx_r,
                   a.alpha, a.beta, bplan};
    sdm_chunk_bwd_plan_kernel<G><<<(unsigned)(a.B * a.H * nch), 256, 0, st>>>(pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslice = a.dv / CW;
    const int total = a.B * a.H * nslice;
    const int grid = ((total + 127) / 128) * 128;
    if (a.dtype != 0)
        sdm_chunk_bwd_kernel<bf16_t, G><<<grid, 64 * NWAVE, 0, st>>>(a, fplan, bplan, nslice, total, nch);
    else
        sdm_chunk_bwd_kernel<float, G><<<grid, 64 * NWAVE, 0, st>>>(a, fplan, bplan, nslice, total, nch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_sdm_bwd_reduce(a, CW, st);
}

}  // namespace

size_t sdm_chunk_bwd_plan_bytes(int B, int T, int H, int W) {
    const int cc = W == 64 ? GeoW64::CC : GeoW32::CC;
    const long long nch = (T + cc - 1) / cc;
    return (size_t)B * H * nch * BPL_WORDS * 4;
}

hipError_t launch_sdm_backward_chunked(const SdmBwdArgs& a, void* fplan, void* bplan,
                                       hipStream_t st) {
    static_assert(kChunkBwdSliceCols == CW, "slice width of the chunked backward");
    uint32_t* fp = static_cast<uint32_t*>(fplan);
    uint32_t* bp = static_cast<uint32_t*>(bplan);
    if (a.W == 64) return launch_bwd<GeoW64>(a, fp, bp, st);
    return launch_bwd<GeoW32>(a, fp, bp, st);
}

}  // namespace sslp
