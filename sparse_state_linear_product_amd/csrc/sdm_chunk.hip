// K2 (chunk-parallel): the Sparse Delta Memory recurrence given the addressing,
// computed a chunk of tokens at a time (16 tokens with 32 write and 32 read
// rows each, or 8 tokens with 64 and 64).
//
// Same operation as the per-token kernel in sdm_update.hip (slides "Sparse
// Delta Memory: Scaling the State of Linear RNNs through Sparsity", Eqs.
// (3)-(5), with the shared-prediction figure form or the per-slot form of the
// residual); here the token recurrence is unrolled over a chunk of C tokens
// so that no per-token dependency chain remains.
//
// Within a chunk every quantity is linear in the chunk-start table M0 and the
// residuals.  For a slot s, let its write visits in the chunk be tokens
// tau_1 < tau_2 < ..., each visit multiplying the slot by a decay d (alpha_tau
// for the shared form, alpha_tau (1 - beta_tau w) for the per-slot form) and
// adding beta_tau w res_tau.  Then, with P(s, range) the product of d over the
// visits in the range:
//   shared form:  res_t = v_t - sum_i alpha_t w_ti M_{t-1}[n_ti]
//                 M_{t-1}[n] = P(n, <t) M0[n] + sum_{tau<t} P(n, (tau,t)) beta_tau w_tau,n res_tau
//   so (I + A) res = v - g, g_t = sum_i c_ti M0[n_ti], c_ti = alpha_t w_ti P(n_ti, <t),
//   A[t][tau] = sum over slots written by both: alpha_t w_ti P(n, (tau,t)) beta_tau w_tau,n;
//   per-slot form: res_t = v_t (A = 0, c = 0), the per-slot factor lives in d.
//   reads  y_t = sum_k e_tk M0[m_tk] + sum_{tau<=t} Bm[t][tau] res_tau
//   final  M_C[s] = P(s, all) M0[s] + sum_visits P(s, (tau, end]) beta_tau w res_tau,
//          formed at the slot's last visit by carrying M0[s] through its visits
//          in order (row <- d row + beta_tau w res_tau), which passes every
//          visit's pre-write row M_{tau-1}[s] on the way (kept for the backward
//          by undoing writes when the caller asks for them).
// A plan kernel derives, per (b, h, chunk), everything that does not depend on
// the table (row offsets, c, e, T = (I + A)^-1, Bm, each visit's decay and
// beta w, the visit order of every slot, and which rows of the NEXT chunk hold
// a slot this chunk writes); the apply kernel then streams the table: one
// workgroup per 8-column slice of a head gathers the chunk's C x (W + R) =
// 1024 rows with LDS-DMA (global_load_lds_dwordx4), forms g, h,
// res = T (v - g), y = h + Bm res, and writes every written slot once with its
// final value.
//
// Pipelining: the rows of chunk c+1 are DMA'd while chunk c is computed, i.e.
// before chunk c's write-back; rows of chunk c+1 that chunk c writes are then
// overwritten in LDS with their final values (the plan lists them), after the
// DMA has landed.  Rows written by earlier chunks were stored before the DMA
// was issued: every wavefront waits for its stores to complete before the
// barrier that ends a chunk step, and the DMAs of chunk c+2 are issued after
// it.  The plans run two chunks ahead; a chunk's plan is DMA'd after the solve
// of the step before the one that uses it, apart from that step's row burst.
#include "common.h"
#include "kernels.h"
#include "sdm_chunk.h"

namespace sslp {

namespace {

using namespace chunk;

struct PlanArgs {
    int B, T, H, N, dv, nch, mode;
    const int32_t* idx_w;
    const float* wt_w;
    const int32_t* idx_r;
    const float* wt_r;
    const float* alpha;
    const float* beta;
    uint32_t* plan;  // [B, H, nch, PL_WORDS]
    unsigned* err;   // set to 1 when a chunk holds a slot index outside [0, N); may be null
};

// ---------------------------------------------------------------------------
// plan kernel: one workgroup of 256 threads per (b, h, chunk)
// ---------------------------------------------------------------------------
template <class G>
__global__ __launch_bounds__(256) void sdm_chunk_plan_kernel(PlanArgs a) {
    constexpr int CC = G::CC, NW = G::NW, NR = G::NR, NQ = G::NQ, LOGNW = G::LOGNW;
    constexpr int PL_LAST = G::PL_LAST, PL_FIRST = G::PL_FIRST, PL_EXC = G::PL_EXC, PL_EXCB = G::PL_EXCB,
                  PL_HDR = G::PL_HDR;
    constexpr int PL_FIN = G::PL_FIN, PL_BM = G::PL_BM, PL_TM = G::PL_TM, TB_LD = G::TB_LD;
    __shared__ uint64_t key[NE];       // write entries sorted by (slot, token, rank)
    __shared__ float s_d[NE];          // decay of the visit at sorted position p
    __shared__ int s_gs[NE], s_ge[NE];  // slot group [gs, ge) of sorted position p
    __shared__ int s_pos[NE];          // sorted position of write entry e = t*NW + i
    __shared__ int s_scan[NE];         // group starts, then their inclusive prefix count
    __shared__ float s_ww[NE];         // write weights by entry
    __shared__ int s_ir[CC * NR];      // read slots by entry (-1: no token)
    __shared__ float s_wr[CC * NR];
    __shared__ int s_rgs[CC * NR], s_rend[CC * NR];  // write visits of a read slot up to its token
    __shared__ float s_al[CC], s_be[CC];
    __shared__ float s_A[CC][CC + 1];
    __shared__ int s_fcnt[NE], s_fbeg[NE], s_ffill[NE];
    __shared__ __align__(8) int s_fwdl[2 * NE];         // forward rows, grouped per slot (first
                                                        // the sort's exchange buffer)
    __shared__ int s_tot[8];                            // wavefront totals of the scans
    __shared__ uint32_t s_fm[NE / 32];                  // bit i of word e / 32: entry e is its slot's first visit
    __shared__ uint32_t s_rnz[NE / 32];                 // bit i of word e / 32: read entry e follows a write visit
    __shared__ float s_P[NE], s_f[NE];                  // decay and beta w, by entry
    __shared__ uint32_t s_first[NE], s_pk[NE];          // by entry (exception data)
    __shared__ int s_exc[NE];                           // exception flags, then their prefix count
    __shared__ uint32_t s_xt[NE];                       // extra records, by extra index
    __shared__ float s_xd[NE], s_xb[NE];

    const int tid = threadIdx.x;
    const int nch = a.nch;
    const int c = blockIdx.x % nch, bh = blockIdx.x / nch;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int t0 = c * CC;
    // S1: load the chunk's addressing (every load of a thread issued before any
    // is used).  A chunk holding a slot index outside [0, N) is planned as an
    // empty chunk: its tokens write nothing and read nothing (y = 0), and no
    // row offset outside the table reaches the apply kernel.
    static_assert(NE % 256 == 0, "whole passes of the 256 threads");
    const uint64_t NONE = ~0ull;
    __shared__ int s_bad;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    const int nt = a.T - t0 < CC ? a.T - t0 : CC;
    bool bad = false;
    // (rows past the sequence end load the last token's values, then unused)
    unsigned sw[NE / 256], sr[NE / 256];
    float ww[NE / 256], wr[NE / 256], al = 1.f, be = 0.f;
#pragma unroll
    for (int r = 0; r < NE / 256; ++r) {
        const int e = tid + 256 * r;
        const int t = e >> LOGNW < nt ? e >> LOGNW : nt - 1, i = e & (NW - 1);
        const size_t bth = ((size_t)b * a.T + t0 + t) * a.H + h;
        sw[r] = (unsigned)a.idx_w[bth * NW + i];
        sr[r] = (unsigned)a.idx_r[bth * NR + i];
        ww[r] = a.wt_w[bth * NW + i];
        wr[r] = a.wt_r[bth * NR + i];
    }
    if (tid < CC) {
        const size_t bth = ((size_t)b * a.T + t0 + (tid < nt ? tid : nt - 1)) * a.H + h;
        al = a.alpha[bth];
        be = a.beta[bth];
    }
#pragma unroll
    for (int r = 0; r < NE / 256; ++r) {
        const int e = tid + 256 * r;
        if ((e >> LOGNW) < nt) {
            bad |= sw[r] >= (unsigned)a.N || sr[r] >= (unsigned)a.N;
            key[e] = ((uint64_t)sw[r] << 9) | (uint64_t)e;
            s_ww[e] = ww[r];
            s_ir[e] = (int)sr[r];
            s_wr[e] = wr[r];
        } else {
            key[e] = NONE;
            s_ww[e] = 0.f;
            s_ir[e] = -1;
            s_wr[e] = 0.f;
        }
        s_fcnt[e] = 0;
        s_ffill[e] = 0;
    }
    if (tid < CC) {
        const bool ok = tid < nt;
        s_al[tid] = ok ? al : 1.f;
        s_be[tid] = ok ? be : 0.f;
    }
    if (bad) s_bad = 1;
    __syncthreads();
    if (s_bad) {  // (a uniform branch) plan the chunk as empty
        if (tid == 0 && a.err != nullptr) atomicOr(a.err, 1u);
#pragma unroll
        for (int r = 0; r < NE / 256; ++r) {
            const int e = tid + 256 * r;
            key[e] = NONE;
            s_ww[e] = 0.f;
            s_ir[e] = -1;
            s_wr[e] = 0.f;
        }
        if (tid < CC) {
            s_al[tid] = 1.f;
            s_be[tid] = 0.f;
        }
        __syncthreads();
    }
    const int ntok = s_bad ? 0 : nt;
    uint32_t* out = a.plan + (size_t)blockIdx.x * PL_WORDS;

    // S2: bitonic sort of the 512 keys, ascending
    static_assert(NE == 512, "two keys per thread");
    {
        uint64_t kr[2] = {key[tid], key[tid + 256]};
        chunk::block_sort_asc<2>(kr, key, reinterpret_cast<uint64_t*>(s_fwdl));
        __syncthreads();
    }

    // S3: groups of equal slot (a slot is written at most once per token, so
    // a group lists its visits in token order), per-visit decays
    for (int p = tid; p < NE; p += 256) {
        const uint64_t kp = key[p];
        const bool valid = kp != NONE;
        const int e = (int)(kp & 511u);
        const int t = e >> LOGNW;
        int gs = p, ge = p + 1;
        if (valid) {
            const uint64_t sl = kp >> 9;
            while (gs > 0 && (key[gs - 1] >> 9) == sl) --gs;
            while (ge < NE && key[ge] != NONE && (key[ge] >> 9) == sl) ++ge;
            s_pos[e] = p;
            s_d[p] = a.mode == 0 ? s_al[t] : s_al[t] * (1.f - s_be[t] * s_ww[e]);
        } else {
            s_d[p] = 1.f;
        }
        s_gs[p] = gs;
        s_ge[p] = ge;
        s_scan[p] = (valid && gs == p) ? 1 : 0;
    }
    __syncthreads();
    // inclusive prefix count of group starts
    {
        int v[2] = {s_scan[tid], s_scan[tid + 256]};
        chunk::block_scan<2>(v, s_tot);
        s_scan[tid] = v[0];
        s_scan[tid + 256] = v[1];
        __syncthreads();
    }

    // S4: read entries: the write visits of their slot at or before their token
    // (two entries per thread, their lower bounds of (slot << 9) among the
    // sorted keys found side by side in log2(NE) fixed steps)
    static_assert(CC * NR == 2 * 256, "two read entries per thread");
    {
        const int lane = tid & 63;
        int sl[2], lo[2] = {0, 0};
        uint64_t want[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            sl[r] = s_ir[tid + 256 * r];
            want[r] = (uint64_t)(uint32_t)sl[r] << 9;
        }
#pragma unroll
        for (int step = NE / 2; step >= 1; step >>= 1) {
#pragma unroll
            for (int r = 0; r < 2; ++r) lo[r] += key[lo[r] + step - 1] < want[r] ? step : 0;
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int e = tid + 256 * r;
            const int t = e >> LOGNW;
            int rgs = 0, rend = 0;
            if (sl[r] >= 0 && lo[r] < NE && key[lo[r]] != NONE &&
                (key[lo[r]] >> 9) == (uint64_t)(uint32_t)sl[r]) {
                rgs = lo[r];
                rend = lo[r];
                const int ge = s_ge[lo[r]];
                while (rend < ge && (int)((key[rend] & 511u) >> LOGNW) <= t) ++rend;
            }
            s_rgs[e] = rgs;
            s_rend[e] = rend;
            const uint64_t bal = __ballot(rend > rgs);
            if ((lane & 31) == 0) s_rnz[e >> 5] = (uint32_t)(bal >> (lane & 32));
        }
    }

    // S5: forward targets: rows of the next chunk whose slot this chunk writes
    // (counted per group, at the group's last visit)
    const int t1 = t0 + CC;
    const int ntok1 = c + 1 < nch ? (a.T - t1 < CC ? a.T - t1 : CC) : 0;
    // (the four rows of a thread loaded first, then searched side by side)
    int fgrp[4];
    {
        int slv[4], lo[4];
        uint64_t want[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int ne = tid + 256 * x;  // 0..1023 as (t, q)
            const int t = ne / NQ, q = ne & (NQ - 1);
            slv[x] = -1;
            if (t < ntok1) {
                const size_t bth = ((size_t)b * a.T + t1 + t) * a.H + h;
                slv[x] = q < NW ? a.idx_w[bth * NW + q] : a.idx_r[bth * NR + (q - NW)];
            }
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            want[x] = (uint64_t)(uint32_t)slv[x] << 9;
            lo[x] = 0;
        }
#pragma unroll
        for (int step = NE / 2; step >= 1; step >>= 1) {
#pragma unroll
            for (int x = 0; x < 4; ++x) lo[x] += key[lo[x] + step - 1] < want[x] ? step : 0;
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int t = (tid + 256 * x) / NQ;
            fgrp[x] = -1;
            if (t < ntok1 && lo[x] < NE && key[lo[x]] != NONE &&
                (key[lo[x]] >> 9) == (uint64_t)(uint32_t)slv[x]) {
                fgrp[x] = s_ge[lo[x]] - 1;
                atomicAdd(&s_fcnt[fgrp[x]], 1);
            }
        }
    }
    __syncthreads();
    // inclusive prefix of the forward counts over sorted positions
    {
        int v[2] = {s_fcnt[tid], s_fcnt[tid + 256]};
        chunk::block_scan<2>(v, s_tot);
        s_fbeg[tid] = v[0];
        s_fbeg[tid + 256] = v[1];
        __syncthreads();
    }
    for (int x = 0; x < 4; ++x) {
        if (fgrp[x] >= 0) {
            const int ne = tid + 256 * x;
            const int t = ne / NQ, q = ne & (NQ - 1);
            const int g = fgrp[x];
            const int slot = atomicAdd(&s_ffill[g], 1);
            s_fwdl[s_fbeg[g] - s_fcnt[g] + slot] = q * CC + t;
        }
    }

    // S6: per write entry: gather coefficient, the visit's decay and beta w; at a
    // slot's last visit, its earlier visits in order (the final value and the
    // pre-write rows follow them as a chain from the chunk-start row)
    for (int e = tid; e < NE; e += 256) {
        const int t = e >> LOGNW, i = e & (NW - 1);
        s_P[e] = 0.f;
        s_f[e] = 0.f;
        s_exc[e] = 0;
        s_first[e] = 0u;
        s_pk[e] = 0u;
        if (t >= ntok) {
            out[G::coef_word(t, i)] = 0u;
            continue;
        }
        const int p = s_pos[e];
        const int gs = s_gs[p], ge = s_ge[p];
        float pre = 1.f;
        for (int l = gs; l < p; ++l) pre *= s_d[l];
        const float w = s_ww[e];
        out[G::coef_word(t, i)] = __float_as_uint(a.mode == 0 ? s_al[t] * w * pre : 0.f);
        s_P[e] = s_d[p];
        s_f[e] = s_be[t] * w;
        if (p != ge - 1) continue;  // the slot is written once, at its last visit
        const int xstart = gs - (s_scan[gs] - 1);  // earlier visits of earlier groups
        const int xcnt = ge - gs - 1;
        for (int l = gs; l < ge - 1; ++l) {
            const int el = (int)(key[l] & 511u);
            s_xt[xstart + (l - gs)] = (uint32_t)(el >> LOGNW) | ((uint32_t)(el & (NW - 1)) << 8);
            s_xd[xstart + (l - gs)] = s_d[l];
            s_xb[xstart + (l - gs)] = s_be[el >> LOGNW] * s_ww[el];
        }
        const int fcnt = s_fcnt[p], fbeg = s_fbeg[p] - fcnt;
        if (xcnt > 0 || fcnt > 0) {
            const int e1 = (int)(key[gs] & 511u);
            s_exc[e] = 1;
            s_first[e] = (uint32_t)((e1 & (NW - 1)) * CC + (e1 >> LOGNW));
            s_pk[e] = (uint32_t)xstart | ((uint32_t)xcnt << 9) | ((uint32_t)fbeg << 14) |
                      ((uint32_t)fcnt << 24);
        }
    }
    __syncthreads();
    // token masks of last and first visits and of exception records, word wd of
    // token t covering entries (t, 32 wd + i)
    // (one entry per lane, words from wavefront ballots: word e / 32 holds
    // entries 32 (e / 32) .. + 31, i.e. word t * NMW + wd of token t)
    {
        const int lane = tid & 63;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int e = tid + 256 * r;
            const bool valid = (e >> LOGNW) < ntok;
            const int p = valid ? s_pos[e] : 0;
            const uint64_t bl = __ballot(valid && s_ge[p] - 1 == p);
            const uint64_t bf = __ballot(valid && s_gs[p] == p);
            const uint64_t bx = __ballot(valid && s_exc[e] != 0);
            if ((lane & 31) == 0) {
                const int wdi = e >> 5, sh = lane & 32;
                out[PL_LAST + wdi] = (uint32_t)(bl >> sh);
                out[PL_FIRST + wdi] = (uint32_t)(bf >> sh);
                out[PL_EXC + wdi] = (uint32_t)(bx >> sh);
                s_fm[wdi] = (uint32_t)(bf >> sh);
            }
        }
    }
    __syncthreads();
    // inclusive prefix count of exception flags (entry order)
    {
        int v[2] = {s_exc[tid], s_exc[tid + 256]};
        chunk::block_scan<2>(v, s_tot);
        s_exc[tid] = v[0];
        s_exc[tid + 256] = v[1];
        __syncthreads();
    }
    {
        const int n_exc = s_exc[NE - 1];
        const int extra_base = 2 * n_exc;
        const int nxp = ntok * NW - s_scan[NE - 1];  // valid entries - slot groups = extra pairs
        const int fwd_base = extra_base + 3 * nxp;
        const int n_fwd = s_fbeg[NE - 1];
        if (tid == 0) {
            out[PL_HDR + 0] = (uint32_t)extra_base;
            out[PL_HDR + 1] = (uint32_t)fwd_base;
            out[PL_HDR + 2] = (uint32_t)n_exc;
            out[PL_HDR + 3] = (uint32_t)(fwd_base + n_fwd);
        }
        if (tid < CC) out[PL_EXCB + tid] = (uint32_t)(tid == 0 ? 0 : s_exc[tid * NW - 1]);
        for (int e = tid; e < NE; e += 256) {
            const int t = e >> LOGNW, i = e & (NW - 1);
            out[PL_FIN + (i * CC + t) * 2 + 0] = __float_as_uint(s_P[e]);
            out[PL_FIN + (i * CC + t) * 2 + 1] = __float_as_uint(s_f[e]);
            const int prev = e == 0 ? 0 : s_exc[e - 1];
            if (s_exc[e] != prev) {  // entry e has exception record `prev`
                out[PL_TAIL + 2 * prev + 0] = s_first[e];
                out[PL_TAIL + 2 * prev + 1] = s_pk[e];
            }
        }
        for (int x = tid; x < nxp; x += 256) {
            out[PL_TAIL + extra_base + 3 * x + 0] = s_xt[x];
            out[PL_TAIL + extra_base + 3 * x + 1] = __float_as_uint(s_xd[x]);
            out[PL_TAIL + extra_base + 3 * x + 2] = __float_as_uint(s_xb[x]);
        }
        for (int x = tid; x < n_fwd; x += 256) out[PL_TAIL + fwd_base + x] = (uint32_t)s_fwdl[x];
    }

    // S7: read coefficients e = w * P(m, <= t)
    for (int e = tid; e < CC * NR; e += 256) {
        const int t = e >> LOGNW, k = e & (NR - 1);
        float pr = 1.f;
        for (int l = s_rgs[e]; l < s_rend[e]; ++l) pr *= s_d[l];
        out[G::coef_word(t, NW + k)] = __float_as_uint(t < ntok ? s_wr[e] * pr : 0.f);
    }

    // S8: A[t][tau] (shared form) and Bm[t][tau], one thread per pair, sums in a fixed order
    if (tid < CC * CC) {
        const int t = tid / CC, tau = tid % CC;
        float av = 0.f, bv = 0.f;
        if (t < ntok && tau <= t) {
            // (only entries with an earlier visit of their slot in the chunk,
            // and read entries after a write visit, contribute: the others
            // are skipped by their mask bits, in the same entry order)
            if (a.mode == 0 && tau < t) {
                for (int wd = 0; wd < G::NMW; ++wd) {
                    for (uint32_t todo = ~s_fm[t * G::NMW + wd]; todo != 0u; todo &= todo - 1u) {
                        const int e = t * NW + 32 * wd + __builtin_ctz(todo);
                        const int p = s_pos[e];
                        float between = 1.f;  // decays of the visits strictly between
                        for (int l = p - 1; l >= s_gs[p]; --l) {
                            const int el = (int)(key[l] & 511u);
                            if ((el >> LOGNW) == tau) {
                                av += s_al[t] * s_ww[e] * between * s_be[tau] * s_ww[el];
                                break;
                            }
                            between *= s_d[l];
                        }
                    }
                }
            }
            for (int wd = 0; wd < NR / 32; ++wd) {
                for (uint32_t todo = s_rnz[t * (NR / 32) + wd]; todo != 0u; todo &= todo - 1u) {
                    const int e = t * NR + 32 * wd + __builtin_ctz(todo);
                    float after = 1.f;  // decays of the visits after tau's, up to token t
                    for (int l = s_rend[e] - 1; l >= s_rgs[e]; --l) {
                        const int el = (int)(key[l] & 511u);
                        if ((el >> LOGNW) == tau) {
                            bv += s_wr[e] * after * s_be[tau] * s_ww[el];
                            break;
                        }
                        after *= s_d[l];
                    }
                }
            }
        }
        s_A[t][tau] = av;
        out[PL_BM + t * TB_LD + tau] = __float_as_uint(bv);
    }
    __syncthreads();

    // S9: T = (I + A)^-1 by forward substitution, one column per thread
    if (tid < CC) {
        const int j = tid;
        float col[CC];
#pragma unroll
        for (int t = 0; t < CC; ++t) {
            float v = (t == j) ? 1.f : 0.f;
#pragma unroll
            for (int tau = 0; tau < t; ++tau) v -= s_A[t][tau] * col[tau];
            col[t] = v;
            out[PL_TM + t * TB_LD + j] = __float_as_uint(v);
        }
    }

    // S10: byte offsets of every staged row (the slots from LDS: a write
    // entry's in its sorted key, a read entry's in s_ir)
    for (int x = tid; x < CC * NQ; x += 256) {
        const int t = x / NQ, q = x & (NQ - 1);
        uint32_t off = 0u;
        if (t < ntok) {
            const uint32_t sl = q < NW ? (uint32_t)(key[s_pos[t * NW + q]] >> 9)
                                       : (uint32_t)s_ir[t * NR + (q - NW)];
            off = sl * (uint32_t)a.dv * 4u;
        }
        out[G::offs_word(q, t)] = off;
    }
}

// ---------------------------------------------------------------------------
// apply kernel: one workgroup of NWAVE wavefronts per (b, h, 8-column slice).
// DMA j (j = 0..31) stages rows q = RPD j .. RPD j + RPD - 1 of the chunk's C
// tokens (RPD = 32 / C); wave w owns the DMAs j = w + NWAVE m: it gathers those
// rows, forms the partial row sums over them, and writes back the write rows
// among them (j < 16).  Several wavefronts per CU keep that many times more
// gathers in flight than one, and split the compute.
// ---------------------------------------------------------------------------
template <typename io_t, class G, bool SAVE>
__global__ __launch_bounds__(64 * NWAVE) void sdm_chunk_apply_kernel(SdmUpdateArgs a,
                                                                     const uint32_t* __restrict__ plan,
                                                                     int nslice, int total, int nch) {
    constexpr int CC = G::CC, NQ = G::NQ, RPD = G::RPD, NMW = G::NMW;
    constexpr int LPT = 64 / CC;                     // compute lanes per token
    constexpr int CPL = CW / LPT;                    // columns per compute lane (2 or 1)
    constexpr int VB = CC * CW * (int)sizeof(io_t);  // value bytes of a chunk
    constexpr int VBP = (VB + 255) / 256 * 256;      // padded to whole dword DMAs
    constexpr int VDMA = VBP / 256;                  // dword DMAs per chunk
    constexpr int ROWB = CC * CW * 4;                // bytes of one staged row index q (C tokens)
    constexpr int NPIECE = PL_DMA_WORDS / 256;       // 1 KB plan pieces per chunk
    constexpr int NWD = 16;                          // DMAs holding write rows (j < 16)
    constexpr int WB = NWD / NWAVE;                  // write-row DMAs per wave
    using cv = typename VecOf<CPL>::type;            // a compute lane's columns
    using mask_t = typename std::conditional<NMW == 1, uint32_t, uint64_t>::type;
    static_assert(RPD * NWD == G::NW && NWD % NWAVE == 0, "write rows fill the first 16 DMAs");
    static_assert(CPL * LPT == CW && (CPL == 1 || CPL == 2), "compute mapping");
    static_assert(NPIECE % NWAVE == 0 && JW == 4 && WB >= 1, "work split over the wavefronts");

    __shared__ __align__(16) float stage[2][NQ * CC][CW];  // rows (q, t) at q*16 + t
    __shared__ __align__(16) uint32_t pbuf[3][PL_DMA_WORDS];
    __shared__ __align__(16) uint32_t vbuf[2][VBP / 4];
    __shared__ __align__(16) float part[NWAVE][2][CC][CW];  // partial g, h per wave
    __shared__ __align__(16) float xr[CC][CW];             // v - g
    __shared__ __align__(16) float xs[CC][CW];             // residuals

    // XCD-aware placement: the 16 slices of a 128-column group share an XCD
    const int id = blockIdx.x;
    const int xcd = id & 7, kq = id >> 3;
    const int L = (kq >> 4) * 128 + xcd * 16 + (kq & 15);
    if (L >= total) return;
    const int bh = L / nslice, slice = L - (L / nslice) * nslice;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col0 = slice * CW;
    const int T = a.T, H = a.H, dv = a.dv;
    const int b = bh / H, h = bh - (bh / H) * H;
    const char* tabc = reinterpret_cast<const char*>(a.M + (size_t)bh * a.N * dv);
    char* tabw = reinterpret_cast<char*>(a.M + (size_t)bh * a.N * dv);
    const char* vin = static_cast<const char*>(a.v);
    char* yout = static_cast<char*>(a.y);
    const uint32_t* planb = plan + (size_t)bh * nch * PL_WORDS;

    const uint32_t stage0 = lds_addr(&stage[0][0][0]);
    const uint32_t pbuf0 = lds_addr(&pbuf[0][0]);
    const uint32_t vbuf0 = lds_addr(&vbuf[0][0]);
    const uint32_t part0 = lds_addr(&part[0][0][0][0]);
    const uint32_t xr0 = lds_addr(&xr[0][0]);
    const uint32_t xs0 = lds_addr(&xs[0][0]);
    constexpr uint32_t STAGE_BYTES = NQ * CC * CW * 4;
    constexpr uint32_t PLAN_BYTES = PL_DMA_WORDS * 4;

    // DMA lane mapping (also the write-back mapping): lane l covers 16 bytes
    // (half l%2) of row (q = RPD j + (l/2) / C, t = (l/2) % C)
    const int dq = (lane >> 1) / CC, dt = (lane >> 1) % CC, dh = lane & 1;
    const uint32_t colbyte = 4u * (uint32_t)(col0 + 4 * dh);
    // this lane's JW row offsets for its wave's DMAs j = wave + NWAVE m
    const uint32_t offs_lane = 4u * (uint32_t)(G::PL_OFFS + (lane >> 1) * G::OFFS_LD + wave * JW);

    auto plan_dma = [&](int ch) {  // this wave's pieces of chunk ch's plan -> pbuf[ch % 3]
        const uint32_t* src = planb + (size_t)ch * PL_WORDS;
        uint32_t* dst = &pbuf[ch % 3][0];
#pragma unroll
        for (int k = 0; k < NPIECE / NWAVE; ++k) {
            const int s = wave + NWAVE * k;
            dma16(src + s * 256 + 4 * lane, dst + s * 256);
        }
    };
    auto row_dma = [&](int ch) {  // this wave's rows of chunk ch -> stage[ch % 2]
        u32x4 o = lds_u32x4(pbuf0 + (uint32_t)(ch % 3) * PLAN_BYTES + offs_lane);
        lds_wait(o);
        float* dst = &stage[ch % 2][0][0];
#pragma unroll
        for (int m = 0; m < JW; ++m) dma16(tabc + o[m] + colbyte, dst + (wave + NWAVE * m) * 256);
        if (wave == NWAVE - 1) {
            const int tb = ch * CC;
#pragma unroll
            for (int s = 0; s < VDMA; ++s) {
                const int byte = (s * 64 + lane) * 4;  // bytes past VB fill the padding
                const int tt = tb + byte / (CW * (int)sizeof(io_t));
                const char* src = byte < VB && tt < T ? vin + ((((size_t)b * T + tt) * H + h) * dv + col0) * sizeof(io_t) +
                                               byte % (CW * (int)sizeof(io_t))
                                         : vin;
                dma4(src, &vbuf[ch % 2][s * 64]);
            }
        }
    };

    // -- prologue: plans of chunks 0 and 1, rows and values of chunk 0 --
    plan_dma(0);
    if (nch > 1) plan_dma(1);
    wait_vm0();
    block_sync_lds();
    row_dma(0);
    wait_vm0();
    block_sync_lds();

    // compute mapping: lane (t, qt) = (lane / LPT, lane % LPT) owns the CPL
    // columns CPL qt .. CPL qt + CPL - 1 of token t
    const int ct = lane / LPT, qt = lane % LPT;
    const uint32_t cofs = (uint32_t)((ct * CW + CPL * qt) * 4);  // (token, columns) in a row
    const uint32_t xq = (uint32_t)(CPL * qt * 4);

    for (int c = 0; c < nch; ++c) {
        const int ntok = T - c * CC < CC ? T - c * CC : CC;
        const uint32_t P = pbuf0 + (uint32_t)(c % 3) * PLAN_BYTES;
        const uint32_t S = stage0 + (uint32_t)(c % 2) * STAGE_BYTES;
        if (c + 1 < nch) row_dma(c + 1);

        // ---- partial g, h over this wave's rows: q = RPD j + r for j = wave + NWAVE m ----
        {
            typename VecOf<RPD>::type cf[JW];
            cv rw[RPD * JW];
            const uint32_t cfa = P + 4u * (uint32_t)G::coef_word(ct, RPD * wave);  // + RPD NWAVE words per m
            const uint32_t rowa = S + cofs + (uint32_t)(RPD * wave * ROWB);        // + RPD NWAVE rows per m
            static_for<JW>([&](auto m) {
                constexpr int M = decltype(m)::value;
                cf[M] = lds_vec<RPD, 4 * RPD * NWAVE * M>(cfa);
                static_for<RPD>([&](auto r) {
                    constexpr int R = decltype(r)::value;
                    rw[RPD * M + R] = lds_vec<CPL, (RPD * NWAVE * M + R) * ROWB>(rowa);
                });
            });
            lds_wait();
            tie_all(cf);
            tie_all(rw);
            float g[CPL], hh[CPL];
#pragma unroll
            for (int k = 0; k < CPL; ++k) g[k] = hh[k] = 0.f;
            static_for<JW>([&](auto m) {
                constexpr int M = decltype(m)::value;
                auto step = [&](float(&acc)[CPL]) {
#pragma unroll
                    for (int r = 0; r < RPD; ++r)
#pragma unroll
                        for (int k = 0; k < CPL; ++k)
                            acc[k] = fmaf(elem(cf[M], r), elem(rw[RPD * M + r], k), acc[k]);
                };
                // DMA j = wave + NWAVE M holds write rows iff j < 16, i.e. NWAVE M < 16
                if constexpr (NWAVE * M < NWD) step(g);
                else step(hh);
            });
            lds_write_cols(part0 + (uint32_t)((wave * 2 + 0) * CC * CW * 4) + cofs, g);
            lds_write_cols(part0 + (uint32_t)((wave * 2 + 1) * CC * CW * 4) + cofs, hh);
        }
        block_sync_lds();

        // ---- wave 0: g, h, r = v - g, res = T r, y = h + Bm res ----
        const bool tok_ok = ct < ntok;
        if (wave == 0) {
            cv pg[NWAVE], ph[NWAVE];
            static_for<NWAVE>([&](auto w) {
                pg[w] = lds_vec<CPL, (w * 2 + 0) * CC * CW * 4>(part0 + cofs);
                ph[w] = lds_vec<CPL, (w * 2 + 1) * CC * CW * 4>(part0 + cofs);
            });
            float vv[CPL];
            const uint32_t va = vbuf0 + (uint32_t)((c % 2) * VBP + (ct * CW + CPL * qt) * (int)sizeof(io_t));
            if constexpr (sizeof(io_t) == 2 && CPL == 2) {
                uint32_t w = lds_u32(va);
                lds_wait(w);
                vv[0] = bf16lo(w);
                vv[1] = bf16hi(w);
            } else if constexpr (sizeof(io_t) == 2) {
                uint32_t w = lds_u16(va);
                lds_wait(w);
                vv[0] = bf16lo(w);
            } else {
                cv w = lds_vec<CPL>(va);
                lds_wait(w);
#pragma unroll
                for (int k = 0; k < CPL; ++k) vv[k] = elem(w, k);
            }
            tie_all(pg);
            tie_all(ph);
            float gs[CPL], hs[CPL], r[CPL];
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                gs[k] = hs[k] = 0.f;
#pragma unroll
                for (int w = 0; w < NWAVE; ++w) {
                    gs[k] += elem(pg[w], k);
                    hs[k] += elem(ph[w], k);
                }
                r[k] = tok_ok ? vv[k] - gs[k] : 0.f;
            }
            lds_write_cols(xr0 + cofs, r);
            float res[CPL];
            {
                f32x4 tm[CC / 4];
                cv rr[CC];
                const uint32_t ta = P + 4u * (uint32_t)(G::PL_TM + ct * G::TB_LD);
                static_for<CC / 4>([&](auto k) { tm[k] = lds_f32x4<16 * k>(ta); });
                static_for<CC>([&](auto k) { rr[k] = lds_vec<CPL, k * CW * 4>(xr0 + xq); });
                lds_wait();
                tie_all(tm);
                tie_all(rr);
                float sacc[CPL][2];
#pragma unroll
                for (int k = 0; k < CPL; ++k) sacc[k][0] = sacc[k][1] = 0.f;
#pragma unroll
                for (int tau = 0; tau < CC; ++tau) {
                    const float tv = tm[tau >> 2][tau & 3];
#pragma unroll
                    for (int k = 0; k < CPL; ++k)
                        sacc[k][tau & 1] = fmaf(tv, elem(rr[tau], k), sacc[k][tau & 1]);
                }
#pragma unroll
                for (int k = 0; k < CPL; ++k) res[k] = sacc[k][0] + sacc[k][1];
            }
            lds_write_cols(xs0 + cofs, res);
            {
                f32x4 bm[CC / 4];
                cv rs[CC];
                const uint32_t ba = P + 4u * (uint32_t)(G::PL_BM + ct * G::TB_LD);
                static_for<CC / 4>([&](auto k) { bm[k] = lds_f32x4<16 * k>(ba); });
                static_for<CC>([&](auto k) { rs[k] = lds_vec<CPL, k * CW * 4>(xs0 + xq); });
                lds_wait();
                tie_all(bm);
                tie_all(rs);
                float sacc[CPL][2], yv[CPL];
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    sacc[k][0] = hs[k];
                    sacc[k][1] = 0.f;
                }
#pragma unroll
                for (int tau = 0; tau < CC; ++tau) {
                    const float bv = bm[tau >> 2][tau & 3];
#pragma unroll
                    for (int k = 0; k < CPL; ++k)
                        sacc[k][tau & 1] = fmaf(bv, elem(rs[tau], k), sacc[k][tau & 1]);
                }
#pragma unroll
                for (int k = 0; k < CPL; ++k) yv[k] = sacc[k][0] + sacc[k][1];
                if (tok_ok) {
                    char* dst = yout + ((((size_t)b * T + c * CC + ct) * H + h) * dv + col0 + CPL * qt) * sizeof(io_t);
                    if constexpr (sizeof(io_t) == 2 && CPL == 2) {
                        const uint32_t w = (uint32_t)f32_to_bf16(yv[0]).bits | ((uint32_t)f32_to_bf16(yv[1]).bits << 16);
                        *reinterpret_cast<uint32_t*>(dst) = w;
                    } else if constexpr (sizeof(io_t) == 2) {
                        *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(yv[0]).bits;
                    } else if constexpr (CPL == 2) {
                        *reinterpret_cast<float2*>(dst) = make_float2(yv[0], yv[1]);
                    } else {
                        *reinterpret_cast<float*>(dst) = yv[0];
                    }
                }
            }
        }
        block_sync_lds();

        // ---- write-back of this wave's write rows (j = wave + NWAVE m < 16): each
        //      written slot once, at its last visit; entries with an exception
        //      record were visited earlier in the chunk or feed the next chunk.
        //      With SAVE (a.saved set), every write entry's pre-write row too: a
        //      first visit stores the chunk-start row, a last visit the rows of
        //      the later visits, as it walks the slot's visits in order ----
        // the plan of chunk c+2 (its buffer was last read in step c-1): issued
        // here rather than with the rows at the top of the step, where the
        // wavefronts stalled on both bursts of requests at once (2.30 -> 2.25 ms)
        if (c + 2 < nch) plan_dma(c + 2);
        const bool wb_ok = dt < ntok;
        const uint32_t* tailg = planb + (size_t)c * PL_WORDS + PL_TAIL;
        auto tail = [&](uint32_t k) -> uint32_t {  // tail word k (LDS window, else memory)
            if (k < (uint32_t)PL_TAILWIN) {
                uint32_t v = lds_u32(P + 4u * (PL_TAIL + k));
                lds_wait(v);
                return v;
            }
            return tailg[k];
        };
        const uint32_t q0 = (uint32_t)(RPD * wave + dq);  // + RPD NWAVE per m
        f32x4 rj = lds_f32x4(xs0 + (uint32_t)((dt * CW + 4 * dh) * 4));
        u32x4 offv = lds_u32x4(P + offs_lane);
        u32x4 hdr = lds_u32x4(P + 4u * G::PL_HDR);
        uint32_t lmw[NMW], fmw[NMW], emw[NMW];
        static_for<NMW>([&](auto k) {
            lmw[k] = lds_u32(P + 4u * (uint32_t)(G::PL_LAST + dt * NMW + k));
            fmw[k] = SAVE ? lds_u32(P + 4u * (uint32_t)(G::PL_FIRST + dt * NMW + k)) : 0u;
            emw[k] = lds_u32(P + 4u * (uint32_t)(G::PL_EXC + dt * NMW + k));
        });
        uint32_t eb = lds_u32(P + 4u * (uint32_t)(G::PL_EXCB + dt));
        f32x2 pf[WB];
        f32x4 m0[WB];
        const uint32_t fina = P + 4u * (uint32_t)(G::PL_FIN + (q0 * CC + dt) * 2);  // + RPD NWAVE rows per m
        const uint32_t own = S + (uint32_t)(((q0 * CC + dt) * CW + 4 * dh) * 4);
        static_for<WB>([&](auto m) {
            pf[m] = lds_f32x2<RPD * NWAVE * m * CC * 8>(fina);
            m0[m] = lds_f32x4<RPD * NWAVE * m * ROWB>(own);
        });
        lds_wait(rj, offv, hdr, eb);
        tie_all(lmw);
        tie_all(fmw);
        tie_all(emw);
        tie_all(pf);
        tie_all(m0);
        mask_t lm = lmw[0], fm = fmw[0], em = emw[0];
        if constexpr (NMW == 2) {
            lm |= (mask_t)lmw[NMW - 1] << 32;
            fm |= (mask_t)fmw[NMW - 1] << 32;
            em |= (mask_t)emw[NMW - 1] << 32;
        }
        // this lane's 16 bytes of the pre-write row of write entry (tok, row)
        auto saved_at = [&](uint32_t tok, uint32_t row) -> f32x4* {
            return reinterpret_cast<f32x4*>(
                a.saved + ((((size_t)b * T + c * CC + tok) * H + h) * G::NW + row) * dv + col0 + 4 * dh);
        };
        const uint32_t extra_base = hdr.x, fwd_base = hdr.y;
        bool any_fwd = false;
        f32x4 keep[WB];
        uint32_t kpk[WB];
#pragma unroll
        for (int m = 0; m < WB; ++m) {
            const uint32_t q = q0 + RPD * NWAVE * m;
            kpk[m] = 0u;
            keep[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!wb_ok) continue;
            f32x4 mv = m0[m];
            if (SAVE && ((fm >> q) & 1u)) *saved_at(dt, q) = mv;
            if (!((lm >> q) & 1u)) continue;
            const float dec = pf[m].x, bw = pf[m].y;  // this visit's decay and beta w
            uint32_t pk = 0u;
            if ((em >> q) & 1u) {
                const uint32_t k = eb + (uint32_t)__builtin_popcountll((uint64_t)(em & (((mask_t)1 << q) - 1u)));
                const uint32_t first = tail(2 * k);
                pk = tail(2 * k + 1);
                if (first != q * CC + dt) {
                    mv = lds_f32x4(S + (first * CW + 4 * dh) * 4);
                    lds_wait(mv);
                }
            }
            // the slot's earlier visits in order: the row before each is the
            // chunk-start row carried through the visits before it
            const uint32_t xst = pk & 511u, xcnt = (pk >> 9) & 31u;
            for (uint32_t x = 0; x < xcnt; ++x) {
                const uint32_t tr = tail(extra_base + 3 * (xst + x));
                const float dx = __uint_as_float(tail(extra_base + 3 * (xst + x) + 1));
                const float bx = __uint_as_float(tail(extra_base + 3 * (xst + x) + 2));
                const uint32_t tau = tr & 255u;
                if (SAVE && x > 0) *saved_at(tau, tr >> 8) = mv;
                f32x4 rt = lds_f32x4(xs0 + (tau * CW + 4 * dh) * 4);
                lds_wait(rt);
                mv.x = fmaf(bx, rt.x, dx * mv.x);
                mv.y = fmaf(bx, rt.y, dx * mv.y);
                mv.z = fmaf(bx, rt.z, dx * mv.z);
                mv.w = fmaf(bx, rt.w, dx * mv.w);
            }
            if (SAVE && xcnt > 0) *saved_at(dt, q) = mv;
            f32x4 val;
            val.x = fmaf(bw, rj.x, dec * mv.x);
            val.y = fmaf(bw, rj.y, dec * mv.y);
            val.z = fmaf(bw, rj.z, dec * mv.z);
            val.w = fmaf(bw, rj.w, dec * mv.w);
            *reinterpret_cast<f32x4*>(tabw + offv[m] + colbyte) = val;
            keep[m] = val;
            kpk[m] = pk;
            any_fwd |= (pk >> 24) != 0u;
        }

        // ---- rows of chunk c+1 (and plan c+2) have landed in every wave: forward
        //      this chunk's final values into the rows of chunk c+1 holding the same slot ----
        wait_vm0();
        block_sync_lds();
        if (__ballot(any_fwd) != 0ull) {
            const uint32_t Sn = stage0 + (uint32_t)((c + 1) % 2) * STAGE_BYTES;
#pragma unroll
            for (int m = 0; m < WB; ++m) {
                const uint32_t fbeg = (kpk[m] >> 14) & 1023u, fcnt = kpk[m] >> 24;
                for (uint32_t x = 0; x < fcnt; ++x) {
                    const uint32_t pos = tail(fwd_base + fbeg + x);
                    lds_write_f32x4(Sn + (pos * CW + 4 * dh) * 4, keep[m]);
                }
            }
        }
        block_sync_lds();
    }
    wait_vm0();
}

}  // namespace

// One workgroup per CU (its LDS footprint), one per column slice: with more
// slices than compute units they run in rounds, which still beats the
// per-token kernel (1.4B-layer shape, B = 5: 12.0 against 22.3 ms; B = 8:
// 18.7 against 26.6 ms).  Sequences shorter than 64 tokens (decode steps,
// short prompts) are left to the per-token kernel.  W = R = 32 runs in chunks
// of 16 tokens, W = R = 64 in chunks of 8.
bool sdm_chunked_supported(int B, int T, int H, int W, int R, int dv, long long N) {
    (void)B;
    (void)H;
    if (!((W == 32 || W == 64) && R == W) || dv % CW != 0) return false;
    if ((unsigned long long)N * (unsigned long long)dv * 4ull >= (1ull << 31)) return false;
    if (N >= (1ll << 31)) return false;
    return T >= 64;
}

size_t sdm_chunk_plan_bytes(int B, int T, int H, int W) {
    const int cc = W == 64 ? GeoW64::CC : GeoW32::CC;
    const long long nch = (T + cc - 1) / cc;
    return (size_t)B * H * nch * PL_WORDS * 4;
}

namespace {
template <class G>
hipError_t launch_plans(const SdmUpdateArgs& a, uint32_t* plan, hipStream_t st) {
    const int nch = (a.T + G::CC - 1) / G::CC;
    PlanArgs pa{a.B, a.T, a.H, a.N, a.dv, nch, a.residual_mode, a.idx_w, a.wt_w, a.idx_r, a.wt_r,
                a.alpha, a.beta, plan, a.err};
    sdm_chunk_plan_kernel<G><<<(unsigned)(a.B * a.H * nch), 256, 0, st>>>(pa);
    return hipGetLastError();
}

template <class G>
hipError_t launch_chunked(const SdmUpdateArgs& a, uint32_t* plan, hipStream_t st) {
    const int nch = (a.T + G::CC - 1) / G::CC;
    hipError_t e = launch_plans<G>(a, plan, st);
    if (e != hipSuccess) return e;
    const int nslice = a.dv / CW;
    const int total = a.B * a.H * nslice;
    const int grid = ((total + 127) / 128) * 128;
    const bool save = a.saved != nullptr;
    if (a.dtype != 0 && save)
        sdm_chunk_apply_kernel<bf16_t, G, true><<<grid, 64 * NWAVE, 0, st>>>(a, plan, nslice, total, nch);
    else if (a.dtype != 0)
        sdm_chunk_apply_kernel<bf16_t, G, false><<<grid, 64 * NWAVE, 0, st>>>(a, plan, nslice, total, nch);
    else if (save)
        sdm_chunk_apply_kernel<float, G, true><<<grid, 64 * NWAVE, 0, st>>>(a, plan, nslice, total, nch);
    else
        sdm_chunk_apply_kernel<float, G, false><<<grid, 64 * NWAVE, 0, st>>>(a, plan, nslice, total, nch);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_sdm_chunk_plans(const SdmUpdateArgs& a, void* planws, hipStream_t st) {
    uint32_t* plan = static_cast<uint32_t*>(planws);
    if (a.W == 64) return launch_plans<GeoW64>(a, plan, st);
    return launch_plans<GeoW32>(a, plan, st);
}

hipError_t launch_sdm_update_chunked(const SdmUpdateArgs& a, void* planws, hipStream_t st) {
    uint32_t* plan = static_cast<uint32_t*>(planws);
    if (a.W == 64) return launch_chunked<GeoW64>(a, plan, st);
    return launch_chunked<GeoW32>(a, plan, st);
}

}  // namespace sslp
