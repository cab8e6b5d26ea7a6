// K5 + K6: Sparse State Expansion forward -- gated top-k routing over N state
// partitions, per-chunk bucketing of the routed tokens, and the GLA recurrence
// of every visited partition with decay advancing only on visits, plus the
// always-active shared partition.
//
// Slides "Scaling Linear Attention with Sparse State Expansion": "One gate
// controls both writes and reads" (Eqs. (9)-(14)): e_t = softmax(logits),
// T_t = top-k, S^i_t = Lambda_t S^i_{t-1} + e^i_t k_t^T v_t for i in T_t (else
// unchanged), o_t = sum_{i in T_t} e^i_t q_t S^i_t; "A memory decays only when
// its partition is visited"; "Varlen groups tokens while preserving causal
// order" (group by partition, keep time order, one batched pass, then sum);
// backup "Selected gate mass is usually below one" (no renormalisation).
// The shared partition (index N) is visited by every token with weight 1 and
// its own key/query (the slides leave its formula out; reading stated in the
// header).
//
// Execution.  sse_route_kernel first routes every token on its own thread
// (fp32 softmax and top-k, ties to the lowest index) into the sel / e_sel
// arrays.  Then one workgroup per (batch, head, 32-column block of d) walks the
// sequence in chunks of 64 tokens.  Per chunk, wave 0 reads the routing and
// builds, for every routed partition, the time-ordered list of its visits
// inside the chunk (ballot + popcount counting sort).  Then every partition is advanced independently by
// its own wavefront: routed partition i by wave 2+i (32 columns), the shared
// partition by waves 0 and 1 (16 columns each).  A wave processes its visits
// in blocks of up to 16 as one GLA step in chunked form:
//     o_p   = e_p [ (q_p * AF E+_p) S + sum_{p'<=p} e_p' (q_p * E+_p).(k_p' * E-_p') v_p' ]
//     S_new = (AF PX) S + sum_p' (k_p' * PX E-_p')^T e_p' v_p'
// with AF the first visit's decay, E+_p the product of decays after it
// (E-_p = 1/E+_p, PX = E+ of the last visit).  A block ends early before the
// visit that would take E+ below 2^-60 in any state row, so E- stays below
// 2^60 whatever the decays in (0, 1] (a one-visit block takes no inverse).  The state stays in MFMA accumulator registers; the three
// products run on 16x16x32 / 16x16x16 bf16 MFMA with fp32 accumulation.  The
// k+1 contributions of a token are summed in a fixed order (routed in rank
// order, then shared) once all partitions are done with the chunk.  The
// column blocks of a (batch, head) are placed on one XCD, whose L2 then serves
// their common q, k and Lambda reads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = 64;     // chunk length (tokens)
constexpr int CR = 128;   // partition rows (key width c)
constexpr int DB = 32;    // columns of d per workgroup
constexpr int MAXN = 8;   // routed partitions supported
constexpr int LDQ = CR + 8;
constexpr int LDV = 20;
constexpr float kMinBlockDecay = 0x1p-60f;  // smallest product of decays inside a block

struct __align__(16) WaveScratch {
    uint16_t qs[16][LDQ];  // q * E+ (bf16)
    uint16_t ks[16][LDQ];  // k * E- (bf16)
    uint16_t vt[32][LDV];  // gated values, transposed: vt[n][p] = e_p v_p[n]
    float af[CR];          // decay of the block's first visit
    float px[CR];          // product of the decays after the first visit
};

template <int TOPK>
struct __align__(16) Smem {
    WaveScratch ws[MAXN + 2];
    float contrib[C][TOPK][DB];  // routed contributions by rank
    float osh[C][DB];            // shared-partition contribution
    int16_t vis[MAXN][C];        // visits of each routed partition (local token ids)
    int8_t vrank[MAXN][C];       // rank of the partition in the visiting token's top-k
    float vgate[MAXN][C];        // its gate value
    int cnt[MAXN];
};

SSLP_DEVICE __bf16 bfv(float f) { return __builtin_bit_cast(__bf16, f32_to_bf16(f).bits); }
SSLP_DEVICE short bfs(float f) { return (short)f32_to_bf16(f).bits; }
SSLP_DEVICE float bf2f(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

template <typename io_t>
SSLP_DEVICE float ld(const io_t* p) {
    return to_f32(*p);
}

struct SseArgs {
    int B, T, H, N, topk, dv;
    const float* logits;
    const void* q;
    const void* k;
    const void* v;
    const float* lam;
    const void* q_sh;
    const void* k_sh;
    float* S;
    void* o;
    int32_t* sel;
    float* e_sel;
    int masking;  // 1: every routed partition runs over every token (masked execution)
};

// One block of up to L <= 16 visits of one partition on one wave; returns the
// number of visits taken.  The block ends early before a visit that would take
// the product of decays after its first visit below kMinBlockDecay in any state
// row, so that the inverse products stay below 2^60 whatever the decays in
// (0, 1] (a block of one visit takes no inverse at all).
//   NY      number of 16-column tiles this wave owns (2 routed, 1 shared)
//   St      the partition state slice, accumulator layout: tile (m, y) holds
//           rows 16m + 4(lane/16) + j, column 16y + lane%16
//   visits  local token ids and gate weights of the visits (p < L)
template <typename io_t, int NY>
SSLP_DEVICE int gla_block(f32x4_t (&St)[8][NY], WaveScratch& ws, const SseArgs& a,
                           const io_t* qg, const io_t* kg, const io_t* vg, int b, int h, int t0,
                           int col0, const int16_t* vtok, const float* vgate, int tbase, int L,
                           int lane, f32x4_t (&ot)[NY], const int8_t* vmask = nullptr) {
    // visit p: token tok(p) of the chunk with gate gate(p) (LDS lists, or
    // consecutive tokens from tbase with gate 1)
    auto tok = [&](int p) { return vtok ? (int)vtok[p] : tbase + p; };
    auto gate = [&](int p) { return vgate ? vgate[p] : 1.f; };
    const int T = a.T, H = a.H;
    const int g4 = lane >> 4, l16 = lane & 15;
    int Le = L;
    bool alive = true;     // wave-uniform: the block still takes visits
    bool careful = false;  // wave-uniform: visits are tested for the block end
    // ---- a. decay-scaled operands (lane owns rows 2 lane, 2 lane + 1); the
    //      loads of 8 visits are issued before any of them is used ----
    {
        constexpr int NV = NY * 16 * 16 / 64;
        float vv[NV];
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            const int idx = lane + 64 * e;
            const int p = idx >> (NY == 2 ? 5 : 4), n = idx & (NY * 16 - 1);
            const int tp = p < L ? tok(p) : tok(0);
            const size_t bth = ((size_t)b * T + t0 + tp) * H + h;
            vv[e] = ld(vg + bth * a.dv + col0 + n);
        }
        float ep0 = 1.f, ep1 = 1.f, em0 = 1.f, em1 = 1.f, af0 = 1.f, af1 = 1.f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float2 lam[8];
            uint32_t qw[8], kw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int p = 8 * half + u;
                const int tp = p < L ? tok(p) : tok(0);
                const size_t bth = ((size_t)b * T + t0 + tp) * H + h;
                lam[u] = *reinterpret_cast<const float2*>(a.lam + bth * CR + 2 * lane);
                qw[u] = *reinterpret_cast<const uint32_t*>(qg + bth * CR + 2 * lane);
                kw[u] = *reinterpret_cast<const uint32_t*>(kg + bth * CR + 2 * lane);
            }
            // the block-end test is needed only from the first half holding a decay
            // below 2^-4 on (fifteen decays of at least 2^-4 keep the product >= 2^-60)
            bool small = false;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                small |= 8 * half + u < L && (lam[u].x < 0x1p-4f || lam[u].y < 0x1p-4f);
            careful = careful || __ballot(small) != 0ull;
            // one of two copies of the half, chosen once: without and with the test
            auto stage_half = [&](auto test) __attribute__((always_inline)) {
                constexpr bool TEST = decltype(test)::value;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int p = 8 * half + u;
                    float q0 = 0.f, q1 = 0.f, k0 = 0.f, k1 = 0.f;
                    if (p < L) {
                        // masked execution: a token that does not select the partition leaves
                        // its state undecayed (and writes nothing: its gate is 0)
                        const bool frozen = vmask != nullptr && vmask[p] < 0;
                        const float l0 = frozen ? 1.f : lam[u].x, l1 = frozen ? 1.f : lam[u].y;
                        if (p == 0) {
                            af0 = l0;
                            af1 = l1;
                        } else if (!TEST) {
                            ep0 *= l0;
                            ep1 *= l1;
                            // hardware reciprocal (within 1 ulp, not an IEEE division):
                            // the factor only scales a key that is rounded to bf16
                            em0 *= __builtin_amdgcn_rcpf(l0);
                            em1 *= __builtin_amdgcn_rcpf(l1);
                        } else if (alive) {
                            const float n0 = ep0 * l0, n1 = ep1 * l1;
                            if (__ballot(n0 < kMinBlockDecay || n1 < kMinBlockDecay) != 0ull) {
                                alive = false;  // this visit starts the next block
                                Le = p;
                            } else {
                                ep0 = n0;
                                ep1 = n1;
                                em0 *= __builtin_amdgcn_rcpf(l0);
                                em1 *= __builtin_amdgcn_rcpf(l1);
                            }
                        }
                        if (!TEST || alive) {
                            q0 = __uint_as_float(qw[u] << 16);
                            q1 = __uint_as_float(qw[u] & 0xFFFF0000u);
                            k0 = __uint_as_float(kw[u] << 16);
                            k1 = __uint_as_float(kw[u] & 0xFFFF0000u);
                        }
                    }
                    *reinterpret_cast<uint32_t*>(&ws.qs[p][2 * lane]) =
                        (uint32_t)f32_to_bf16(q0 * ep0).bits | ((uint32_t)f32_to_bf16(q1 * ep1).bits << 16);
                    *reinterpret_cast<uint32_t*>(&ws.ks[p][2 * lane]) =
                        (uint32_t)f32_to_bf16(k0 * em0).bits | ((uint32_t)f32_to_bf16(k1 * em1).bits << 16);
                }
            };
            if (careful) stage_half(std::true_type{});
            else stage_half(std::false_type{});
        }
        *reinterpret_cast<float2*>(&ws.af[2 * lane]) = make_float2(af0, af1);
        *reinterpret_cast<float2*>(&ws.px[2 * lane]) = make_float2(ep0, ep1);
        // gated values, transposed
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            const int idx = lane + 64 * e;
            const int p = idx >> (NY == 2 ? 5 : 4), n = idx & (NY * 16 - 1);
            ws.vt[n][p] = f32_to_bf16(p < Le ? gate(p) * vv[e] : 0.f).bits;
        }
    }
    wave_sync();
    // ---- b. state decayed by the first visit (per row) ----
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 f = *reinterpret_cast<const float4*>(&ws.af[16 * m + 4 * g4]);
#pragma unroll
        for (int y = 0; y < NY; ++y) {
            St[m][y][0] *= f.x;
            St[m][y][1] *= f.y;
            St[m][y][2] *= f.z;
            St[m][y][3] *= f.w;
        }
    }
    // ---- c. O^T = S^T (Qs)^T, k-slots of group g4 = rows {32s+4g4+j, 32s+16+4g4+j} ----
#pragma unroll
    for (int y = 0; y < NY; ++y) ot[y] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8_t bq;
        {
            const uint16_t* r0 = &ws.qs[l16][32 * s + 4 * g4];
            const uint16_t* r1 = &ws.qs[l16][32 * s + 16 + 4 * g4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bq[j] = __builtin_bit_cast(__bf16, r0[j]);
                bq[4 + j] = __builtin_bit_cast(__bf16, r1[j]);
            }
        }
#pragma unroll
        for (int y = 0; y < NY; ++y) {
            bf16x8_t as;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                as[j] = bfv(St[2 * s][y][j]);
                as[4 + j] = bfv(St[2 * s + 1][y][j]);
            }
            ot[y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as, bq, ot[y], 0, 0, 0);
        }
    }
    // ---- d. Pm^T[p'][p] = Ks Qs^T, causal within the block ----
    f32x4_t pm = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(&ws.ks[l16][32 * s + 8 * g4]);
        const bf16x8_t bq = *reinterpret_cast<const bf16x8_t*>(&ws.qs[l16][32 * s + 8 * g4]);
        pm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bq, pm, 0, 0, 0);
    }
    s16x4_t bp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int pp = 4 * g4 + j;  // p' (row), column p = l16
        bp[j] = bfs((pp <= l16 && l16 < Le) ? pm[j] : 0.f);
    }
    // ---- e. O^T += Ve^T Pm^T ----
    // (own accumulator, added with VALU: a 16x16x16 MFMA must not take the
    // accumulator of a 16x16x32 MFMA as its C operand -- the compiler's
    // hazard handling left that chain unpadded and the C input was stale)
#pragma unroll
    for (int y = 0; y < NY; ++y) {
        s16x4_t av;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = (short)ws.vt[16 * y + l16][4 * g4 + i];
        const f32x4_t oe = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            av, bp, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) ot[y][j] += oe[j];
    }
    // ---- g. S = PX * S + (Ks * PX)^T Ve ----
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 f = *reinterpret_cast<const float4*>(&ws.px[16 * m + 4 * g4]);
        const float pxr = ws.px[16 * m + l16];
        s16x4_t ak;
#pragma unroll
        for (int i = 0; i < 4; ++i) ak[i] = bfs(bf2f(ws.ks[4 * g4 + i][16 * m + l16]) * pxr);
#pragma unroll
        for (int y = 0; y < NY; ++y) {
            St[m][y][0] *= f.x;
            St[m][y][1] *= f.y;
            St[m][y][2] *= f.z;
            St[m][y][3] *= f.w;
            s16x4_t bv;
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = (short)ws.vt[16 * y + l16][4 * g4 + i];
            St[m][y] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ak, bv, St[m][y], 0, 0, 0);
        }
    }
    wave_sync();
    return Le;
}

// Routing of every token (one thread per (b, t, h)): e = softmax(logits) over
// the N partitions in fp32, top-k by logit with ties to the lowest index
// (the selected gate values are not renormalised).
__global__ __launch_bounds__(256) void sse_route_kernel(const float* __restrict__ logits, int P,
                                                        int N, int topk, int32_t* __restrict__ sel,
                                                        float* __restrict__ esel) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const float* lg = logits + (size_t)p * N;
    float lv[MAXN];
    float mx = lg[0];
#pragma unroll
    for (int i = 0; i < MAXN; ++i) {
        lv[i] = i < N ? lg[i] : 0.f;
        if (i < N && lv[i] > mx) mx = lv[i];
    }
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < MAXN; ++i)
        if (i < N) z += __expf(lv[i] - mx);
    unsigned taken = 0;
    for (int r = 0; r < topk; ++r) {
        int best = -1;
#pragma unroll
        for (int i = 0; i < MAXN; ++i)
            if (i < N && !((taken >> i) & 1u) && (best < 0 || lv[i] > lv[best])) best = i;
        taken |= 1u << best;
        sel[(size_t)p * topk + r] = best;
        esel[(size_t)p * topk + r] = __expf(lv[best] - mx) / z;
    }
}

template <typename io_t, int TOPK>
__global__ __launch_bounds__(64 * (MAXN + 2)) void sse_chunk_kernel(SseArgs a) {
    __shared__ Smem<TOPK> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nblk = a.dv / DB;
    // XCD-aware placement: workgroups x and x + 8 share an XCD; the nblk column
    // blocks of a (batch, head) take consecutive multiples of 8 on one XCD, so
    // that its L2 serves their common q, k and Lambda reads
    const int x = blockIdx.x, xcd = x & 7, kq = x >> 3;
    const int bh = (kq / nblk) * 8 + xcd, cb = kq % nblk;
    if (bh >= a.B * a.H) return;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int n0 = cb * DB;
    const int T = a.T, H = a.H, N = a.N, topk = a.topk, dv = a.dv;
    const int g4 = lane >> 4, l16 = lane & 15;
    const io_t* qg = static_cast<const io_t*>(a.q);
    const io_t* kg = static_cast<const io_t*>(a.k);
    const io_t* vg = static_cast<const io_t*>(a.v);
    const io_t* qsh = a.q_sh ? static_cast<const io_t*>(a.q_sh) : qg;
    const io_t* ksh = a.k_sh ? static_cast<const io_t*>(a.k_sh) : kg;
    io_t* og = static_cast<io_t*>(a.o);

    // role of this wave: 0,1 shared partition (16 columns each); 2+i routed partition i
    const bool shared = w < 2;
    const int part = shared ? N : w - 2;
    const bool active = shared || part < N;
    const int colw = shared ? 16 * w : 0;  // column offset inside the block
    float* Sg = a.S + (((size_t)b * H + h) * (N + 1) + part) * CR * dv;
    const int nchunks = (T + C - 1) / C;

    // The chunk loop, instantiated per role so that a wave keeps only its own
    // state slice (accumulator layout) live: NY = 1 (shared, 16 columns) or
    // NY = 2 (routed, 32 columns).  Both instantiations pass the same barriers.
    auto run = [&](auto& St, auto nyc) {
        constexpr int NY = decltype(nyc)::value;
        if (active) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int y = 0; y < NY; ++y)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        St[m][y][j] = Sg[(size_t)(16 * m + 4 * g4 + j) * dv + n0 + colw + 16 * y + l16];
        }
        for (int c = 0; c < nchunks; ++c) {
            const int t0 = c * C;
            const int Tc = (T - t0) < C ? (T - t0) : C;
            // ---------------- routing and bucketing (wave 0) ----------------
            if (w == 0) {
                const int t = lane;
                int sel[TOPK];
                float gsel[TOPK];
#pragma unroll
                for (int r = 0; r < TOPK; ++r) {
                    sel[r] = -1;
                    gsel[r] = 0.f;
                }
                if (t < Tc) {
                    const size_t bth = ((size_t)b * T + t0 + t) * H + h;
#pragma unroll
                    for (int r = 0; r < TOPK; ++r)
                        if (r < topk) {
                            sel[r] = a.sel[bth * topk + r];
                            gsel[r] = a.e_sel[bth * topk + r];
                        }
                }
                for (int i = 0; i < N; ++i) {
                    bool hit = false;
                    int rk = 0;
                    float gv = 0.f;
#pragma unroll
                    for (int r = 0; r < TOPK; ++r)
                        if (sel[r] == i) {
                            hit = true;
                            rk = r;
                            gv = gsel[r];
                        }
                    if (a.masking) {
                        // every token, in order; rank -1 marks the ones that do not select i
                        if (t < Tc) {
                            sm.vis[i][t] = (int16_t)t;
                            sm.vrank[i][t] = (int8_t)(hit ? rk : -1);
                            sm.vgate[i][t] = hit ? gv : 0.f;
                        }
                        if (lane == 0) sm.cnt[i] = Tc;
                        continue;
                    }
                    const unsigned long long m = __ballot(hit);
                    if (hit) {
                        const int pos = __popcll(m & ((1ull << lane) - 1ull));
                        sm.vis[i][pos] = (int16_t)t;
                        sm.vrank[i][pos] = (int8_t)rk;
                        sm.vgate[i][pos] = gv;
                    }
                    if (lane == 0) sm.cnt[i] = __popcll(m);
                }
            }
            block_sync_lds();
            // ---------------- every partition advances over its visits ----------------
            if (active) {
                WaveScratch& ws = sm.ws[w];
                if constexpr (NY == 1) {
                    for (int p0 = 0; p0 < Tc;) {
                        const int L = (Tc - p0) < 16 ? (Tc - p0) : 16;
                        f32x4_t ot[1];
                        const int Le = gla_block<io_t, 1>(St, ws, a, qsh, ksh, vg, b, h, t0, n0 + colw,
                                                          nullptr, nullptr, p0, L, lane, ot);
                        // O^T tile: column p = l16, rows n = 4 g4 + j
                        if (l16 < Le) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) sm.osh[p0 + l16][colw + 4 * g4 + j] = ot[0][j];
                        }
                        p0 += Le;
                    }
                } else {
                    const int cnt = sm.cnt[part];
                    for (int p0 = 0; p0 < cnt;) {
                        const int L = (cnt - p0) < 16 ? (cnt - p0) : 16;
                        f32x4_t ot[NY];
                        const int Le = gla_block<io_t, NY>(St, ws, a, qg, kg, vg, b, h, t0, n0,
                                                           &sm.vis[part][p0], &sm.vgate[part][p0], 0,
                                                           L, lane, ot,
                                                           a.masking ? &sm.vrank[part][p0] : nullptr);
                        const int rk = l16 < Le ? sm.vrank[part][p0 + l16] : -1;
                        if (rk >= 0) {
                            const int tp = sm.vis[part][p0 + l16];
                            const float e = sm.vgate[part][p0 + l16];
#pragma unroll
                            for (int y = 0; y < NY; ++y)
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    sm.contrib[tp][rk][16 * y + 4 * g4 + j] = e * ot[y][j];
                        }
                        p0 += Le;
                    }
                }
            }
            block_sync_lds();
            // ---------------- fixed-order combine: routed by rank, then shared ----------------
            for (int idx = tid; idx < C * DB; idx += blockDim.x) {
                const int t = idx / DB, n = idx - (idx / DB) * DB;
                if (t < Tc) {
                    float acc = 0.f;
#pragma unroll
                    for (int r = 0; r < TOPK; ++r)
                        if (r < topk) acc += sm.contrib[t][r][n];
                    acc += sm.osh[t][n];
                    og[(((size_t)b * T + t0 + t) * H + h) * dv + n0 + n] = from_f32<io_t>(acc);
                }
            }
            block_sync_lds();
        }
        if (active) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int y = 0; y < NY; ++y)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        Sg[(size_t)(16 * m + 4 * g4 + j) * dv + n0 + colw + 16 * y + l16] = St[m][y][j];
        }
    };
    if (shared) {
        f32x4_t St[8][1];
        run(St, std::integral_constant<int, 1>{});
    } else {
        f32x4_t St[8][2];
        run(St, std::integral_constant<int, 2>{});
    }
}

}  // namespace

hipError_t launch_sse(int B, int T, int H, int N, int topk, int dv, int dtype,
                      const float* logits, const void* q, const void* k, const void* v,
                      const float* lam, const void* q_sh, const void* k_sh, float* S, void* o,
                      int32_t* sel, float* e_sel, hipStream_t st, int masking) {
    if (dtype != 1 || N > MAXN || topk > 4 || dv % DB != 0) return hipErrorInvalidValue;
    SseArgs a{B, T, H, N, topk, dv, logits, q, k, v, lam, q_sh, k_sh, S, o, sel, e_sel, masking};
    const int P = B * T * H;
    sse_route_kernel<<<(unsigned)((P + 255) / 256), 256, 0, st>>>(logits, P, N, topk, sel, e_sel);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 8 * nblk consecutive workgroups hold 8 (batch, head) groups, one per XCD
    dim3 grid((unsigned)(((B * H + 7) / 8) * 8 * (dv / DB)));
    dim3 block(64 * (N + 2));
    if (topk <= 2) sse_chunk_kernel<bf16_t, 2><<<grid, block, 0, st>>>(a);
    else sse_chunk_kernel<bf16_t, 4><<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace sslp
