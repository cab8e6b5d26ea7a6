// K5 + K6: Sparse State Expansion forward -- gated top-k routing over N state
// partitions, grouping of every partition's visits in time order, and the GLA
// recurrence of every visited partition with decay advancing only on visits,
// plus the always-active shared partition.
//
// Slides "Scaling Linear Attention with Sparse State Expansion": "One gate
// controls both writes and reads" (Eqs. (9)-(14)): e_t = softmax(logits),
// T_t = top-k, S^i_t = Lambda_t S^i_{t-1} + e^i_t k_t^T v_t for i in T_t (else
// unchanged), o_t = sum_{i in T_t} e^i_t q_t S^i_t; "A memory decays only when
// its partition is visited"; "Varlen groups tokens while preserving causal
// order" (group by sample and partition, new sequence offsets, one batched
// chunked pass, then scatter and sum); backup "Selected gate mass is usually
// below one" (no renormalisation).  The shared partition (index N) is visited
// by every token with weight 1 and its own key/query (the slides leave its
// formula out; reading stated in the header).
//
// Four launches:
//  * sse_route_kernel: every token on its own thread (fp32 softmax and top-k,
//    ties to the lowest index) into sel / e_sel, and a (batch, head)-major
//    copy (ranks packed in 4 bits each, gates) for the bucket kernel.
//  * sse_bucket_kernel: one workgroup per (batch, head) lists every routed
//    partition's visits in time order (token << 3 | rank), with its count --
//    the grouped sequences of the varlen layout.  The masking execution lists
//    every token for every partition, rank 7 marking the ones that do not
//    select it.
//  * sse_gla_kernel: one workgroup of four wavefronts per (partition
//    sequence, 64 columns of d); the shared partitions' workgroups come first
//    (their sequences are the longest).  The workgroup walks its sequence in
//    chunks of 64 visits.  Per chunk each wavefront stages one 16-visit
//    sub-block -- the decay-scaled query and key tiles shared by all columns
//    -- and the gated values of its own 16 columns; then every wavefront
//    advances its 16-column slice of the state (MFMA accumulator registers)
//    over the four sub-blocks in order:
//        S   <- AF * S                               (first visit's decay)
//        o_p  = (q_p * E+_p) S + sum_{p'<=p} (q_p * E+_p).(k_p' * E-_p') e_p' v_p'
//        S   <- PX * (S + sum_p' (k_p' * E-_p')^T e_p' v_p')
//    (E+_p the product of the decays after the first visit, E- its inverse,
//    PX = E+ of the last visit), and writes e_p o_p into the token's slot of
//    a contribution buffer (its rank; the shared partition's slot is topk).
//    A sub-block holding a decay below 2^-4 could take an inverse product past
//    2^60; such a chunk is redone instead as blocks of up to 16 visits that
//    end before the product of decays falls below 2^-60, each wavefront
//    staging its own blocks (exact for any decay in (0, 1]).
//  * sse_combine_kernel: o_t = the token's slots summed in a fixed order
//    (routed by rank, then shared), rounded once to the output type.
// The column blocks of a partition sequence run on one XCD, whose L2 then
// serves their common q, k and Lambda rows.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int CR = 128;   // partition rows (key width c)
constexpr int DB = 64;    // columns of d per workgroup
constexpr int NWV = 4;    // wavefronts per workgroup, 16 columns each
constexpr int CH = 64;    // visits per chunk: four sub-blocks of 16
constexpr int MAXN = 8;   // routed partitions supported
constexpr int MAXK = 4;   // top-k supported
constexpr int LDQ = CR + 8;  // bf16 row stride of [visit][row] tiles
constexpr int LDT = 24;      // bf16 row stride of the [row][visit] key tile
constexpr int LDV = CH + 8;  // bf16 row stride of the [column][visit] value tile
constexpr uint32_t kNoRank = 7;  // rank field of a masked visit (the token does not select the partition)
constexpr float kMinBlockDecay = 0x1p-60f;  // smallest product of decays inside a block
constexpr float kSmallDecay = 0x1p-4f;      // 15 decays at least this keep the product >= 2^-60

// the decay-scaled operands of one sub-block of up to 16 visits
struct __align__(16) SubBlock {
    uint16_t qs[16][LDQ];  // q * E+ [visit][row]
    uint16_t ks[16][LDQ];  // k * E- [visit][row]
    uint16_t kt[CR][LDT];  // k * E- [row][visit]
    float af[CR];          // decay of the first visit
    float px[CR];          // product of the decays after the first visit
};

struct __align__(16) GlaSmem {
    SubBlock sb[NWV];             // sub-block r staged by wavefront r (slow path: private)
    uint16_t vt[NWV][16][LDV];    // per wavefront: gated values of its 16 columns [column][visit]
    int vtok[2][CH];              // token of each visit of the chunk (two chunks in flight)
    float vgate[2][CH];           // its gate (1 for the shared partition, 0 when masked)
    int vslot[2][CH];             // its contribution slot, -1 for a masked visit
    int small[NWV];
};

// the visits of one chunk (one of the two buffers)
struct Meta {
    const int* tok;
    const float* gate;
    const int* slot;
};
static_assert(sizeof(GlaSmem) <= 80 * 1024, "two workgroups per compute unit");

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

SSLP_DEVICE short bfs(float f) { return (short)f32_to_bf16(f).bits; }
// two fp32 values rounded to bf16 in one instruction: lo in bits 0-15
SSLP_DEVICE uint32_t pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
SSLP_DEVICE __bf16 bfv(float f) { return __builtin_bit_cast(__bf16, f32_to_bf16(f).bits); }

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
    int masking;      // 1: every routed partition runs over every token (masked execution)
    uint32_t* vis;    // [B*H][N][T] visits, token << 3 | rank
    float* vgl;       // [B*H][N][T] their gates (0 for a masked visit)
    uint32_t* rsel;   // [B*H][T] the routing, (b, h)-major: 4 bits per rank
    float4* rgate;    // [B*H][T] the selected gates by rank
    int* cnt;         // [B*H][N] visits per routed partition
    bf16_t* opart;    // [B*T*H][topk + 1][dv] contributions by slot
};

// Routing of every token (one thread per (b, t, h)): e = softmax(logits) over
// the N partitions in fp32, top-k by logit with ties to the lowest index
// (the selected gate values are not renormalised).
// Besides sel / e_sel ([B,T,H,k]) it writes a (b, h)-major copy for the
// bucket kernel, whose reads of a head's tokens are then contiguous.
__global__ __launch_bounds__(256) void sse_route_kernel(const float* __restrict__ logits, int P,
                                                        int N, int topk, int32_t* __restrict__ sel,
                                                        float* __restrict__ esel, int T, int H,
                                                        uint32_t* __restrict__ rsel,
                                                        float4* __restrict__ rgate) {
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
    uint32_t packed = 0;
    float g4[MAXK] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < MAXK; ++r) {
        if (r >= topk) break;
        int best = -1;
#pragma unroll
        for (int i = 0; i < MAXN; ++i)
            if (i < N && !((taken >> i) & 1u) && (best < 0 || lv[i] > lv[best])) best = i;
        taken |= 1u << best;
        const float g = __expf(lv[best] - mx) / z;
        sel[(size_t)p * topk + r] = best;
        esel[(size_t)p * topk + r] = g;
        packed |= (uint32_t)best << (4 * r);
        g4[r] = g;
    }
    const int h = p % H, t = (p / H) % T, b = p / (H * T);
    const size_t q = ((size_t)b * H + h) * T + t;
    rsel[q] = packed;
    rgate[q] = make_float4(g4[0], g4[1], g4[2], g4[3]);
}

// Visit lists of every routed partition of one (batch, head), in time order.
// Wave w (of 16) takes a sixteenth of the sequence, loads its routing at once,
// and scans it twice: first counting each partition's visits (ballot +
// popcount), then, from the counts of the waves before it, placing them.
constexpr int BKW = 16;  // wavefronts of the bucket kernel
constexpr int BKI = 4;   // 64-token steps a wavefront holds at once

__global__ __launch_bounds__(64 * BKW) void sse_bucket_kernel(SseArgs a) {
    __shared__ int s_cnt[BKW][MAXN];
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int T = a.T, N = a.N, topk = a.topk;
    uint32_t* vis = a.vis + (size_t)bh * N * T;
    float* vgl = a.vgl + (size_t)bh * N * T;
    if (a.masking) {
        for (int t = threadIdx.x; t < T; t += 64 * BKW) {
            const uint32_t pk = a.rsel[(size_t)bh * T + t];
            const float4 g4 = a.rgate[(size_t)bh * T + t];
            int sl[MAXK];
            const float ge[MAXK] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int r = 0; r < MAXK; ++r) sl[r] = r < topk ? (int)((pk >> (4 * r)) & 15u) : -1;
            for (int i = 0; i < N; ++i) {
                uint32_t rk = kNoRank;
                float g = 0.f;
#pragma unroll
                for (int r = 0; r < MAXK; ++r)
                    if (sl[r] == i) {
                        rk = (uint32_t)r;
                        g = ge[r];
                    }
                vis[(size_t)i * T + t] = ((uint32_t)t << 3) | rk;
                vgl[(size_t)i * T + t] = g;
            }
        }
        if (threadIdx.x < N) a.cnt[bh * N + threadIdx.x] = T;
        return;
    }
    const int per = ((T + 64 * BKW - 1) / (64 * BKW)) * 64;  // tokens per wave, a multiple of 64
    const int t_beg = min(w * per, T), t_end = min(t_beg + per, T);
    const unsigned long long below = (1ull << lane) - 1ull;
    int pos[MAXN];
    for (int pass = 0; pass < 2; ++pass) {
        int mine = 0;  // pass 0, lane i < N: visits of partition i in this wave's range
        for (int t0 = t_beg; t0 < t_end; t0 += 64 * BKI) {
            // the routing of BKI steps of 64 tokens, loaded before any is used
            int sl[BKI][MAXK];
#pragma unroll
            for (int s = 0; s < BKI; ++s) {
                const int t = t0 + 64 * s + lane;
                const uint32_t pk = a.rsel[(size_t)bh * T + (t < t_end ? t : 0)];
#pragma unroll
                for (int r = 0; r < MAXK; ++r) sl[s][r] = r < topk ? (int)((pk >> (4 * r)) & 15u) : -1;
            }
            float ge[BKI][MAXK];  // the gates, needed by the placing pass only
            if (pass == 1) {
#pragma unroll
                for (int s = 0; s < BKI; ++s) {
                    const int t = t0 + 64 * s + lane;
                    const float4 g4 = a.rgate[(size_t)bh * T + (t < t_end ? t : 0)];
                    ge[s][0] = g4.x;
                    ge[s][1] = g4.y;
                    ge[s][2] = g4.z;
                    ge[s][3] = g4.w;
                }
            }
#pragma unroll
            for (int s = 0; s < BKI; ++s) {
                const int t = t0 + 64 * s + lane;
                const bool ok = t < t_end;
#pragma unroll
                for (int i = 0; i < MAXN; ++i) {
                    if (i >= N) break;
                    int rk = -1;
#pragma unroll
                    for (int r = 0; r < MAXK; ++r)
                        if (ok && sl[s][r] == i) rk = r;
                    const unsigned long long m = __ballot(rk >= 0);
                    if (pass == 0) {
                        if (lane == i) mine += __popcll(m);
                    } else {
                        if (rk >= 0) {
                            const size_t at = (size_t)i * T + pos[i] + __popcll(m & below);
                            vis[at] = ((uint32_t)t << 3) | (uint32_t)rk;
                            float g = 0.f;
#pragma unroll
                            for (int r = 0; r < MAXK; ++r)
                                if (r == rk) g = ge[s][r];
                            vgl[at] = g;
                        }
                        pos[i] += __popcll(m);
                    }
                }
            }
        }
        if (pass == 0) {
            if (lane < N) s_cnt[w][lane] = mine;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < MAXN; ++i) {
                pos[i] = 0;
                for (int u = 0; u < w; ++u) pos[i] += i < N ? s_cnt[u][i] : 0;
            }
        }
    }
    if (w == 0 && lane < N) {
        int c = 0;
        for (int u = 0; u < BKW; ++u) c += s_cnt[u][lane];
        a.cnt[bh * N + lane] = c;
    }
}

// The raw inputs of one sub-block (lane l: state rows 2l, 2l+1) and of the
// gated values (lane: 4 columns of 4 visits), loaded together before any of
// them is used so that the chunk's staging waits for one memory round trip.
struct SubIn {
    float2 lam[16];
    uint32_t qw[16], kw[16];
};
struct ValIn {
    uint2 raw[4];
};

// Row addresses as a batch base (uniform) plus a 32-bit byte offset, so that
// each load needs one address register (the launcher keeps T*H*c*4 < 2^31).
struct RowBases {
    const char* q;    // q (or q_sh) rows of batch b
    const char* k;    // k (or k_sh) rows
    const char* lam;  // Lambda rows (fp32)
    const char* v;    // v rows
};

SSLP_DEVICE void load_sub(SubIn& in, const SseArgs& a, const RowBases& rb, int h, const Meta& mt,
                          int p0, int L, int lane) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int tp = mt.tok[p0 + (p < L ? p : L - 1)];
        const uint32_t off = ((uint32_t)tp * (uint32_t)a.H + (uint32_t)h) * (CR * 2) + 4u * lane;
        in.lam[p] = *reinterpret_cast<const float2*>(rb.lam + 2u * off);
        in.qw[p] = *reinterpret_cast<const uint32_t*>(rb.q + off);
        in.kw[p] = *reinterpret_cast<const uint32_t*>(rb.k + off);
    }
}

SSLP_DEVICE void load_values(ValIn& in, const SseArgs& a, const RowBases& rb, int h, const Meta& mt,
                             int L, int col0, int lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = lane + 64 * e;  // visit idx >> 2, columns 4 (idx & 3) ..
        const int p = idx >> 2;
        const int tp = mt.tok[p < L ? p : L - 1];
        const uint32_t off = (((uint32_t)tp * (uint32_t)a.H + (uint32_t)h) * (uint32_t)a.dv +
                              (uint32_t)(col0 + 4 * (idx & 3))) * 2u;
        in.raw[e] = *reinterpret_cast<const uint2*>(rb.v + off);
    }
}

// The chunk-start form of load_sub and stage_sub<false> (p0 a multiple of
// 16): the visit list is read with vector reads, row offsets are one 24-bit
// multiply, and every per-visit decision is a select (visits past L load the
// first visit's rows and stage zeros; a masked visit decays by 1).  Frozen
// visits exist only in the masking execution (may_freeze).
SSLP_DEVICE void load_sub16(SubIn& in, const SseArgs& a, const RowBases& rb, int h, const Meta& mt,
                            int p0, int L, int lane) {
    int tk[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int4 t4 = *reinterpret_cast<const int4*>(&mt.tok[p0 + 4 * q]);
        tk[4 * q] = t4.x;
        tk[4 * q + 1] = t4.y;
        tk[4 * q + 2] = t4.z;
        tk[4 * q + 3] = t4.w;
    }
    const uint32_t stride = (uint32_t)a.H * (CR * 2);  // bytes between tokens of a bf16 row array
    const uint32_t base = (uint32_t)h * (CR * 2) + 4u * lane;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int tp = p < L ? tk[p] : tk[0];
        const uint32_t off = __umul24((uint32_t)tp, stride) + base;
        in.lam[p] = *reinterpret_cast<const float2*>(rb.lam + 2u * off);
        in.qw[p] = *reinterpret_cast<const uint32_t*>(rb.q + off);
        in.kw[p] = *reinterpret_cast<const uint32_t*>(rb.k + off);
    }
}

SSLP_DEVICE int stage_sub16(SubBlock& sb, const SubIn& in, const Meta& mt, int p0, int L, int lane,
                            bool may_freeze) {
    uint32_t frozen = 0;  // bit p: visit p does not select the partition (masking)
    if (may_freeze) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4 s4 = *reinterpret_cast<const int4*>(&mt.slot[p0 + 4 * q]);
            frozen |= ((s4.x < 0 ? 1u : 0u) | (s4.y < 0 ? 2u : 0u) | (s4.z < 0 ? 4u : 0u) |
                       (s4.w < 0 ? 8u : 0u)) << (4 * q);
        }
    }
    float ep0 = 1.f, ep1 = 1.f, em0 = 1.f, em1 = 1.f, af0 = 1.f, af1 = 1.f;
    bool small = false;
    uint32_t kt0[8], kt1[8];  // rows 2l, 2l+1: bf16 pairs of visits (2u, 2u+1)
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const bool valid = p < L;
        const bool live = valid && ((frozen >> p) & 1u) == 0u;
        const float l0 = live ? in.lam[p].x : 1.f, l1 = live ? in.lam[p].y : 1.f;
        small |= l0 < kSmallDecay || l1 < kSmallDecay;
        if (p == 0) {
            af0 = l0;
            af1 = l1;
        } else {
            ep0 *= l0;
            ep1 *= l1;
            // hardware reciprocal (within 1 ulp, not an IEEE division): the
            // factor only scales a key that is rounded to bf16
            em0 *= __builtin_amdgcn_rcpf(l0);
            em1 *= __builtin_amdgcn_rcpf(l1);
        }
        const uint32_t qw = valid ? in.qw[p] : 0u, kw = valid ? in.kw[p] : 0u;
        const float q0 = __uint_as_float(qw << 16), q1 = __uint_as_float(qw & 0xFFFF0000u);
        const float k0 = __uint_as_float(kw << 16), k1 = __uint_as_float(kw & 0xFFFF0000u);
        const uint32_t kp = pk_bf16(k0 * em0, k1 * em1);  // rows 2l (lo), 2l+1 (hi)
        *reinterpret_cast<uint32_t*>(&sb.qs[p][2 * lane]) = pk_bf16(q0 * ep0, q1 * ep1);
        *reinterpret_cast<uint32_t*>(&sb.ks[p][2 * lane]) = kp;
        if (p & 1) {
            // visits p-1 (lo) and p of row 2l, of row 2l+1: byte selects of the two pairs
            kt0[p >> 1] = __builtin_amdgcn_perm(kp, kt0[p >> 1], 0x05040100u);
            kt1[p >> 1] = __builtin_amdgcn_perm(kp, kt1[p >> 1], 0x07060302u);
        } else {
            kt0[p >> 1] = kp;  // completed by the next visit
            kt1[p >> 1] = kp;
        }
    }
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane][0]) = make_uint4(kt0[0], kt0[1], kt0[2], kt0[3]);
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane][8]) = make_uint4(kt0[4], kt0[5], kt0[6], kt0[7]);
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane + 1][0]) = make_uint4(kt1[0], kt1[1], kt1[2], kt1[3]);
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane + 1][8]) = make_uint4(kt1[4], kt1[5], kt1[6], kt1[7]);
    *reinterpret_cast<float2*>(&sb.af[2 * lane]) = make_float2(af0, af1);
    *reinterpret_cast<float2*>(&sb.px[2 * lane]) = make_float2(ep0, ep1);
    return __ballot(small) != 0ull ? 1 : 0;
}

// Stages visits p0 .. p0+L-1 (L <= 16) of the chunk as one sub-block (lane l
// owns state rows 2l, 2l+1).  CUT = false: all L visits; returns whether a
// decay below 2^-4 was met.  CUT = true: ends the block before the visit that
// would take the product of decays after the first visit below 2^-60 in any
// row; returns the number of visits taken.
template <bool CUT>
SSLP_DEVICE int stage_sub(SubBlock& sb, const SubIn& in, const Meta& mt, int p0, int L, int lane) {
    float ep0 = 1.f, ep1 = 1.f, em0 = 1.f, em1 = 1.f, af0 = 1.f, af1 = 1.f;
    int Le = L;
    bool alive = true, small = false;
    uint32_t kt0[8], kt1[8];  // rows 2l, 2l+1: bf16 pairs of visits (2u, 2u+1)
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        float q0 = 0.f, q1 = 0.f, k0 = 0.f, k1 = 0.f;
        if (p < L) {
            // masked execution: a token that does not select the partition
            // leaves its state undecayed (and writes nothing: its gate is 0)
            const bool frozen = mt.slot[p0 + p] < 0;
            const float l0 = frozen ? 1.f : in.lam[p].x, l1 = frozen ? 1.f : in.lam[p].y;
            small |= l0 < kSmallDecay || l1 < kSmallDecay;
            bool take = true;
            if (p == 0) {
                af0 = l0;
                af1 = l1;
            } else if (!CUT) {
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
            if (CUT) take = alive;
            if (take) {
                q0 = __uint_as_float(in.qw[p] << 16);
                q1 = __uint_as_float(in.qw[p] & 0xFFFF0000u);
                k0 = __uint_as_float(in.kw[p] << 16);
                k1 = __uint_as_float(in.kw[p] & 0xFFFF0000u);
            }
        }
        const uint32_t kb0 = f32_to_bf16(k0 * em0).bits, kb1 = f32_to_bf16(k1 * em1).bits;
        *reinterpret_cast<uint32_t*>(&sb.qs[p][2 * lane]) =
            (uint32_t)f32_to_bf16(q0 * ep0).bits | ((uint32_t)f32_to_bf16(q1 * ep1).bits << 16);
        *reinterpret_cast<uint32_t*>(&sb.ks[p][2 * lane]) = kb0 | (kb1 << 16);
        if (p & 1) {
            kt0[p >> 1] |= kb0 << 16;
            kt1[p >> 1] |= kb1 << 16;
        } else {
            kt0[p >> 1] = kb0;
            kt1[p >> 1] = kb1;
        }
    }
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane][0]) = make_uint4(kt0[0], kt0[1], kt0[2], kt0[3]);
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane][8]) = make_uint4(kt0[4], kt0[5], kt0[6], kt0[7]);
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane + 1][0]) = make_uint4(kt1[0], kt1[1], kt1[2], kt1[3]);
    *reinterpret_cast<uint4*>(&sb.kt[2 * lane + 1][8]) = make_uint4(kt1[4], kt1[5], kt1[6], kt1[7]);
    *reinterpret_cast<float2*>(&sb.af[2 * lane]) = make_float2(af0, af1);
    *reinterpret_cast<float2*>(&sb.px[2 * lane]) = make_float2(ep0, ep1);
    if (CUT) return Le;
    return __ballot(small) != 0ull ? 1 : 0;
}

// The gated values of this wavefront's 16 columns for the chunk's L visits
// (zero past L), transposed: vt[n][p] = e_p v_p[col0 + n].
SSLP_DEVICE void stage_values(uint16_t (&vt)[16][LDV], const ValIn& in, const Meta& mt, int L,
                              int lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = lane + 64 * e;
        const int p = idx >> 2, n = 4 * (idx & 3);
        const float g = p < L ? mt.gate[p] : 0.f;
        vt[n][p] = f32_to_bf16(g * __uint_as_float(in.raw[e].x << 16)).bits;
        vt[n + 1][p] = f32_to_bf16(g * __uint_as_float(in.raw[e].x & 0xFFFF0000u)).bits;
        vt[n + 2][p] = f32_to_bf16(g * __uint_as_float(in.raw[e].y << 16)).bits;
        vt[n + 3][p] = f32_to_bf16(g * __uint_as_float(in.raw[e].y & 0xFFFF0000u)).bits;
    }
}

// One sub-block's products on this wavefront's 16-column state slice St
// (accumulator layout: tile m holds rows 16m + 4(lane/16) + j, column
// lane%16).  The sub-block's visits are vt columns vofs .. vofs+L-1 (ALIGNED:
// vofs a multiple of 4 and zero past L).  Returns O^T (rows: columns
// 4(lane/16) + j of the slice; column lane%16: the visit).
template <bool ALIGNED>
SSLP_DEVICE f32x4_t sub_products(f32x4_t (&St)[8], const SubBlock& sb, const uint16_t (&vt)[16][LDV],
                                 int vofs, int L, int lane) {
    const int g4 = lane >> 4, l16 = lane & 15;
    // ---- state decayed by the first visit (per row) ----
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 f = *reinterpret_cast<const float4*>(&sb.af[16 * m + 4 * g4]);
        St[m][0] *= f.x;
        St[m][1] *= f.y;
        St[m][2] *= f.z;
        St[m][3] *= f.w;
    }
    // ---- O^T = S^T Qs^T, k-slots of group g4 = rows {32s+4g4+j, 32s+16+4g4+j} ----
    f32x4_t ot = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8_t bq;
        const uint2 r0 = *reinterpret_cast<const uint2*>(&sb.qs[l16][32 * s + 4 * g4]);
        const uint2 r1 = *reinterpret_cast<const uint2*>(&sb.qs[l16][32 * s + 16 + 4 * g4]);
        bq[0] = __builtin_bit_cast(__bf16, (uint16_t)(r0.x & 0xFFFFu));
        bq[1] = __builtin_bit_cast(__bf16, (uint16_t)(r0.x >> 16));
        bq[2] = __builtin_bit_cast(__bf16, (uint16_t)(r0.y & 0xFFFFu));
        bq[3] = __builtin_bit_cast(__bf16, (uint16_t)(r0.y >> 16));
        bq[4] = __builtin_bit_cast(__bf16, (uint16_t)(r1.x & 0xFFFFu));
        bq[5] = __builtin_bit_cast(__bf16, (uint16_t)(r1.x >> 16));
        bq[6] = __builtin_bit_cast(__bf16, (uint16_t)(r1.y & 0xFFFFu));
        bq[7] = __builtin_bit_cast(__bf16, (uint16_t)(r1.y >> 16));
        bf16x8_t as;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            as[j] = bfv(St[2 * s][j]);
            as[4 + j] = bfv(St[2 * s + 1][j]);
        }
        ot = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as, bq, ot, 0, 0, 0);
    }
    // ---- Pm^T[p'][p] = Ks Qs^T, causal within the sub-block ----
    f32x4_t pm = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(&sb.ks[l16][32 * s + 8 * g4]);
        const bf16x8_t bq = *reinterpret_cast<const bf16x8_t*>(&sb.qs[l16][32 * s + 8 * g4]);
        pm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bq, pm, 0, 0, 0);
    }
    s16x4_t bp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int pp = 4 * g4 + j;  // p' (row), column p = l16
        bp[j] = bfs((pp <= l16 && l16 < L) ? pm[j] : 0.f);
    }
    // the gated values of visits 4 g4 .. 4 g4 + 3 in column l16
    s16x4_t vv;
    if constexpr (ALIGNED) {
        vv = *reinterpret_cast<const s16x4_t*>(&vt[l16][vofs + 4 * g4]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = 4 * g4 + i < L ? (short)vt[l16][vofs + 4 * g4 + i] : (short)0;
    }
    // ---- O^T += Ve^T Pm^T ----
    // (own accumulator, added with VALU: a 16x16x16 MFMA does not take the
    // accumulator of a 16x16x32 MFMA as its C operand)
    {
        const f32x4_t oe = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, bp, f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                                     0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) ot[j] += oe[j];
    }
    // ---- S = PX * (S + Ks^T Ve) ----
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const s16x4_t ak = *reinterpret_cast<const s16x4_t*>(&sb.kt[16 * m + l16][4 * g4]);
        St[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ak, vv, St[m], 0, 0, 0);
        const float4 f = *reinterpret_cast<const float4*>(&sb.px[16 * m + 4 * g4]);
        St[m][0] *= f.x;
        St[m][1] *= f.y;
        St[m][2] *= f.z;
        St[m][3] *= f.w;
    }
    return ot;
}

// e_p o_p of the sub-block's visits into their contribution slots
SSLP_DEVICE void write_contrib(const SseArgs& a, const Meta& mt, f32x4_t ot, int b, int h, int vofs,
                               int L, int col, int lane) {
    const int g4 = lane >> 4, l16 = lane & 15;
    if (l16 >= L) return;
    const int vp = vofs + l16;
    const int slot = mt.slot[vp];
    if (slot < 0) return;
    const float e = mt.gate[vp];
    const size_t bth = ((size_t)b * a.T + mt.tok[vp]) * a.H + h;
    bf16_t* dst = a.opart + (bth * (a.topk + 1) + slot) * a.dv + col + 4 * g4;
    const uint32_t lo = (uint32_t)f32_to_bf16(e * ot[0]).bits | ((uint32_t)f32_to_bf16(e * ot[1]).bits << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(e * ot[2]).bits | ((uint32_t)f32_to_bf16(e * ot[3]).bits << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
}

template <typename io_t>
__global__ __launch_bounds__(64 * NWV, 2) void sse_gla_kernel(SseArgs a) {
    __shared__ GlaSmem sm;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int BH = a.B * a.H, N = a.N, T = a.T, dv = a.dv;
    const int ncb = dv / DB;
    // XCD-aware placement: workgroups x and x + 8 share an XCD; the ncb column
    // blocks of a partition sequence take consecutive multiples of 8
    const int x = blockIdx.x, xcd = x & 7, kq = x >> 3;
    const int inst = (kq / ncb) * 8 + xcd, cb = kq % ncb;
    if (inst >= BH * (N + 1)) return;
    // sequences 0 .. BH-1: shared partitions; then the routed ones, (b, h) major
    const bool shared = inst < BH;
    const int bh = shared ? inst : (inst - BH) / N;
    const int part = shared ? N : (inst - BH) - ((inst - BH) / N) * N;
    const int cnt = shared ? T : a.cnt[bh * N + part];
    if (cnt == 0) return;  // an idle partition keeps its state untouched
    // the shared sequences (every token) are the kernel's critical path: their
    // wavefronts win the issue arbitration against the routed ones on a unit
    if (shared) __builtin_amdgcn_s_setprio(3);
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const io_t* qg = static_cast<const io_t*>(shared && a.q_sh ? a.q_sh : a.q);
    const io_t* kg = static_cast<const io_t*>(shared && a.k_sh ? a.k_sh : a.k);
    const io_t* vg = static_cast<const io_t*>(a.v);
    const uint32_t* vis = a.vis + ((size_t)bh * N + part) * T;
    const float* vgl = a.vgl + ((size_t)bh * N + part) * T;
    const int col = cb * DB + 16 * w;  // this wavefront's 16 columns
    const size_t brow = (size_t)b * T * a.H;  // first (token, head) row of batch b
    const RowBases rb{reinterpret_cast<const char*>(qg + brow * CR), reinterpret_cast<const char*>(kg + brow * CR),
                      reinterpret_cast<const char*>(a.lam + brow * CR), reinterpret_cast<const char*>(vg + brow * dv)};
    float* Sg = a.S + ((size_t)bh * (N + 1) + part) * CR * dv;

    // state element (row 16m + 4 g4 + j, column col + l16): a uniform row base
    // plus one per-lane offset, so no address is held through the chunk loop
    const uint32_t soff = (uint32_t)(4 * g4) * (uint32_t)dv + (uint32_t)(col + l16);
    f32x4_t St[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) St[m][j] = (Sg + (size_t)(16 * m + j) * dv)[soff];

    // The visits of chunk c sit in LDS buffer c & 1.  Wavefront 0 holds the
    // next chunk's list in registers (requested a chunk ahead) and writes it
    // out while the current chunk is staged.
    const int nch = (cnt + CH - 1) / CH;
    const bool may_freeze = a.masking && !shared;
    uint32_t nx_ent = 0;  // wavefront 0, lane p: visit p of the chunk to come
    float nx_gate = 0.f;
    auto fetch_list = [&](int c) {
        const int p = c * CH + lane;
        if (!shared && p < cnt) {
            nx_ent = vis[p];
            nx_gate = vgl[p];
        }
    };
    auto put_list = [&](int c) {
        const int p = c * CH + lane;
        if (p < cnt) {
            int t, slot;
            float gate;
            if (shared) {
                t = p;
                slot = a.topk;
                gate = 1.f;
            } else {
                const uint32_t rk = nx_ent & 7u;
                t = (int)(nx_ent >> 3);
                slot = rk == kNoRank ? -1 : (int)rk;
                gate = nx_gate;
            }
            sm.vtok[c & 1][lane] = t;
            sm.vslot[c & 1][lane] = slot;
            sm.vgate[c & 1][lane] = gate;
        }
    };
    if (w == 0) {
        fetch_list(0);
        put_list(0);
        if (nch > 1) fetch_list(1);
    }
    block_sync_lds();
    for (int c = 0; c < nch; ++c) {
        const int L = cnt - c * CH < CH ? cnt - c * CH : CH;
        const Meta mc{sm.vtok[c & 1], sm.vgate[c & 1], sm.vslot[c & 1]};
        // ---- sub-block w (shared by all columns) and this wave's values, from
        //      one batch of loads ----
        {
            const int Lw = L - 16 * w < 16 ? L - 16 * w : 16;
            SubIn in;
            ValIn vin;
            if (Lw > 0) load_sub16(in, a, rb, h, mc, 16 * w, Lw, lane);
            load_values(vin, a, rb, h, mc, L, col, lane);
            int small = 0;
            if (Lw > 0) small = stage_sub16(sm.sb[w], in, mc, 16 * w, Lw, lane, may_freeze);
            if (lane == 0) sm.small[w] = small;
            stage_values(sm.vt[w], vin, mc, L, lane);
        }
        if (w == 0 && c + 1 < nch) {
            put_list(c + 1);
            if (c + 2 < nch) fetch_list(c + 2);
        }
        block_sync_lds();
        if ((sm.small[0] | sm.small[1] | sm.small[2] | sm.small[3]) == 0) {
            for (int r = 0; r < NWV && 16 * r < L; ++r) {
                const int Lr = L - 16 * r < 16 ? L - 16 * r : 16;
                const f32x4_t ot = sub_products<true>(St, sm.sb[r], sm.vt[w], 16 * r, Lr, lane);
                write_contrib(a, mc, ot, b, h, 16 * r, Lr, col, lane);
            }
        } else {
            // a decay below 2^-4 in the chunk: blocks that end before the product
            // of decays falls below 2^-60, each wavefront staging its own
            for (int p0 = 0; p0 < L;) {
                const int Lb = L - p0 < 16 ? L - p0 : 16;
                SubIn in;
                load_sub(in, a, rb, h, mc, p0, Lb, lane);
                const int Le = stage_sub<true>(sm.sb[w], in, mc, p0, Lb, lane);
                wave_sync();
                const f32x4_t ot = sub_products<false>(St, sm.sb[w], sm.vt[w], p0, Le, lane);
                write_contrib(a, mc, ot, b, h, p0, Le, col, lane);
                wave_sync();
                p0 += Le;
            }
        }
        block_sync_lds();
    }
    // the store addresses are formed here, not kept from the loads through the
    // chunk loop (the compiler otherwise holds all 32 of them in registers)
    float* Sout = Sg;
    uint32_t sout = soff;
    asm volatile("" : "+s"(Sout), "+v"(sout));
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) (Sout + (size_t)(16 * m + j) * dv)[sout] = St[m][j];
}

// o_t = its topk routed contributions in rank order, then the shared one
template <typename io_t>
__global__ __launch_bounds__(256) void sse_combine_kernel(const bf16_t* __restrict__ opart, int K1,
                                                          int dv, long long nquad,
                                                          io_t* __restrict__ o) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= nquad) return;
    const long long pth = idx / (dv / 4);
    const int c = (int)(idx - pth * (dv / 4)) * 4;
    // every slot's load is issued before the sums (slots past K1 re-read the
    // last one and are not added), which are taken in slot order
    uint2 u[MAXK + 1];
#pragma unroll
    for (int r = 0; r <= MAXK; ++r)
        u[r] = *reinterpret_cast<const uint2*>(opart + ((size_t)pth * K1 + (r < K1 ? r : K1 - 1)) * dv + c);
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int r = 0; r <= MAXK; ++r) {
        const bool in = r < K1;  // adding +0 for the slots past K1 leaves each sum unchanged
        s0 += in ? __uint_as_float(u[r].x << 16) : 0.f;
        s1 += in ? __uint_as_float(u[r].x & 0xFFFF0000u) : 0.f;
        s2 += in ? __uint_as_float(u[r].y << 16) : 0.f;
        s3 += in ? __uint_as_float(u[r].y & 0xFFFF0000u) : 0.f;
    }
    io_t* dst = o + (size_t)pth * dv + c;
    dst[0] = from_f32<io_t>(s0);
    dst[1] = from_f32<io_t>(s1);
    dst[2] = from_f32<io_t>(s2);
    dst[3] = from_f32<io_t>(s3);
}

}  // namespace

size_t sse_scratch_bytes(int B, int T, int H, int N, int topk, int dv) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return 2 * al((size_t)B * H * N * T * 4) + al((size_t)B * H * N * 4) +
           al((size_t)B * T * H * (topk + 1) * dv * 2) + al((size_t)B * H * T * 4) +
           al((size_t)B * H * T * 16);
}

hipError_t launch_sse(int B, int T, int H, int N, int topk, int dv, int dtype,
                      const float* logits, const void* q, const void* k, const void* v,
                      const float* lam, const void* q_sh, const void* k_sh, float* S, void* o,
                      int32_t* sel, float* e_sel, void* scratch, hipStream_t st, int masking) {
    if (dtype != 1 || N > MAXN || topk > MAXK || dv % DB != 0) return hipErrorInvalidValue;
    // row offsets inside a batch are 32-bit (fp32 Lambda rows: T*H*c*4 bytes)
    if ((long long)T * H * CR * 4 >= (1ll << 31) || (long long)T * H * dv * 2 >= (1ll << 31))
        return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char* ws = static_cast<char*>(scratch);
    const size_t lb = al((size_t)B * H * N * T * 4);
    uint32_t* vis = reinterpret_cast<uint32_t*>(ws);
    float* vgl = reinterpret_cast<float*>(ws + lb);
    int* cnt = reinterpret_cast<int*>(ws + 2 * lb);
    const size_t lo = 2 * lb + al((size_t)B * H * N * 4);
    bf16_t* opart = reinterpret_cast<bf16_t*>(ws + lo);
    const size_t lr = lo + al((size_t)B * T * H * (topk + 1) * dv * 2);
    uint32_t* rsel = reinterpret_cast<uint32_t*>(ws + lr);
    float4* rgate = reinterpret_cast<float4*>(ws + lr + al((size_t)B * H * T * 4));
    SseArgs a{B, T, H, N, topk, dv, logits, q, k, v, lam, q_sh, k_sh, S, o, sel, e_sel, masking,
              vis, vgl, rsel, rgate, cnt, opart};
    const int P = B * T * H;
    sse_route_kernel<<<(unsigned)((P + 255) / 256), 256, 0, st>>>(logits, P, N, topk, sel, e_sel, T,
                                                                   H, rsel, rgate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    sse_bucket_kernel<<<(unsigned)(B * H), 64 * BKW, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 8 * ncb consecutive workgroups hold 8 partition sequences, one per XCD
    const long long nseq = (long long)B * H * (N + 1);
    const long long grid = ((nseq + 7) / 8) * 8 * (dv / DB);
    sse_gla_kernel<bf16_t><<<(unsigned)grid, 64 * NWV, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long long nquad = (long long)P * (dv / 4);
    sse_combine_kernel<bf16_t><<<(unsigned)((nquad + 255) / 256), 256, 0, st>>>(
        opart, topk + 1, dv, nquad, static_cast<bf16_t*>(o));
    return hipGetLastError();
}

}  // namespace sslp
