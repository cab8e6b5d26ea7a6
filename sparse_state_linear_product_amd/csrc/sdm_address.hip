// K1: product-key addressing for Sparse Delta Memory, one wavefront per problem.
//
// Slides "Sparse Delta Memory: Scaling the State of Linear RNNs through
// Sparsity", "Product keys select addresses without scoring every slot":
// slot (a,b) scores k'_1[a] + k'_2[b]; keep each half's top-k, form the k^2
// candidate sums, select the top `budget`, softmax over the selected scores.
//
// Ranking everywhere is (fp32 score desc, index asc) encoded as a 64-bit key
// (common.h), so selection results are unique and reproducible bit for bit.
//
// Algorithm per problem (one wave64):
//  1. both halves -> keys, wave bitonic sort (EH keys per lane), top-k of each
//     half is then held by lanes 0..k-1 (k <= 64) and staged in LDS; with k
//     and the budget at most KC (32 or 64) only the top KC of each half and of
//     D (step 2) are sorted (bitonic_topk_desc), else everything is;
//  2. D = {(i,j) : (i+1)(j+1) <= budget} over the two sorted top-k lists.  With
//     no rounding ties the top-budget candidates all lie in D, because a pair
//     outside D is dominated (both ranks smaller or equal) by more than
//     `budget` pairs whose fp32 sums are >= its own.  D depends on k and the
//     budget only: the host lists its (i, j) pairs in the launch arguments
//     (DMap), lane l forms the keys of positions e*64 + l.  D is sorted (ED
//     keys per lane) and tau = its budget-th key;
//  3. F = #{all k^2 candidates with key >= tau} is counted exactly.  F ==
//     budget proves D's top-budget is the answer.  Otherwise (rounding ties
//     let a pair outside D win on the slot index) the exact top-budget is
//     extracted from all k^2 candidates by repeated wave max;
//  4. softmax in fp32 over the selected scores.
#include <type_traits>

#include "addr_wg.h"
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

struct AddrArgs {
    const void* s1;
    const void* s2;
    int32_t* idx;
    float* wt;
    int P, sqrtN, k, budget, nD;
};

constexpr int kWavesPerBlock = 4;

// the pairs of D, (i << 8) | j at position p < nD (i, j < 64)
template <int ED>
struct DMap {
    uint16_t ij[64 * ED];
};

// KC: 32 or 64 when k and the budget are at most KC (top-KC sorts), 0 otherwise
template <typename in_t, int EH, int ED, int KC>
__global__ __launch_bounds__(256) void sdm_address_kernel(AddrArgs a, DMap<ED> dm) {
    __shared__ float s_score[kWavesPerBlock][2][64];
    __shared__ int s_index[kWavesPerBlock][2][64];

    const int wv = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.x * kWavesPerBlock + wv;
    if (p >= a.P) return;  // whole wave leaves; no block barrier is used below

    const int n = a.sqrtN, k = a.k, budget = a.budget;
    const in_t* h1 = static_cast<const in_t*>(a.s1) + (size_t)p * n;
    const in_t* h2 = static_cast<const in_t*>(a.s2) + (size_t)p * n;

    // 1. per-half sort; key 0 is below every finite score's key (padding)
    {
        // all scores requested at once, from clamped positions (a conditional
        // load would be waited for one at a time); padding is applied after
        in_t r1[EH], r2[EH];
#pragma unroll
        for (int e = 0; e < EH; ++e) {
            const int pos = min(e * 64 + lane, n - 1);
            r1[e] = h1[pos];
            r2[e] = h2[pos];
        }
        if constexpr (std::is_same<in_t, bf16_t>::value) {
            // bf16 scores and indices below 2^16 fit a 32-bit key of the same order
            uint32_t x1[EH], x2[EH];
#pragma unroll
            for (int e = 0; e < EH; ++e) {
                const int pos = e * 64 + lane;
                x1[e] = pos < n ? make_key32(to_f32(r1[e]), (uint32_t)pos) : 0u;
                x2[e] = pos < n ? make_key32(to_f32(r2[e]), (uint32_t)pos) : 0u;
            }
            if constexpr (KC == 0) {
                bitonic_sort_desc32<EH>(x1, lane);
                bitonic_sort_desc32<EH>(x2, lane);
            } else {
                bitonic_topk_desc<KC>(x1, lane);
                bitonic_topk_desc<KC>(x2, lane);
            }
            if (lane < k) {
                s_score[wv][0][lane] = key32_score(x1[0]);
                s_index[wv][0][lane] = (int)key32_index(x1[0]);
                s_score[wv][1][lane] = key32_score(x2[0]);
                s_index[wv][1][lane] = (int)key32_index(x2[0]);
            }
        } else {
            uint64_t x1[EH], x2[EH];
#pragma unroll
            for (int e = 0; e < EH; ++e) {
                const int pos = e * 64 + lane;
                x1[e] = pos < n ? make_key(to_f32(r1[e]), (uint32_t)pos) : 0ull;
                x2[e] = pos < n ? make_key(to_f32(r2[e]), (uint32_t)pos) : 0ull;
            }
            if constexpr (KC == 0) {
                bitonic_sort_desc<EH>(x1, lane);
                bitonic_sort_desc<EH>(x2, lane);
            } else {
                bitonic_topk_desc<KC>(x1, lane);
                bitonic_topk_desc<KC>(x2, lane);
            }
            if (lane < k) {
                s_score[wv][0][lane] = key_score(x1[0]);
                s_index[wv][0][lane] = (int)key_index(x1[0]);
                s_score[wv][1][lane] = key_score(x2[0]);
                s_index[wv][1][lane] = (int)key_index(x2[0]);
            }
        }
    }
    wave_sync();

    // 2. the keys of D's pairs, positions e*64 + lane
    uint64_t d[ED];
#pragma unroll
    for (int e = 0; e < ED; ++e) {
        const int pos = e * 64 + lane;
        const uint32_t ij = dm.ij[pos];
        const int i = (int)(ij >> 8), j = (int)(ij & 255u);
        const float sum = s_score[wv][0][i] + s_score[wv][1][j];  // one fp32 RNE add
        const uint32_t slot = (uint32_t)s_index[wv][0][i] * (uint32_t)n + (uint32_t)s_index[wv][1][j];
        d[e] = pos < a.nD ? make_key(sum, slot) : 0ull;
    }
    if constexpr (KC == 0) bitonic_sort_desc<ED>(d, lane);
    else bitonic_topk_desc<KC>(d, lane);  // (only d[0] is kept: budget <= KC <= 64)
    const uint64_t tau = wave_get<ED>(d, budget - 1);

    // 3. exact count of candidates at or above tau: 64 / k rows of the k x k
    //    candidates per pass, lane = (row in pass) * k + column, the column's
    //    score and index held in registers
    int F = 0;
    {
        const int rpp = 64 / k;  // rows per pass
        const int li = lane / k, lj = lane - li * k;
        const bool lane_ok = li < rpp;
        const float sb = s_score[wv][1][lane_ok ? lj : 0];
        const uint32_t ib = (uint32_t)s_index[wv][1][lane_ok ? lj : 0];
        for (int i0 = 0; i0 < k; i0 += rpp) {
            const int i = i0 + li;
            const bool ok = lane_ok && i < k;
            const int ic = ok ? i : 0;
            const float sum = s_score[wv][0][ic] + sb;  // one fp32 RNE add, as in step 2
            const uint32_t slot = (uint32_t)s_index[wv][0][ic] * (uint32_t)n + ib;
            F += __popcll(__ballot(ok && make_key(sum, slot) >= tau));
        }
    }

    int32_t* out_i = a.idx + (size_t)p * budget;
    float* out_w = a.wt + (size_t)p * budget;
    if (F == budget) {
        // 4. softmax over the selected fp32 scores (rank 0 holds the maximum)
        const float smax = key_score(wave_get<ED>(d, 0));
        float w[ED];
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < ED; ++e) {
            const int pos = e * 64 + lane;
            w[e] = pos < budget ? __expf(key_score(d[e]) - smax) : 0.f;
            part += w[e];
        }
        const float z = wave_sum(part);
#pragma unroll
        for (int e = 0; e < ED; ++e) {
            const int pos = e * 64 + lane;
            if (pos < budget) {
                out_i[pos] = (int32_t)key_index(d[e]);
                out_w[pos] = w[e] / z;
            }
        }
        return;
    }

    // rare path: exact top-`budget` of all k^2 candidates by repeated maximum
    const int kk = k * k;
    uint64_t bound = ~0ull;  // exclusive upper bound (no finite key reaches it)
    float smax = 0.f, z = 0.f;
    float wl0 = 0.f, wl1 = 0.f;  // weight of rank r kept by lane r % 64 (budget <= 128)
    for (int r = 0; r < budget; ++r) {
        uint64_t best = 0ull;
        for (int base = 0; base < kk; base += 64) {
            const int x = base + lane;
            if (x < kk) {
                const int i = x / k, j = x - (x / k) * k;
                const float sum = s_score[wv][0][i] + s_score[wv][1][j];
                const uint32_t slot =
                    (uint32_t)s_index[wv][0][i] * (uint32_t)n + (uint32_t)s_index[wv][1][j];
                const uint64_t key = make_key(sum, slot);
                if (key < bound && key > best) best = key;
            }
        }
        best = wave_max_u64(best);
        bound = best;
        const float sc = key_score(best);
        if (r == 0) smax = sc;
        const float w = __expf(sc - smax);
        z += w;
        if (lane == 0) out_i[r] = (int32_t)key_index(best);
        if (lane == (r & 63)) {
            if (r < 64) wl0 = w;
            else wl1 = w;
        }
    }
    if (lane < budget) out_w[lane] = wl0 / z;
    if (lane + 64 < budget) out_w[lane + 64] = wl1 / z;
}

// ---------------------------------------------------------------------------
// Latency-oriented variant for small batches (a decode step): one workgroup of
// 256 threads per problem (the steps of addr_wg.h), and the write and read
// problems of a step in one launch.
// ---------------------------------------------------------------------------
constexpr int WG = kAddrGroup;

struct AddrPairArgs {
    const void* s1[2];
    const void* s2[2];
    int32_t* idx[2];
    float* wt[2];
    int k[2], budget[2], nD[2];
    int P, sqrtN;
};

template <typename in_t>
__global__ __launch_bounds__(WG) void sdm_address_wg_kernel(AddrPairArgs a) {
    __shared__ WgAddrSmem sm;
    const int t = threadIdx.x;
    const int set = blockIdx.x >= (unsigned)a.P ? 1 : 0;
    const int p = (int)blockIdx.x - set * a.P;
    const size_t off = (size_t)p * a.sqrtN;
    const WgAddrProblem pr{static_cast<const in_t*>(a.s1[set]) + off,
                           static_cast<const in_t*>(a.s2[set]) + off, a.sqrtN, a.k[set],
                           a.budget[set], a.nD[set]};
    int32_t* oi = a.idx[set] + (size_t)p * pr.budget;
    float* ow = a.wt[set] + (size_t)p * pr.budget;
    wg_addr_select<in_t>(pr, t, sm, oi, ow, nullptr, nullptr);
    if (sm.F != pr.budget) {  // uniform over the workgroup
        wg_addr_rank_all(pr, t, sm);
        wg_addr_softmax(pr, t, sm, oi, ow, nullptr, nullptr);
    }
}

int ceil_pow2_units(int n) {  // smallest power of two >= ceil(n/64), at least 1
    int e = 1;
    while (64 * e < n) e <<= 1;
    return e;
}

// Set sizes that each KC can meet: with k, budget <= 32 the set D holds at
// most 119 keys (ED <= 2), with budget <= 64 at most 512; KC = 0 takes every
// size (dispatch_kc falls back to it).
constexpr bool ed_instantiated(int KC, int ED) { return KC == 0 || ED <= (KC == 32 ? 2 : 8); }

template <typename in_t, int EH, int ED, int KC>
void launch_one(dim3 grid, hipStream_t st, const AddrArgs& a) {
    if constexpr (ed_instantiated(KC, ED)) {
        DMap<ED> dm{};  // pairs row by row; positions past nD stay (0, 0) and are padded
        int p = 0;
        for (int i = 0; i < a.k; ++i) {
            const int c = a.budget / (i + 1) < a.k ? a.budget / (i + 1) : a.k;
            for (int j = 0; j < c; ++j) dm.ij[p++] = (uint16_t)((i << 8) | j);
        }
        sdm_address_kernel<in_t, EH, ED, KC><<<grid, 256, 0, st>>>(a, dm);
    }
}

template <typename in_t, int EH, int KC>
hipError_t dispatch_ed(int ED, dim3 grid, hipStream_t st, const AddrArgs& a) {
    switch (ED) {
        case 1: launch_one<in_t, EH, 1, KC>(grid, st, a); break;
        case 2: launch_one<in_t, EH, 2, KC>(grid, st, a); break;
        case 4: launch_one<in_t, EH, 4, KC>(grid, st, a); break;
        case 8: launch_one<in_t, EH, 8, KC>(grid, st, a); break;
        case 16: launch_one<in_t, EH, 16, KC>(grid, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename in_t, int KC>
hipError_t dispatch_eh(int EH, int ED, dim3 grid, hipStream_t st, const AddrArgs& a) {
    switch (EH) {
        case 1: return dispatch_ed<in_t, 1, KC>(ED, grid, st, a);
        case 2: return dispatch_ed<in_t, 2, KC>(ED, grid, st, a);
        case 4: return dispatch_ed<in_t, 4, KC>(ED, grid, st, a);
        case 8: return dispatch_ed<in_t, 8, KC>(ED, grid, st, a);
        case 16: return dispatch_ed<in_t, 16, KC>(ED, grid, st, a);
        default: return hipErrorInvalidValue;
    }
}

template <typename in_t>
hipError_t dispatch_kc(int EH, int ED, dim3 grid, hipStream_t st, const AddrArgs& a) {
    // top-KC sorts where k and the budget allow them (k <= 64 always)
    if (a.k <= 32 && a.budget <= 32 && ed_instantiated(32, ED))
        return dispatch_eh<in_t, 32>(EH, ED, grid, st, a);
    if (a.budget <= 64 && ed_instantiated(64, ED)) return dispatch_eh<in_t, 64>(EH, ED, grid, st, a);
    return dispatch_eh<in_t, 0>(EH, ED, grid, st, a);
}

}  // namespace

int address_set_size(int k, int budget) { return address_set_size_host(k, budget); }

// below this many problems the one-workgroup-per-problem kernel has the lower latency
constexpr int kWgMaxProblems = 1024;

hipError_t launch_sdm_address_pair(int P, int sqrtN, int dtype, const void* sw1, const void* sw2,
                                   int k_w, int W, int32_t* iw, float* ww, const void* sr1,
                                   const void* sr2, int k_r, int R, int32_t* ir, float* wr,
                                   hipStream_t st) {
    if (P <= 0) return hipSuccess;
    if (P <= kWgMaxProblems && wg_address_fits(sqrtN, k_w, W) && wg_address_fits(sqrtN, k_r, R)) {
        AddrPairArgs a{{sw1, sr1}, {sw2, sr2}, {iw, ir}, {ww, wr}, {k_w, k_r}, {W, R},
                       {address_set_size(k_w, W), address_set_size(k_r, R)}, P, sqrtN};
        if (dtype == 0) sdm_address_wg_kernel<float><<<(unsigned)(2 * P), WG, 0, st>>>(a);
        else sdm_address_wg_kernel<bf16_t><<<(unsigned)(2 * P), WG, 0, st>>>(a);
        return hipGetLastError();
    }
    hipError_t e = launch_sdm_address(P, sqrtN, dtype, sw1, sw2, k_w, W, iw, ww, st);
    if (e != hipSuccess) return e;
    return launch_sdm_address(P, sqrtN, dtype, sr1, sr2, k_r, R, ir, wr, st);
}

hipError_t launch_sdm_address(int P, int sqrtN, int dtype, const void* s1, const void* s2, int k,
                              int budget, int32_t* idx, float* wt, hipStream_t st) {
    if (P <= 0) return hipSuccess;
    if (P <= kWgMaxProblems && wg_address_fits(sqrtN, k, budget)) {  // one set: blocks 0..P-1
        const int nD = address_set_size(k, budget);
        AddrPairArgs g{{s1, s1}, {s2, s2}, {idx, idx}, {wt, wt}, {k, k}, {budget, budget}, {nD, nD},
                       P, sqrtN};
        if (dtype == 0) sdm_address_wg_kernel<float><<<(unsigned)P, WG, 0, st>>>(g);
        else sdm_address_wg_kernel<bf16_t><<<(unsigned)P, WG, 0, st>>>(g);
        return hipGetLastError();
    }
    AddrArgs a{s1, s2, idx, wt, P, sqrtN, k, budget, address_set_size(k, budget)};
    const int EH = ceil_pow2_units(sqrtN);
    const int ED = ceil_pow2_units(a.nD);
    dim3 grid((P + kWavesPerBlock - 1) / kWavesPerBlock);
    if (dtype == 0) return dispatch_kc<float>(EH, ED, grid, st, a);
    return dispatch_kc<bf16_t>(EH, ED, grid, st, a);
}

}  // namespace sslp
