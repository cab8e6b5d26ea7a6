// Product-key addressing of one problem by a group of 256 threads (slides
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// "Product keys select addresses without scoring every slot"): the steps of
// the latency-oriented workgroup variant, as device functions so that the
// standalone addressing kernel and the fused decode kernel run the same code.
//
// Ranking is (fp32 score desc, index asc) as a 64-bit key (common.h; a 32-bit
// key of the same order for bf16 half scores):
//   1. per-half top-k: each wavefront sorts its 64 keys of each half in
//      registers; one wavefront per half merges the four sorted lists into the
//      half's top 64 in rank order (merge4_top64; keys are distinct, padding
//      keys are 0, below every key);
//   2. the dominance set D = {(i, j) : (i+1)(j+1) <= budget}: each wavefront
//      sorts its 64 entries, one wavefront merges them (merge4_top64);
//      tau = the budget-th key;
//   3. F = #{k^2 candidates with key >= tau}, counted by the group's four
//      wavefronts; F == budget proves D's top-budget is the answer, else all
//      k^2 candidates are ranked by counting (wg_addr_rank_all, the rare path
//      of rounding ties);
//   4. softmax over the selected scores: on the common path by wavefront 0
//      inside wg_addr_select, else by wg_addr_softmax.
// Every function contains block-wide barriers (LDS-only: they do not wait for
// global stores): all threads of the workgroup call it, each 256-thread group
// on its own problem and shared memory.
// Limits: sqrtN <= 256, k <= 64, budget <= 64, |D| <= 256.
#pragma once

#include <type_traits>

#include "common.h"

namespace sslp {

constexpr int kAddrGroup = 256;  // threads per addressing problem

// NCAND >= max(256, k^2): D on the common path, all k^2 candidates on the rare one
template <int NCAND>
struct WgAddrSmemT {
    union {
        uint64_t top[2][kAddrGroup];    // per half: each wave's sorted top-k of its 64 keys
        uint32_t top32[2][kAddrGroup];  // the same as 32-bit keys (bf16 scores)
    };
    float hsc[2][64];
    int hix[2][64];
    uint64_t cand[NCAND];  // D, or all k^2 candidates on the rare path
    uint64_t sel[64];
    uint64_t tau;
    int F;
    int Fw[kAddrGroup / 64];  // per-wavefront counts
    int drow[kAddrGroup], doff[65];  // D: row of each entry, first entry of each row
};
using WgAddrSmem = WgAddrSmemT<4096>;  // any k <= 64

struct WgAddrProblem {
    const void* s1;  // [.., sqrtN] half scores of this problem
    const void* s2;
    int n, k, budget, nD;
};

inline int address_set_size_host(int k, int budget) {
    int nD = 0;
    for (int i = 0; i < k; ++i) {
        int c = budget / (i + 1);
        nD += c < k ? c : k;
    }
    return nD;
}

inline bool wg_address_fits(int sqrtN, int k, int budget) {
    return sqrtN <= kAddrGroup && k <= 64 && budget <= 64 &&
           address_set_size_host(k, budget) <= kAddrGroup;
}

// Descending order of a bitonic sequence of 64 keys held one per lane: at each
// distance J = 32 .. 1 the lower lane of a pair keeps the larger key.
template <typename Key>
SSLP_DEVICE Key bitonic_merge64_desc(Key x, int lane) {
    auto step = [&](auto jc) {
        constexpr int J = decltype(jc)::value;
        const Key o = xor_lane_c<J>(x, lane);
        x = ((lane & J) == 0) ? (x > o ? x : o) : (x > o ? o : x);
    };
    step(std::integral_constant<int, 32>{});
    step(std::integral_constant<int, 16>{});
    step(std::integral_constant<int, 8>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 1>{});
    return x;
}

// The 64 largest of two descending lists of 64 keys (lst[i], lst[64 + i]), in
// rank order: lane r returns the rank-r key.  Run by one whole wavefront.
template <typename Key>
SSLP_DEVICE Key merge2_top64(const Key* lst, int lane) {
    const Key a = lst[lane], b = lst[64 + 63 - lane];
    return bitonic_merge64_desc(a > b ? a : b, lane);
}

// The 64 largest of four descending lists of 64 keys (lst[64 l + i], list l),
// in rank order: lane r returns the rank-r key.  Run by one whole wavefront.
// The elementwise maximum of a descending list and a reversed one holds the 64
// largest of the two as a bitonic sequence; two rounds of that and a merge.
template <typename Key>
SSLP_DEVICE Key merge4_top64(const Key* lst, int lane) {
    Key a0 = lst[lane], b0 = lst[64 + 63 - lane];
    Key a1 = lst[128 + lane], b1 = lst[192 + 63 - lane];
    a0 = bitonic_merge64_desc(a0 > b0 ? a0 : b0, lane);
    a1 = bitonic_merge64_desc(a1 > b1 ? a1 : b1, lane);
    Key r1;  // a1 reversed across the lanes
    if constexpr (sizeof(Key) == 8) {
        r1 = shfl_u64(a1, 63 - lane);
    } else {
        r1 = (Key)__shfl((uint32_t)a1, 63 - lane, 64);
    }
    return bitonic_merge64_desc(a0 > r1 ? a0 : r1, lane);
}

// Steps 1-3 and, when F == budget, step 4 into idx / wt (and idx2 / wt2; any
// of them may be null).  Ends with a barrier: sm.F is then valid for every
// thread, and F != budget calls for wg_addr_rank_all and wg_addr_softmax.
template <typename in_t, typename Sm>
SSLP_DEVICE void wg_addr_select(const WgAddrProblem& pr, int t, Sm& sm, int32_t* idx,
                                float* wt, int32_t* idx2, float* wt2) {
    const int lane = t & 63, wv = t >> 6;
    const int n = pr.n, k = pr.k, budget = pr.budget, nD = pr.nD;
    const in_t* h1 = static_cast<const in_t*>(pr.s1);
    const in_t* h2 = static_cast<const in_t*>(pr.s2);
    // the half scores, requested before the wave 0 work below
    in_t r1 = h1[min(t, n - 1)], r2 = h2[min(t, n - 1)];
    if (wv == 0) {
        // D row by row: row i has min(budget / (i+1), k) entries; lane i
        // writes its row's entries of the map
        int c = lane < k ? budget / (lane + 1) : 0;
        c = c < k ? c : k;
        int incl = c;
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
            const int o = __shfl_up(incl, s, 64);
            if (lane >= s) incl += o;
        }
        const int off = incl - c;
        if (lane < k) sm.doff[lane] = off;
        for (int e = 0; e < c; ++e) sm.drow[off + e] = lane;
    }
    if (t == 0) {
        sm.F = 0;
        sm.tau = 0ull;  // below every key: only read if D had fewer than budget entries
    }
    if constexpr (std::is_same<in_t, bf16_t>::value) {
        // bf16 scores and indices below 2^16: 32-bit keys of the same order
        uint32_t x1[1] = {t < n ? make_key32(to_f32(r1), (uint32_t)t) : 0u};
        uint32_t x2[1] = {t < n ? make_key32(to_f32(r2), (uint32_t)t) : 0u};
        bitonic_sort_desc32<1>(x1, lane);
        bitonic_sort_desc32<1>(x2, lane);
        sm.top32[0][t] = x1[0];
        sm.top32[1][t] = x2[0];
        block_sync_lds();
        if (wv < 2) {  // wavefront hh ranks half hh
            const uint32_t key = merge4_top64(&sm.top32[wv][0], lane);
            if (lane < k) {
                sm.hsc[wv][lane] = key32_score(key);
                sm.hix[wv][lane] = (int)key32_index(key);
            }
        }
    } else {
        uint64_t x1[1] = {t < n ? make_key(to_f32(r1), (uint32_t)t) : 0ull};
        uint64_t x2[1] = {t < n ? make_key(to_f32(r2), (uint32_t)t) : 0ull};
        bitonic_sort_desc<1>(x1, lane);
        bitonic_sort_desc<1>(x2, lane);
        sm.top[0][t] = x1[0];
        sm.top[1][t] = x2[0];
        block_sync_lds();
        if (wv < 2) {  // wavefront hh ranks half hh
            const uint64_t key = merge4_top64(&sm.top[wv][0], lane);
            if (lane < k) {
                sm.hsc[wv][lane] = key_score(key);
                sm.hix[wv][lane] = (int)key_index(key);
            }
        }
    }
    block_sync_lds();
    // 2. D in rank order: the wavefronts holding entries sort their 64 (past
    //    nD: key 0, below all keys), one wavefront merges the lists; tau = the
    //    budget-th key (0 if D has fewer than budget entries)
    uint64_t dkey[1] = {0ull};
    if (t < nD) {
        const int i = sm.drow[t];
        const int j = t - sm.doff[i];
        const float sum = sm.hsc[0][i] + sm.hsc[1][j];  // one fp32 RNE add
        dkey[0] = make_key(sum, (uint32_t)sm.hix[0][i] * (uint32_t)n + (uint32_t)sm.hix[1][j]);
    }
    if (wv * 64 < nD) bitonic_sort_desc<1>(dkey, lane);  // uniform over the wavefront
    sm.cand[t] = dkey[0];
    block_sync_lds();
    // tau = the budget-th key of D (0 if D has fewer than budget entries),
    // merged by wavefront 0, which keeps D's ranked top 64 in `key`
    uint64_t key = 0ull;
    if (wv == 0) {
        key = nD <= 128 ? merge2_top64(&sm.cand[0], lane) : merge4_top64(&sm.cand[0], lane);
        const uint64_t tau = shfl_u64(key, budget - 1);
        if (lane == 0) sm.tau = tau;
    }
    block_sync_lds();
    // 3. exact count of all k^2 candidates at or above tau, spread over the
    //    group's four wavefronts: kAddrGroup / k rows of candidates (i, j) per
    //    pass, thread t on row t / k of the pass and column t % k
    {
        const uint64_t tau = sm.tau;
        const int rpp = kAddrGroup / k;
        const int li = t / k, lj = t - li * k;
        const bool t_ok = li < rpp;
        const float sb = sm.hsc[1][t_ok ? lj : 0];
        const uint32_t ib = (uint32_t)sm.hix[1][t_ok ? lj : 0];
        int cnt = 0;
        for (int i0 = 0; i0 < k; i0 += rpp) {
            const int i = i0 + li;
            const bool in = t_ok && i < k;
            const int ic = in ? i : 0;
            const float sum = sm.hsc[0][ic] + sb;  // one fp32 RNE add
            const bool ge = in && make_key(sum, (uint32_t)sm.hix[0][ic] * (uint32_t)n + ib) >= tau;
            cnt += __popcll(__ballot(ge));
        }
        if (lane == 0) sm.Fw[wv] = cnt;
    }
    block_sync_lds();
    if (wv == 0) {
        const int F = sm.Fw[0] + sm.Fw[1] + sm.Fw[2] + sm.Fw[3];
        if (F == budget) {
            // 4. softmax over the selected fp32 scores (rank 0 holds the maximum)
            const float smax = key_score(shfl_u64(key, 0));
            const float w = lane < budget ? __expf(key_score(key) - smax) : 0.f;
            const float z = wave_sum(w);
            if (lane < budget) {
                const int32_t slot = (int32_t)key_index(key);
                if (idx) idx[lane] = slot;
                if (wt) wt[lane] = w / z;
                if (idx2) idx2[lane] = slot;
                if (wt2) wt2[lane] = w / z;
            }
        }
        if (lane == 0) sm.F = F;
    }
    block_sync_lds();
}

// the rare path: rank all k^2 candidates (three barriers)
template <typename Sm>
SSLP_DEVICE void wg_addr_rank_all(const WgAddrProblem& pr, int t, Sm& sm) {
    const int n = pr.n, k = pr.k, budget = pr.budget, kk = k * k;
    block_sync_lds();
    for (int x = t; x < kk; x += kAddrGroup) {
        const int i = x / k, j = x - (x / k) * k;
        const float sum = sm.hsc[0][i] + sm.hsc[1][j];
        sm.cand[x] = make_key(sum, (uint32_t)sm.hix[0][i] * (uint32_t)n + (uint32_t)sm.hix[1][j]);
    }
    block_sync_lds();
    for (int x = t; x < kk; x += kAddrGroup) {
        const uint64_t kx = sm.cand[x];
        int r = 0;
        for (int y = 0; y < kk; ++y) r += sm.cand[y] > kx;
        if (r < budget) sm.sel[r] = kx;
    }
    block_sync_lds();
}

// 4. softmax over the selected scores (rank 0 holds the maximum), by the
// group's first wavefront; either output pair may be null
template <typename Sm>
SSLP_DEVICE void wg_addr_softmax(const WgAddrProblem& pr, int t, const Sm& sm,
                                 int32_t* idx, float* wt, int32_t* idx2, float* wt2) {
    if (t < 64) {
        const int budget = pr.budget;
        const float smax = key_score(sm.sel[0]);
        const float w = t < budget ? __expf(key_score(sm.sel[t]) - smax) : 0.f;
        const float z = wave_sum(w);
        if (t < budget) {
            const int32_t slot = (int32_t)key_index(sm.sel[t]);
            if (idx) idx[t] = slot;
            if (wt) wt[t] = w / z;
            if (idx2) idx2[t] = slot;
            if (wt2) wt2[t] = w / z;
        }
    }
}

}  // namespace sslp
