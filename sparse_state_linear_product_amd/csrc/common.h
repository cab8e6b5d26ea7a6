// Device and host helpers shared by the libsslp HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SSLP_DEVICE __device__ __forceinline__

namespace sslp {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// element types: fp32 or bf16 (stored as raw uint16 bits)
// ---------------------------------------------------------------------------
struct bf16_t {
    uint16_t bits;
};

SSLP_DEVICE float to_f32(float x) { return x; }
SSLP_DEVICE float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x.bits) << 16); }

// round-to-nearest-even fp32 -> bf16 (the gfx950 conversion instruction)
SSLP_DEVICE bf16_t f32_to_bf16(float f) {
    bf16_t r;
    r.bits = __builtin_bit_cast(uint16_t, (__bf16)f);
    return r;
}
template <typename T>
SSLP_DEVICE T from_f32(float f);
template <>
SSLP_DEVICE float from_f32<float>(float f) { return f; }
template <>
SSLP_DEVICE bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }

// ---------------------------------------------------------------------------
// ranking keys: a 64-bit unsigned key whose integer order is the rank order
// "score descending, then index ascending", so that a descending sort of keys
// is the ranking.  -0 is folded onto +0 so that the two tie.
// ---------------------------------------------------------------------------
SSLP_DEVICE uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
SSLP_DEVICE float order_bits_to_float(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}
SSLP_DEVICE uint64_t make_key(float score, uint32_t index) {
    return ((uint64_t)order_bits(score) << 32) | (uint64_t)(~index);
}
SSLP_DEVICE float key_score(uint64_t key) { return order_bits_to_float((uint32_t)(key >> 32)); }
SSLP_DEVICE uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

// The same order in 32 bits for a score that is exactly a bf16 value and an
// index below 2^16: the upper half of the order bits (the lower half is 0x0000
// for a positive and 0xFFFF for a negative bf16 value) and the inverted index.
SSLP_DEVICE uint32_t make_key32(float bf16_exact_score, uint32_t index) {
    return (order_bits(bf16_exact_score) & 0xFFFF0000u) | (~index & 0xFFFFu);
}
SSLP_DEVICE float key32_score(uint32_t key) {
    const uint32_t hi = key & 0xFFFF0000u;
    return order_bits_to_float(hi | ((hi & 0x80000000u) ? 0u : 0xFFFFu));
}
SSLP_DEVICE uint32_t key32_index(uint32_t key) { return ~key & 0xFFFFu; }

// ---------------------------------------------------------------------------
// wave-level helpers
// ---------------------------------------------------------------------------
SSLP_DEVICE int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// The value of x held by lane ^ j (j a power of two below 64; a constant once
// the callers' loops are unrolled), from DPP row moves (j <= 8) or the gfx950
// lane-swap instructions (j = 16, 32) instead of a round trip through the LDS
// crossbar.  Every lane of the wavefront must be active.
SSLP_DEVICE uint32_t xor_lane(uint32_t x, int j, int lane) {
    const int xi = (int)x;
    switch (j) {
        case 1:  // quad_perm [1,0,3,2]
            return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false);
        case 2:  // quad_perm [2,3,0,1]
            return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false);
        case 4: {  // rotations inside a row of 16: by 12 reads lane + 4, by 4 reads lane - 4
            const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x12C, 0xF, 0xF, false);
            const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x124, 0xF, 0xF, false);
            return (lane & 4) ? dn : up;
        }
        case 8:  // row rotation by 8
            return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, false);
        case 16: {  // element 1 holds row r+1's values in even rows, element 0 row r-1's in odd rows
            const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
            return (lane & 16) ? p[0] : p[1];
        }
        default: {  // 32: the same for the two halves of the wavefront
            const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
            return (lane & 32) ? p[0] : p[1];
        }
    }
}
SSLP_DEVICE uint64_t xor_lane_u64(uint64_t v, int j, int lane) {
    const uint32_t lo = xor_lane((uint32_t)v, j, lane), hi = xor_lane((uint32_t)(v >> 32), j, lane);
    return ((uint64_t)hi << 32) | lo;
}
SSLP_DEVICE uint64_t shfl_xor_u64(uint64_t v, int mask) { return xor_lane_u64(v, mask, lane_id()); }
SSLP_DEVICE float xor_lane_f(float x, int j, int lane) {
    return __uint_as_float(xor_lane(__float_as_uint(x), j, lane));
}
SSLP_DEVICE int xor_lane_i(int x, int j, int lane) { return (int)xor_lane((uint32_t)x, j, lane); }
SSLP_DEVICE uint64_t shfl_u64(uint64_t v, int src) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl(lo, src, kWave);
    hi = __shfl(hi, src, kWave);
    return ((uint64_t)hi << 32) | lo;
}
SSLP_DEVICE float wave_sum(float x) {
    const int lane = lane_id();
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __uint_as_float(xor_lane(__float_as_uint(x), m, lane));
    return x;
}
SSLP_DEVICE uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = shfl_xor_u64(x, m);
        x = o > x ? o : x;
    }
    return x;
}

// Orders LDS/global accesses of one wavefront: a compiler barrier plus
// wavefront-scope release/acquire (the hardware keeps a wave's memory
// operations in order, so no wait instruction is needed).
// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// operations, then meets the others.  Unlike __syncthreads(), whose fence also
// waits for every outstanding global load and store, it lets loads issued
// ahead of time (register or LDS-DMA prefetch) stay in flight across it.  Any
// wait for global memory a barrier must cover is written out before it.
// A caller-supplied slot index, kept inside the table: an index outside
// [0, N) becomes slot 0 and sets *err (when given) to 1, so that no access
// leaves the table whatever the input; the call's results are then undefined.
// The check has no branch and no memory access: a branch on a prefetched index
// would make the wavefront wait for that load where the branch stands.  The
// caller accumulates `bad` and reports it once, at its end, with
// report_slot_error.
SSLP_DEVICE int keep_slot(int slot, long long N, bool& bad) {
    const bool ok = (unsigned long long)(unsigned)slot < (unsigned long long)N;
    bad |= !ok;
    return ok ? slot : 0;
}
SSLP_DEVICE void report_slot_error(bool bad, unsigned* err) {
    if (bad && err != nullptr) atomicOr(err, 1u);
}

SSLP_DEVICE void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

SSLP_DEVICE void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// xor_lane with the distance as a template argument
template <int J>
SSLP_DEVICE uint32_t xor_lane_c(uint32_t x, int lane) {
    static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "lane distance");
    const int xi = (int)x;
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false);
    } else if constexpr (J == 4) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x12C, 0xF, 0xF, false);
        const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x124, 0xF, 0xF, false);
        return (lane & 4) ? dn : up;
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, false);
    } else if constexpr (J == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? p[0] : p[1];
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? p[0] : p[1];
    }
}
template <int J>
SSLP_DEVICE uint64_t xor_lane_c(uint64_t v, int lane) {
    const uint32_t lo = xor_lane_c<J>((uint32_t)v, lane), hi = xor_lane_c<J>((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort, descending, of 64*E keys (uint64_t, or uint32_t for the
// 32-bit order of bf16 scores) held E per lane: element e of lane l sits at
// position p = e*64 + l.  Compare-exchange partners at distance J < 64 live in
// another lane (exchanged with xor_lane_c); larger distances are inside the
// lane.  The merge size KK and distance J are template arguments, so every
// stage is resolved at compile time.
template <int KK, int J, int E, typename Key>
SSLP_DEVICE void bitonic_stage(Key (&a)[E], int lane) {
    if constexpr (J >= 64) {
        constexpr int je = J >> 6;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int e2 = e ^ je;
            if (e2 > e) {
                const bool desc = (((e << 6) & KK) == 0);
                const Key x = a[e], y = a[e2];
                const bool sw = desc ? (x < y) : (x > y);
                a[e] = sw ? y : x;
                a[e2] = sw ? x : y;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const Key mine = a[e];
            const Key other = xor_lane_c<J>(mine, lane);
            const int p = (e << 6) | lane;
            const bool desc = ((p & KK) == 0);
            const bool lower = ((lane & J) == 0);
            const bool keep_max = (lower == desc);
            // one compare and one select (equal keys: either is the same value)
            a[e] = ((mine > other) == keep_max) ? mine : other;
        }
    }
}
template <int KK, int J, int E, typename Key>
SSLP_DEVICE void bitonic_stages(Key (&a)[E], int lane) {  // distances J, J/2, ..., 1 of merge KK
    bitonic_stage<KK, J>(a, lane);
    if constexpr (J > 1) bitonic_stages<KK, J / 2>(a, lane);
}
template <int KK, int N, int E, typename Key>
SSLP_DEVICE void bitonic_merges(Key (&a)[E], int lane) {  // merges of size KK, 2 KK, ..., N
    bitonic_stages<KK, KK / 2>(a, lane);
    if constexpr (KK < N) bitonic_merges<KK * 2, N>(a, lane);
}
template <int E>
SSLP_DEVICE void bitonic_sort_desc(uint64_t (&a)[E], int lane) {
    bitonic_merges<2, 64 * E>(a, lane);
}
// The same sort for 32-bit keys (one lane exchange per step instead of two).
template <int E>
SSLP_DEVICE void bitonic_sort_desc32(uint32_t (&a)[E], int lane) {
    bitonic_merges<2, 64 * E>(a, lane);
}

// One compare-exchange step at lane distance J < 64 on registers 0..R-1, each
// register's direction given by desc_of(e) (true: the larger key to the lower
// lane of each pair).
template <int J, int R, int E, typename Key, typename Desc>
SSLP_DEVICE void cx_stage_dir(Key (&a)[E], int lane, Desc desc_of) {
#pragma unroll
    for (int e = 0; e < R; ++e) {
        const Key mine = a[e];
        const Key other = xor_lane_c<J>(mine, lane);
        const bool keep_max = (((lane & J) == 0) == desc_of(e));
        a[e] = ((mine > other) == keep_max) ? mine : other;
    }
}
// Sorts the bitonic runs of 2J lanes in registers 0..R-1 (distances J, ..., 1).
template <int J, int R, int E, typename Key, typename Desc>
SSLP_DEVICE void merge_runs(Key (&a)[E], int lane, Desc desc_of) {
    cx_stage_dir<J, R>(a, lane, desc_of);
    if constexpr (J > 1) merge_runs<J / 2, R>(a, lane, desc_of);
}
// Registers 0..M-1 hold sorted runs of KC keys, register e descending when e
// is even and ascending when odd: pairs of registers are pruned to the KC
// largest keys of each run pair until one register remains, whose runs are
// left descending in lanes 0..31 and ascending in lanes 32..63 (KC = 32) or
// descending (KC = 64).
template <int KC, int M, int E, typename Key>
SSLP_DEVICE void topk_prune(Key (&a)[E], int lane) {
    if constexpr (M > 1) {
#pragma unroll
        for (int r = 0; r < M / 2; ++r) a[r] = a[2 * r] > a[2 * r + 1] ? a[2 * r] : a[2 * r + 1];
        if constexpr (M / 2 > 1) {
            merge_runs<KC / 2, M / 2>(a, lane, [](int e) { return (e & 1) == 0; });
        } else {
            merge_runs<KC / 2, 1>(a, lane, [lane](int) { return KC == 64 || (lane & 32) == 0; });
        }
        topk_prune<KC, M / 2>(a, lane);
    }
}
// The KC largest (KC = 32 or 64) of 64*E keys, sorted descending into lanes
// 0..KC-1 of a[0]; the rest of a[] is left holding keys of no meaning.  Runs of
// KC keys are sorted as in the full sort, then registers are pruned in pairs:
// with run A descending and run B ascending, the lane-wise max(A_l, B_l) holds
// the KC largest keys of A and B as a bitonic sequence (the upper half of the
// first compare-exchange of a bitonic merge), which log2(KC) more steps sort.
// For E = 4 and KC = 32 that is 81 register-steps against the full sort's 132.
template <int KC, int E, typename Key>
SSLP_DEVICE void bitonic_topk_desc(Key (&a)[E], int lane) {
    static_assert(KC == 32 || KC == 64, "run length");
    bitonic_merges<2, KC / 2>(a, lane);  // runs of KC/2, alternating in direction
    merge_runs<KC / 2, E>(a, lane, [lane](int e) {
        return E > 1 ? (e & 1) == 0 : (KC == 64 || (lane & 32) == 0);
    });
    topk_prune<KC, E>(a, lane);
    if constexpr (KC == 32) {  // the two halves of a[0] pruned into one run, then sorted
        const Key other = xor_lane_c<32>(a[0], lane);
        a[0] = a[0] > other ? a[0] : other;
        merge_runs<16, 1>(a, lane, [](int) { return true; });
    }
}

// element at runtime position p (p = e*64 + lane) of a register-held array,
// broadcast to the whole wave
template <int E>
SSLP_DEVICE uint64_t wave_get(const uint64_t (&a)[E], int p) {
    const int e = p >> 6, l = p & 63;
    uint64_t v = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) v = (i == e) ? a[i] : v;
    return shfl_u64(v, l);
}

}  // namespace sslp
