// Shared pieces of the chunk-parallel SDM recurrence (sdm_chunk.hip: forward,
// sdm_chunk_bwd.hip: backward): the chunk geometry and plan layout, and the
// LDS / LDS-DMA helpers of the apply kernels.
#pragma once
#include <type_traits>
#include <utility>

#include "common.h"

namespace sslp {
namespace chunk {

constexpr int CW = 8;                // columns per apply workgroup (one 32-byte row piece)
constexpr int NWAVE = 8;             // wavefronts per apply workgroup
constexpr int NE = 512;              // write entries per chunk (C x W)
constexpr int JW = 32 / NWAVE;       // row DMAs per wavefront and chunk (32 per chunk)

// plan block of one (b, h, chunk), 32-bit words: a fixed part (layout below),
// then a tail of exception records, extra pairs and forward rows.  The fixed
// part and the first PL_TAILWIN words of the tail are staged in LDS; tail words
// past that (only with heavy slot reuse) are read from memory.
constexpr int PL_TAIL = 4096;
constexpr int PL_TAILWIN = 2048;
constexpr int PL_DMA_WORDS = PL_TAIL + PL_TAILWIN;  // 24 KB staged per chunk
constexpr int PL_WORDS = PL_TAIL + 2 * NE + 3 * NE + 2 * NE;  // worst-case tail
static_assert((PL_DMA_WORDS * 4) % 1024 == 0 && (PL_WORDS * 4) % 16 == 0, "plan DMA pieces");
// exception record: (first, packed); packed = extra index (9 bits) | extra count << 9
// (5 bits) | forward index << 14 (10 bits) | forward count << 24 (6 bits).
// extra record (one per earlier visit of a slot, in visit order): (token | row << 8,
// decay d of the visit, beta w of the visit)

// Chunk geometry: CC_ tokens per chunk, NW_ write rows and as many read rows
// per token.  Both configurations (16 x 32 and 8 x 64) have 512 write entries
// and 1024 staged rows per chunk, so the LDS budgets, the plan's size and the
// DMA pattern (32 DMAs of 32 rows of 32 bytes) are shared; only the index maps
// differ.  Rows of the fixed plan part are padded so that the apply kernel's
// LDS reads of them are free of bank conflicts.
template <int CC_, int NW_>
struct Geo {
    static constexpr int CC = CC_;         // tokens per chunk
    static constexpr int NW = NW_;         // write rows per token
    static constexpr int NR = NW_;         // read rows per token
    static constexpr int NQ = NW + NR;     // rows per token
    static constexpr int LOGNW = NW == 32 ? 5 : 6;
    static constexpr int RPD = 32 / CC;    // row indices q per DMA
    static constexpr int NMW = NW / 32;    // mask words per token
    static constexpr int OFFS_LD = 36, COEF_LD = NQ + 4, TB_LD = CC + 4;
    static constexpr int PL_OFFS = 0;                          // row byte offsets (see offs_word)
    static constexpr int PL_COEF = PL_OFFS + 32 * OFFS_LD;     // [t][q]: c (q < NW) or e (q >= NW)
    static constexpr int PL_TM = PL_COEF + CC * COEF_LD;       // [t][tau]: (I + A)^-1
    static constexpr int PL_BM = PL_TM + CC * TB_LD;           // [t][tau]
    static constexpr int PL_FIN = PL_BM + CC * TB_LD;          // [i][t][2]: decay d, beta w of write entry (t, i)
    static constexpr int PL_LAST = PL_FIN + NE * 2;            // [t][NMW] bit i: entry (t, i) is its slot's last visit
    static constexpr int PL_FIRST = PL_LAST + CC * NMW;        // [t][NMW] bit i: entry (t, i) is its slot's first visit
    static constexpr int PL_EXC = PL_FIRST + CC * NMW;         // [t][NMW] bit i: entry (t, i) has an exception record
    static constexpr int PL_EXCB = PL_EXC + CC * NMW;          // [t] index of token t's first exception record
    static constexpr int PL_HDR = PL_EXCB + CC;                // tail offsets of the extra pairs and forward rows
    static_assert(CC * NW == NE && CC * NQ == 2 * NE && 32 % CC == 0 && NW % 32 == 0, "chunk geometry");
    static_assert(PL_HDR + 4 <= PL_TAIL, "plan layout");
    static_assert(PL_COEF % 4 == 0 && COEF_LD % 4 == 0 && PL_TM % 4 == 0 && PL_BM % 4 == 0 &&
                      TB_LD % 4 == 0 && PL_FIN % 2 == 0 && PL_LAST % 2 == 0 && PL_HDR % 4 == 0,
                  "aligned vector reads of the plan");
    // row (q, t) is staged by DMA j = q / RPD of wave j % NWAVE, as row
    // (q % RPD) C + t of that DMA's 32; a lane's JW offsets for its wave are
    // contiguous
    static SSLP_DEVICE int offs_word(int q, int t) {
        const int j = q / RPD;
        return PL_OFFS + ((q % RPD) * CC + t) * OFFS_LD + (j % NWAVE) * JW + j / NWAVE;
    }
    static SSLP_DEVICE int coef_word(int t, int q) { return PL_COEF + t * COEF_LD + q; }
};
using GeoW32 = Geo<16, 32>;
using GeoW64 = Geo<8, 64>;

// ---------------------------------------------------------------------------
// apply kernel helpers
// ---------------------------------------------------------------------------
typedef void __attribute__((address_space(3))) * lds_ptr_t;
typedef float __attribute__((address_space(3))) * lds_f32_ptr_t;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

SSLP_DEVICE void dma16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 16, 0, 0);
}
SSLP_DEVICE void dma4(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 4, 0, 0);
}
SSLP_DEVICE void wait_vm0() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
    __builtin_amdgcn_sched_barrier(0);
}
SSLP_DEVICE uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_f32_ptr_t)p; }

// LDS reads of DMA'd data are issued as inline asm: the compiler cannot tell
// them from reads that alias an LDS-DMA in flight and would drain the vector
// memory queue before each.  Their results are tied to an explicit wait
// (lds_wait) placed before first use; "memory" keeps program order.  OFF is a
// byte offset folded into the instruction.
template <int OFF = 0>
SSLP_DEVICE uint32_t lds_u32(uint32_t a) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF) : "memory");
    return v;
}
template <int OFF = 0>
SSLP_DEVICE float lds_f32(uint32_t a) {
    return __uint_as_float(lds_u32<OFF>(a));
}
template <int OFF = 0>
SSLP_DEVICE f32x2 lds_f32x2(uint32_t a) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    f32x2 v;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF) : "memory");
    return v;
}
template <int OFF = 0>
SSLP_DEVICE f32x4 lds_f32x4(uint32_t a) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    f32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF) : "memory");
    return v;
}
template <int OFF = 0>
SSLP_DEVICE u32x4 lds_u32x4(uint32_t a) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF) : "memory");
    return v;
}
SSLP_DEVICE uint32_t lds_u16(uint32_t a) {
    uint32_t v;
    asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(a) : "memory");
    return v;
}
// reads of N consecutive floats (N = 1, 2, 4) as one value
template <int N>
struct VecOf;
template <>
struct VecOf<1> {
    using type = float;
};
template <>
struct VecOf<2> {
    using type = f32x2;
};
template <>
struct VecOf<4> {
    using type = f32x4;
};
template <int N, int OFF = 0>
SSLP_DEVICE typename VecOf<N>::type lds_vec(uint32_t a) {
    if constexpr (N == 1) return lds_f32<OFF>(a);
    else if constexpr (N == 2) return lds_f32x2<OFF>(a);
    else return lds_f32x4<OFF>(a);
}
SSLP_DEVICE float elem(float v, int) { return v; }
SSLP_DEVICE float elem(f32x2 v, int i) { return v[i]; }
SSLP_DEVICE float elem(f32x4 v, int i) { return v[i]; }
SSLP_DEVICE void lds_write_f32(uint32_t a, float v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}
SSLP_DEVICE void lds_write_f32x2(uint32_t a, f32x2 v) {
    asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
}
SSLP_DEVICE void lds_write_f32x4(uint32_t a, f32x4 v) {
    asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(v) : "memory");
}
template <int N>
SSLP_DEVICE void lds_write_cols(uint32_t a, const float (&x)[N]) {
    if constexpr (N == 1) lds_write_f32(a, x[0]);
    else lds_write_f32x2(a, f32x2{x[0], x[1]});
}
// wait for all LDS operations; each operand then passes through an empty
// volatile asm ordered after the wait, so that no use of it is scheduled before
template <typename X>
SSLP_DEVICE void tie(X& x) {
    asm volatile("" : "+v"(x));
}
template <typename... V>
SSLP_DEVICE void lds_wait(V&... v) {
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    (tie(v), ...);
}
template <typename X, int N>
SSLP_DEVICE void tie_all(X (&x)[N]) {
#pragma unroll
    for (int k = 0; k < N; ++k) tie(x[k]);
}

SSLP_DEVICE float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
SSLP_DEVICE float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// compile-time loops that pass the index as a template argument
template <int N, typename F, int... I>
SSLP_DEVICE void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
SSLP_DEVICE void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

}  // namespace chunk
}  // namespace sslp
