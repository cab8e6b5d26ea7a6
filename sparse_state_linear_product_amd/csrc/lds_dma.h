// LDS and LDS-DMA helpers of the kernels that stage memory through LDS with
// global_load_lds (the chunk-parallel SDM kernels, the GDN state kernel):
// the DMA issue, explicit vector-memory waits, and LDS reads written as inline
// assembly so that the compiler neither waits for the DMAs in flight before
// them nor moves their results' first use above an explicit wait.
#pragma once
#include <type_traits>
#include <utility>

#include "common.h"

namespace sslp {
namespace lds {

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

}  // namespace lds
}  // namespace sslp
