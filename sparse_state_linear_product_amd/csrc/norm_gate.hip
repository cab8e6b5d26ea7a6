// The layer output after the SDM read: RMS-Norm and output gate in one pass.
//
// Sparse Delta Memory slides, "Selected slots decay and update; other slots
// persist": the read y_t is followed by RMS-Norm, output gating and head
// mixing.  Per (token, head) row of d values, with gamma [d] a per-channel
// weight shared by the heads and g the gate pre-activation of the row:
//   o = y / sqrt(mean(y^2) + eps) * gamma * act(g),
//   act = SiLU (g * sigmoid(g)), the logistic sigmoid, or none.
// Head mixing is the dense output projection that follows; it is a plain
// GEMM outside this step.
//
// One wavefront per row: each lane holds up to 16 groups of 4 consecutive
// columns (d <= 4096) of y and of the gate in registers, all requested at
// once, so y and g are read once and o written once; the sum of squares is a
// wavefront reduction.  HBM-bound: 3 d values of
// the I/O type per row.
#include "common.h"
#include "kernels.h"

namespace sslp {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxGroups = 16;  // 16 groups of 4 columns per lane: d <= 4096

SSLP_DEVICE float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
SSLP_DEVICE float4 load4(const bf16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}
SSLP_DEVICE void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
SSLP_DEVICE void store4(bf16_t* p, float4 v) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16(v.x).bits | ((uint32_t)f32_to_bf16(v.y).bits << 16);
    u.y = (uint32_t)f32_to_bf16(v.z).bits | ((uint32_t)f32_to_bf16(v.w).bits << 16);
    *reinterpret_cast<uint2*>(p) = u;
}

// The logistic factor 1 / (1 + e^-x) with the hardware exponential and
// reciprocal (a few ulp in fp32, not an IEEE division): the kernel was bound by
// the per-element division sequence, not by memory.
template <int ACT>
SSLP_DEVICE float gate_fn(float x) {
    if constexpr (ACT == 1) return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
    else if constexpr (ACT == 2) return __builtin_amdgcn_rcpf(1.f + __expf(-x));
    else return 1.f;
}

// MG: groups of 4 columns per lane the instantiation holds (d <= 256 MG)
template <typename io_t, int ACT, int MG>
__global__ __launch_bounds__(64 * kWaves) void norm_gate_kernel(long long rows, int d,
                                                                const io_t* y,
                                                                const io_t* __restrict__ g,
                                                                const float* __restrict__ gamma,
                                                                float eps, io_t* o) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const io_t* yr = y + (size_t)row * d;
    const int ng = d / 4;  // groups of 4 columns
    float4 yv[MG], gv[MG];
    float ss = 0.f;
    // y and the gate are both requested before the reduction waits on y
#pragma unroll
    for (int j = 0; j < MG; ++j) {
        const int grp = lane + 64 * j;
        const bool in = grp < ng;
        yv[j] = in ? load4(yr + 4 * grp) : make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (ACT != 0)
            gv[j] = in ? load4(g + (size_t)row * d + 4 * grp) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < MG; ++j) {
        ss = fmaf(yv[j].x, yv[j].x, ss);
        ss = fmaf(yv[j].y, yv[j].y, ss);
        ss = fmaf(yv[j].z, yv[j].z, ss);
        ss = fmaf(yv[j].w, yv[j].w, ss);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) ss += __shfl_xor(ss, s, 64);
    const float inv = 1.f / __fsqrt_rn(ss / (float)d + eps);
    io_t* orow = o + (size_t)row * d;
#pragma unroll
    for (int j = 0; j < MG; ++j) {
        const int grp = lane + 64 * j;
        if (grp < ng) {
            const float4 w = load4(gamma + 4 * grp);
            float4 f = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (ACT != 0)
                f = make_float4(gate_fn<ACT>(gv[j].x), gate_fn<ACT>(gv[j].y),
                                gate_fn<ACT>(gv[j].z), gate_fn<ACT>(gv[j].w));
            store4(orow + 4 * grp, make_float4(yv[j].x * inv * w.x * f.x, yv[j].y * inv * w.y * f.y,
                                               yv[j].z * inv * w.z * f.z,
                                               yv[j].w * inv * w.w * f.w));
        }
    }
}

template <typename io_t, int MG>
hipError_t dispatch_act(int act, unsigned grid, long long rows, int d, const void* y,
                        const void* g, const float* gamma, float eps, void* o, hipStream_t st) {
    const io_t* yy = static_cast<const io_t*>(y);
    const io_t* gg = static_cast<const io_t*>(g);
    io_t* oo = static_cast<io_t*>(o);
    const dim3 blk(64 * kWaves);
    switch (act) {
        case 0: norm_gate_kernel<io_t, 0, MG><<<grid, blk, 0, st>>>(rows, d, yy, gg, gamma, eps, oo); break;
        case 1: norm_gate_kernel<io_t, 1, MG><<<grid, blk, 0, st>>>(rows, d, yy, gg, gamma, eps, oo); break;
        case 2: norm_gate_kernel<io_t, 2, MG><<<grid, blk, 0, st>>>(rows, d, yy, gg, gamma, eps, oo); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename io_t>
hipError_t dispatch_width(int act, unsigned grid, long long rows, int d, const void* y,
                          const void* g, const float* gamma, float eps, void* o, hipStream_t st) {
    if (d <= 256 * 4) return dispatch_act<io_t, 4>(act, grid, rows, d, y, g, gamma, eps, o, st);
    return dispatch_act<io_t, kMaxGroups>(act, grid, rows, d, y, g, gamma, eps, o, st);
}

}  // namespace

hipError_t launch_norm_gate(long long rows, int d, int dtype, const void* y, const void* g,
                            const float* gamma, float eps, int act, void* o, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (d < 4 || d % 4 != 0 || d > 4 * 64 * kMaxGroups) return hipErrorInvalidValue;
    const long long nblk = (rows + kWaves - 1) / kWaves;
    if (nblk > 0x7fffffffll) return hipErrorInvalidValue;
    if (dtype == 0) return dispatch_width<float>(act, (unsigned)nblk, rows, d, y, g, gamma, eps, o, st);
    return dispatch_width<bf16_t>(act, (unsigned)nblk, rows, d, y, g, gamma, eps, o, st);
}

}  // namespace sslp
