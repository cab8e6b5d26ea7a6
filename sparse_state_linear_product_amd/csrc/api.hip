// C ABI of libsslp.so (declared in include/sslp.h): argument validation on the
// host, workspace carving, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/sslp.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return SSLP_OK;
    return fail(SSLP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

#define REQUIRE(cond, code, ...)                      \
    do {                                              \
        if (!(cond)) return fail((code), __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p)                                                                    \
    do {                                                                                  \
        REQUIRE((p) != nullptr, SSLP_ERR_INVALID_ARG, "%s must not be NULL", #p);        \
        REQUIRE(aligned16(p), SSLP_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p);   \
    } while (0)

#define REQUIRE_ALIGNED(p) \
    REQUIRE(aligned16(p), SSLP_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p)

constexpr int kMaxSqrtN = 1024;
constexpr int kMaxTopK = 64;
constexpr int kMaxBudget = 128;
constexpr int kMaxDv = 4096;

// Device word that the SDM recurrence kernels set to 1 when a caller-supplied
// slot index lies outside [0, N) (sslp_device_error reads and clears it).  In
// host code the name is a host-side stand-in; kernels get the device address
// of each GPU's copy, taken once per device.
__device__ unsigned int device_error_word;

constexpr int kMaxErrDevices = 64;
std::mutex g_errword_mu;
unsigned* g_errword_ptr[kMaxErrDevices] = {};

// device address of the error word on the current device (nullptr on failure:
// the kernels then skip the report but still keep every access in the table)
unsigned* error_word() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxErrDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_errword_mu);
    if (g_errword_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(device_error_word)) != hipSuccess) return nullptr;
        g_errword_ptr[dev] = static_cast<unsigned*>(p);
    }
    return g_errword_ptr[dev];
}

// checks shared by every SDM entry point; `need_k` checks k_w/k_r and W<=k^2
int check_sdm_shape(const sslp_sdm_shape* s, bool need_k) {
    REQUIRE(s != nullptr, SSLP_ERR_INVALID_ARG, "shape must not be NULL");
    REQUIRE(s->B >= 1 && s->H >= 1 && s->T >= 0, SSLP_ERR_INVALID_ARG,
            "B, H must be >= 1 and T >= 0 (B=%d T=%d H=%d)", s->B, s->T, s->H);
    REQUIRE(s->sqrtN >= 1, SSLP_ERR_INVALID_ARG, "sqrtN must be >= 1 (got %d)", s->sqrtN);
    REQUIRE(s->sqrtN <= kMaxSqrtN, SSLP_ERR_UNSUPPORTED, "sqrtN %d > %d", s->sqrtN, kMaxSqrtN);
    REQUIRE(s->d_v >= 1, SSLP_ERR_INVALID_ARG, "d_v must be >= 1 (got %d)", s->d_v);
    REQUIRE(s->d_v % 4 == 0 && s->d_v <= kMaxDv, SSLP_ERR_UNSUPPORTED,
            "d_v must be a multiple of 4 and <= %d (got %d)", kMaxDv, s->d_v);
    REQUIRE(s->W >= 1 && s->R >= 1, SSLP_ERR_INVALID_ARG, "W, R must be >= 1 (W=%d R=%d)", s->W,
            s->R);
    REQUIRE(s->W <= kMaxBudget && s->R <= kMaxBudget, SSLP_ERR_UNSUPPORTED,
            "W, R must be <= %d (W=%d R=%d)", kMaxBudget, s->W, s->R);
    const long long N = (long long)s->sqrtN * s->sqrtN;
    REQUIRE(s->W <= N && s->R <= N, SSLP_ERR_INVALID_ARG, "W, R must be <= N=%lld", N);
    if (need_k) {
        REQUIRE(s->k_w >= 1 && s->k_r >= 1, SSLP_ERR_INVALID_ARG, "k_w, k_r must be >= 1");
        REQUIRE(s->k_w <= s->sqrtN && s->k_r <= s->sqrtN, SSLP_ERR_INVALID_ARG,
                "k_w, k_r must be <= sqrtN (k_w=%d k_r=%d sqrtN=%d)", s->k_w, s->k_r, s->sqrtN);
        REQUIRE(s->k_w <= kMaxTopK && s->k_r <= kMaxTopK, SSLP_ERR_UNSUPPORTED,
                "k_w, k_r must be <= %d", kMaxTopK);
        REQUIRE(s->W <= s->k_w * s->k_w, SSLP_ERR_INVALID_ARG, "W=%d > k_w^2=%d", s->W,
                s->k_w * s->k_w);
        REQUIRE(s->R <= s->k_r * s->k_r, SSLP_ERR_INVALID_ARG, "R=%d > k_r^2=%d", s->R,
                s->k_r * s->k_r);
    }
    return SSLP_OK;
}

int check_dtype(int dtype) {
    REQUIRE(dtype == SSLP_FP32 || dtype == SSLP_BF16, SSLP_ERR_INVALID_ARG,
            "dtype must be SSLP_FP32 or SSLP_BF16 (got %d)", dtype);
    return SSLP_OK;
}

size_t addressing_bytes(const sslp_sdm_shape* s, int T) {
    const size_t bth = (size_t)s->B * T * s->H;
    return align_up(bth * s->W * 4) * 2 + align_up(bth * s->R * 4) * 2;
}

long long slots(const sslp_sdm_shape* s) { return (long long)s->sqrtN * s->sqrtN; }

// bytes the recurrence itself needs (the chunk plans of the chunk-parallel kernel)
size_t recurrence_bytes(const sslp_sdm_shape* s, int T) {
    if (!sslp::sdm_chunked_supported(s->B, T, s->H, s->W, s->R, s->d_v, slots(s))) return 0;
    return align_up(sslp::sdm_chunk_plan_bytes(s->B, T, s->H, s->W));
}

hipError_t run_recurrence(const sslp::SdmUpdateArgs& a, const sslp_sdm_shape* s, void* plan,
                          hipStream_t st) {
    if (sslp::sdm_chunked_supported(a.B, a.T, a.H, s->W, s->R, s->d_v, slots(s)))
        return sslp::launch_sdm_update_chunked(a, plan, st);
    return sslp::launch_sdm_update(a, st);
}

}  // namespace

extern "C" {

const char* sslp_last_error(void) { return g_err; }
int sslp_version(void) { return SSLP_VERSION; }

int sslp_device_error(void* stream) {
    g_err[0] = 0;
    unsigned* w = error_word();
    REQUIRE(w != nullptr, SSLP_ERR_HIP, "device error word not available on this device");
    hipStream_t st = (hipStream_t)stream;
    unsigned host = 0u;
    if (int rc = hip_status(hipMemcpyAsync(&host, w, sizeof(host), hipMemcpyDeviceToHost, st),
                            "read the device error word"))
        return rc;
    if (int rc = hip_status(hipStreamSynchronize(st), "hipStreamSynchronize")) return rc;
    if (host != 0u) {
        if (int rc = hip_status(hipMemsetAsync(w, 0, sizeof(unsigned), st), "clear the word"))
            return rc;
        if (int rc = hip_status(hipStreamSynchronize(st), "hipStreamSynchronize")) return rc;
    }
    return host != 0u ? 1 : 0;
}

size_t sdm_workspace_size(const sslp_sdm_shape* s) {
    if (check_sdm_shape(s, false) != SSLP_OK) return 0;
    return addressing_bytes(s, s->T) + recurrence_bytes(s, s->T);
}

size_t sdm_decode_workspace_size(const sslp_sdm_shape* s) {
    if (check_sdm_shape(s, false) != SSLP_OK) return 0;
    return addressing_bytes(s, 1) + recurrence_bytes(s, 1);
}

int sdm_address(const sslp_sdm_shape* s, int dtype, const void* s1, const void* s2, int k,
                int budget, int32_t* idx, float* wt, void* stream) {
    g_err[0] = 0;
    REQUIRE(s != nullptr, SSLP_ERR_INVALID_ARG, "shape must not be NULL");
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(s->B >= 1 && s->H >= 1 && s->T >= 0, SSLP_ERR_INVALID_ARG, "bad B/T/H");
    REQUIRE(s->sqrtN >= 1, SSLP_ERR_INVALID_ARG, "sqrtN must be >= 1");
    REQUIRE(s->sqrtN <= kMaxSqrtN, SSLP_ERR_UNSUPPORTED, "sqrtN %d > %d", s->sqrtN, kMaxSqrtN);
    REQUIRE(k >= 1 && k <= s->sqrtN, SSLP_ERR_INVALID_ARG, "k must be in [1, sqrtN] (got %d)", k);
    REQUIRE(k <= kMaxTopK, SSLP_ERR_UNSUPPORTED, "k must be <= %d", kMaxTopK);
    REQUIRE(budget >= 1 && budget <= k * k, SSLP_ERR_INVALID_ARG,
            "budget must be in [1, k^2] (got %d)", budget);
    REQUIRE(budget <= kMaxBudget, SSLP_ERR_UNSUPPORTED, "budget must be <= %d", kMaxBudget);
    REQUIRE_PTR(s1);
    REQUIRE_PTR(s2);
    REQUIRE_PTR(idx);
    REQUIRE_PTR(wt);
    const long long P = (long long)s->B * s->T * s->H;
    REQUIRE(P < (1ll << 31), SSLP_ERR_UNSUPPORTED, "too many problems");
    hipStream_t st = (hipStream_t)stream;
    return hip_status(sslp::launch_sdm_address((int)P, s->sqrtN, dtype, s1, s2, k, budget, idx, wt,
                                               st),
                      "sdm_address launch");
}

int sdm_sparse_update(const sslp_sdm_shape* s, int dtype, int residual_mode, const int32_t* idx_w,
                      const float* wt_w, const int32_t* idx_r, const float* wt_r, const void* v,
                      const float* alpha, const float* beta, float* M, void* y, void* workspace,
                      size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (int rc = check_sdm_shape(s, false)) return rc;
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(residual_mode == SSLP_RESIDUAL_SHARED || residual_mode == SSLP_RESIDUAL_PER_SLOT,
            SSLP_ERR_INVALID_ARG, "residual_mode must be 0 or 1 (got %d)", residual_mode);
    REQUIRE_PTR(M);
    REQUIRE_ALIGNED(workspace);
    if (s->T == 0) return SSLP_OK;  // per-token tensors are empty (and may be NULL)
    REQUIRE_PTR(idx_w);
    REQUIRE_PTR(wt_w);
    REQUIRE_PTR(idx_r);
    REQUIRE_PTR(wt_r);
    REQUIRE_PTR(v);
    REQUIRE_PTR(alpha);
    REQUIRE_PTR(beta);
    REQUIRE_PTR(y);
    const size_t need = sdm_workspace_size(s);
    REQUIRE(ws_bytes >= need && (need == 0 || workspace != nullptr), SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (s->T == 0) return SSLP_OK;
    sslp::SdmUpdateArgs a{};
    a.B = s->B;
    a.T = s->T;
    a.H = s->H;
    a.N = s->sqrtN * s->sqrtN;
    a.dv = s->d_v;
    a.W = s->W;
    a.R = s->R;
    a.dtype = dtype;
    a.residual_mode = residual_mode;
    a.idx_w = idx_w;
    a.wt_w = wt_w;
    a.idx_r = idx_r;
    a.wt_r = wt_r;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.M = M;
    a.y = y;
    a.err = error_word();
    return hip_status(run_recurrence(a, s, workspace, (hipStream_t)stream), "sdm update launch");
}

static int sdm_run(const sslp_sdm_shape* s, int T, int dtype, int residual_mode, const void* sw1,
                   const void* sw2, const void* sr1, const void* sr2, const void* v,
                   const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                   float* wt_w, int32_t* idx_r, float* wt_r, void* workspace, size_t ws_bytes,
                   size_t need, void* stream) {
    if (int rc = check_sdm_shape(s, true)) return rc;
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(residual_mode == SSLP_RESIDUAL_SHARED || residual_mode == SSLP_RESIDUAL_PER_SLOT,
            SSLP_ERR_INVALID_ARG, "residual_mode must be 0 or 1 (got %d)", residual_mode);
    REQUIRE_PTR(M);
    if (T == 0) return SSLP_OK;  // per-token tensors are empty (and may be NULL)
    REQUIRE_PTR(sw1);
    REQUIRE_PTR(sw2);
    REQUIRE_PTR(sr1);
    REQUIRE_PTR(sr2);
    REQUIRE_PTR(v);
    REQUIRE_PTR(alpha);
    REQUIRE_PTR(beta);
    REQUIRE_PTR(y);
    REQUIRE_ALIGNED(idx_w);
    REQUIRE_ALIGNED(wt_w);
    REQUIRE_ALIGNED(idx_r);
    REQUIRE_ALIGNED(wt_r);
    REQUIRE_ALIGNED(workspace);
    REQUIRE(ws_bytes >= need && (need == 0 || workspace != nullptr), SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    const long long P = (long long)s->B * T * s->H;
    REQUIRE(P < (1ll << 31), SSLP_ERR_UNSUPPORTED, "too many problems");
    hipStream_t st = (hipStream_t)stream;
    if (T == 1 && sslp::sdm_decode_fused_fits(s->sqrtN, s->d_v, s->k_w, s->W, s->k_r, s->R)) {
        // one token per sequence: addressing and update in one launch
        sslp::SdmDecodeArgs d{};
        d.P = (int)P;
        d.sqrtN = s->sqrtN;
        d.N = s->sqrtN * s->sqrtN;
        d.dv = s->d_v;
        d.dtype = dtype;
        d.residual_mode = residual_mode;
        d.s1[0] = sw1;
        d.s2[0] = sw2;
        d.s1[1] = sr1;
        d.s2[1] = sr2;
        d.idx[0] = idx_w;
        d.wt[0] = wt_w;
        d.idx[1] = idx_r;
        d.wt[1] = wt_r;
        d.k[0] = s->k_w;
        d.k[1] = s->k_r;
        d.budget[0] = s->W;
        d.budget[1] = s->R;
        d.v = v;
        d.alpha = alpha;
        d.beta = beta;
        d.M = M;
        d.y = y;
        return hip_status(sslp::launch_sdm_decode_fused(d, st), "sdm decode launch");
    }
    // addressing outputs: caller buffers when given, else workspace
    char* ws = static_cast<char*>(workspace);
    const size_t bw = align_up((size_t)P * s->W * 4), br = align_up((size_t)P * s->R * 4);
    int32_t* iw = idx_w ? idx_w : reinterpret_cast<int32_t*>(ws);
    float* ww = wt_w ? wt_w : reinterpret_cast<float*>(ws + bw);
    int32_t* ir = idx_r ? idx_r : reinterpret_cast<int32_t*>(ws + 2 * bw);
    float* wr = wt_r ? wt_r : reinterpret_cast<float*>(ws + 2 * bw + br);
    if (int rc = hip_status(sslp::launch_sdm_address_pair((int)P, s->sqrtN, dtype, sw1, sw2, s->k_w,
                                                          s->W, iw, ww, sr1, sr2, s->k_r, s->R, ir,
                                                          wr, st),
                            "sdm addressing launch"))
        return rc;
    sslp::SdmUpdateArgs a{};
    a.B = s->B;
    a.T = T;
    a.H = s->H;
    a.N = s->sqrtN * s->sqrtN;
    a.dv = s->d_v;
    a.W = s->W;
    a.R = s->R;
    a.dtype = dtype;
    a.residual_mode = residual_mode;
    a.idx_w = iw;
    a.wt_w = ww;
    a.idx_r = ir;
    a.wt_r = wr;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.M = M;
    a.y = y;
    a.err = error_word();
    return hip_status(run_recurrence(a, s, ws + addressing_bytes(s, T), st), "sdm update launch");
}

int sdm_forward(const sslp_sdm_shape* s, int dtype, int residual_mode, const void* sw1,
                const void* sw2, const void* sr1, const void* sr2, const void* v,
                const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                float* wt_w, int32_t* idx_r, float* wt_r, void* workspace, size_t ws_bytes,
                void* stream) {
    g_err[0] = 0;
    if (int rc = check_sdm_shape(s, true)) return rc;
    return sdm_run(s, s->T, dtype, residual_mode, sw1, sw2, sr1, sr2, v, alpha, beta, M, y, idx_w,
                   wt_w, idx_r, wt_r, workspace, ws_bytes, sdm_workspace_size(s), stream);
}

// ---------------------------------------------------------------------------
// sdm_forward without any allocation: the workspace is a fixed device array of
// the library, one copy per GPU, shared by every call on that GPU.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// In host code `scratch` names a host-side stand-in; the device address of each
// GPU's copy comes from hipGetSymbolAddress with that GPU current, and only
// that address is ever passed to kernels.
__device__ __align__(256) unsigned char scratch[SSLP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the scratch array on the GPU that `stream` belongs to
int scratch_for_stream(hipStream_t stream, void** out) {
    int cur = 0;
    if (hipError_t e = hipGetDevice(&cur); e != hipSuccess) return hip_status(e, "hipGetDevice");
    int dev = cur;
    if (stream != nullptr) {
        hipDevice_t d = 0;
        if (hipError_t e = hipStreamGetDevice(stream, &d); e != hipSuccess)
            return hip_status(e, "hipStreamGetDevice");
        dev = (int)d;
    }
    REQUIRE(dev >= 0 && dev < kMaxDevices, SSLP_ERR_UNSUPPORTED, "device index %d >= %d", dev,
            kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur)
            if (hipError_t e = hipSetDevice(dev); e != hipSuccess) return hip_status(e, "hipSetDevice");
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        REQUIRE(p != nullptr && ((uintptr_t)p & 255u) == 0, SSLP_ERR_HIP,
                "scratch array address %p is not 256-byte aligned", p);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSLP_OK;
}

}  // namespace

extern "C" {

size_t sdm_noalloc_scratch_bytes(void) { return (size_t)SSLP_NOALLOC_SCRATCH_BYTES; }

int sdm_forward_noalloc(const sslp_sdm_shape* s, int dtype, int residual_mode, const void* sw1,
                        const void* sw2, const void* sr1, const void* sr2, const void* v,
                        const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                        float* wt_w, int32_t* idx_r, float* wt_r, void* stream) {
    g_err[0] = 0;
    if (int rc = check_sdm_shape(s, true)) return rc;
    const size_t need = sdm_workspace_size(s);
    REQUIRE(need <= (size_t)SSLP_NOALLOC_SCRATCH_BYTES, SSLP_ERR_WORKSPACE,
            "sdm_forward_noalloc: this shape needs %zu bytes of scratch, above the fixed %zu "
            "(use sdm_forward with a workspace)",
            need, (size_t)SSLP_NOALLOC_SCRATCH_BYTES);
    // the pointer checks of sdm_forward, before the first HIP call
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE_PTR(M);
    if (s->T > 0) {
        REQUIRE_PTR(sw1);
        REQUIRE_PTR(sw2);
        REQUIRE_PTR(sr1);
        REQUIRE_PTR(sr2);
        REQUIRE_PTR(v);
        REQUIRE_PTR(alpha);
        REQUIRE_PTR(beta);
        REQUIRE_PTR(y);
    }
    void* ws = nullptr;
    if (need > 0 && s->T > 0)
        if (int rc = scratch_for_stream((hipStream_t)stream, &ws)) return rc;
    return sdm_forward(s, dtype, residual_mode, sw1, sw2, sr1, sr2, v, alpha, beta, M, y, idx_w,
                       wt_w, idx_r, wt_r, ws, need, stream);
}

int sdm_decode_step(const sslp_sdm_shape* s, int dtype, int residual_mode, const void* sw1,
                    const void* sw2, const void* sr1, const void* sr2, const void* v,
                    const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                    float* wt_w, int32_t* idx_r, float* wt_r, void* workspace, size_t ws_bytes,
                    void* stream) {
    g_err[0] = 0;
    if (int rc = check_sdm_shape(s, true)) return rc;
    REQUIRE(s->T == 1, SSLP_ERR_INVALID_ARG, "sdm_decode_step needs shape->T == 1 (got %d)", s->T);
    return sdm_run(s, 1, dtype, residual_mode, sw1, sw2, sr1, sr2, v, alpha, beta, M, y, idx_w,
                   wt_w, idx_r, wt_r, workspace, ws_bytes, sdm_decode_workspace_size(s), stream);
}

// ---------------------------------------------------------------------------
// SDM training: forward that keeps the pre-write rows, backward by undoing writes
// ---------------------------------------------------------------------------

static sslp::SdmUpdateArgs update_args(const sslp_sdm_shape* s, int dtype, int residual_mode,
                                       const int32_t* idx_w, const float* wt_w,
                                       const int32_t* idx_r, const float* wt_r, const void* v,
                                       const float* alpha, const float* beta, float* M, void* y,
                                       float* saved) {
    sslp::SdmUpdateArgs a{};
    a.B = s->B;
    a.T = s->T;
    a.H = s->H;
    a.N = s->sqrtN * s->sqrtN;
    a.dv = s->d_v;
    a.W = s->W;
    a.R = s->R;
    a.dtype = dtype;
    a.residual_mode = residual_mode;
    a.idx_w = idx_w;
    a.wt_w = wt_w;
    a.idx_r = idx_r;
    a.wt_r = wt_r;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.M = M;
    a.y = y;
    a.saved = saved;
    a.err = error_word();
    return a;
}

static int check_common(const sslp_sdm_shape* s, bool need_k, int dtype, int residual_mode) {
    if (int rc = check_sdm_shape(s, need_k)) return rc;
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(residual_mode == SSLP_RESIDUAL_SHARED || residual_mode == SSLP_RESIDUAL_PER_SLOT,
            SSLP_ERR_INVALID_ARG, "residual_mode must be 0 or 1 (got %d)", residual_mode);
    return SSLP_OK;
}

// the backward runs chunk-parallel where the forward does
bool backward_chunked(const sslp_sdm_shape* s) {
    return sslp::sdm_chunked_supported(s->B, s->T, s->H, s->W, s->R, s->d_v, slots(s));
}

// workspace of sdm_backward: slice partial sums | weight gradients the caller
// does not keep | (chunk-parallel) forward plans | backward plans
size_t bwd_part_bytes(const sslp_sdm_shape* s) {
    const int cols = backward_chunked(s) ? sslp::kChunkBwdSliceCols : 16;
    return align_up(sslp::sdm_bwd_part_bytes(s->B, s->T, s->H, s->d_v, s->W, s->R, cols));
}

size_t sdm_backward_workspace_size(const sslp_sdm_shape* s) {
    if (check_sdm_shape(s, false) != SSLP_OK) return 0;
    const size_t bth = (size_t)s->B * s->T * s->H;
    size_t n = bwd_part_bytes(s) + align_up(bth * s->W * 4) + align_up(bth * s->R * 4);
    if (backward_chunked(s))
        n += align_up(sslp::sdm_chunk_plan_bytes(s->B, s->T, s->H, s->W)) +
             align_up(sslp::sdm_chunk_bwd_plan_bytes(s->B, s->T, s->H, s->W));
    return n;
}

size_t sdm_train_workspace_size(const sslp_sdm_shape* s) {
    if (check_sdm_shape(s, false) != SSLP_OK) return 0;
    return recurrence_bytes(s, s->T);
}

int sdm_sparse_update_train(const sslp_sdm_shape* s, int dtype, int residual_mode,
                            const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                            const float* wt_r, const void* v, const float* alpha,
                            const float* beta, float* M, void* y, float* saved, void* workspace,
                            size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (int rc = check_common(s, false, dtype, residual_mode)) return rc;
    REQUIRE_PTR(M);
    REQUIRE_ALIGNED(workspace);
    if (s->T == 0) return SSLP_OK;
    REQUIRE_PTR(idx_w);
    REQUIRE_PTR(wt_w);
    REQUIRE_PTR(idx_r);
    REQUIRE_PTR(wt_r);
    REQUIRE_PTR(v);
    REQUIRE_PTR(alpha);
    REQUIRE_PTR(beta);
    REQUIRE_PTR(y);
    REQUIRE_PTR(saved);
    const size_t need = sdm_train_workspace_size(s);
    REQUIRE(ws_bytes >= need && (need == 0 || workspace != nullptr), SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    const sslp::SdmUpdateArgs a = update_args(s, dtype, residual_mode, idx_w, wt_w, idx_r, wt_r, v,
                                              alpha, beta, M, y, saved);
    return hip_status(run_recurrence(a, s, workspace, (hipStream_t)stream),
                      "sdm train update launch");
}

int sdm_forward_train(const sslp_sdm_shape* s, int dtype, int residual_mode, const void* sw1,
                      const void* sw2, const void* sr1, const void* sr2, const void* v,
                      const float* alpha, const float* beta, float* M, void* y, int32_t* idx_w,
                      float* wt_w, int32_t* idx_r, float* wt_r, float* saved, void* workspace,
                      size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (int rc = check_common(s, true, dtype, residual_mode)) return rc;
    REQUIRE_PTR(M);
    REQUIRE_ALIGNED(workspace);
    if (s->T == 0) return SSLP_OK;
    REQUIRE_PTR(sw1);
    REQUIRE_PTR(sw2);
    REQUIRE_PTR(sr1);
    REQUIRE_PTR(sr2);
    REQUIRE_PTR(v);
    REQUIRE_PTR(alpha);
    REQUIRE_PTR(beta);
    REQUIRE_PTR(y);
    REQUIRE_PTR(idx_w);
    REQUIRE_PTR(wt_w);
    REQUIRE_PTR(idx_r);
    REQUIRE_PTR(wt_r);
    REQUIRE_PTR(saved);
    const size_t need = sdm_train_workspace_size(s);
    REQUIRE(ws_bytes >= need && (need == 0 || workspace != nullptr), SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    const long long P = (long long)s->B * s->T * s->H;
    REQUIRE(P < (1ll << 31), SSLP_ERR_UNSUPPORTED, "too many problems");
    hipStream_t st = (hipStream_t)stream;
    if (int rc = hip_status(sslp::launch_sdm_address_pair((int)P, s->sqrtN, dtype, sw1, sw2, s->k_w,
                                                          s->W, idx_w, wt_w, sr1, sr2, s->k_r,
                                                          s->R, idx_r, wt_r, st),
                            "sdm addressing launch"))
        return rc;
    const sslp::SdmUpdateArgs a = update_args(s, dtype, residual_mode, idx_w, wt_w, idx_r, wt_r, v,
                                              alpha, beta, M, y, saved);
    return hip_status(run_recurrence(a, s, workspace, st), "sdm train update launch");
}

int sdm_backward(const sslp_sdm_shape* s, int dtype, int residual_mode, const int32_t* idx_w,
                 const float* wt_w, const int32_t* idx_r, const float* wt_r, const void* v,
                 const float* alpha, const float* beta, float* M, const float* saved,
                 const void* dy, float* dM, void* dv, float* dalpha, float* dbeta, float* dwt_w,
                 float* dwt_r, float* dsw1, float* dsw2, float* dsr1, float* dsr2, void* workspace,
                 size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (int rc = check_common(s, false, dtype, residual_mode)) return rc;
    REQUIRE_PTR(M);
    REQUIRE_PTR(dM);
    if (s->T == 0) return SSLP_OK;
    REQUIRE_PTR(idx_w);
    REQUIRE_PTR(wt_w);
    REQUIRE_PTR(idx_r);
    REQUIRE_PTR(wt_r);
    REQUIRE_PTR(v);
    REQUIRE_PTR(alpha);
    REQUIRE_PTR(beta);
    REQUIRE_PTR(saved);
    REQUIRE_PTR(dy);
    REQUIRE_PTR(dv);
    REQUIRE_PTR(dalpha);
    REQUIRE_PTR(dbeta);
    REQUIRE_ALIGNED(dwt_w);
    REQUIRE_ALIGNED(dwt_r);
    REQUIRE_ALIGNED(dsw1);
    REQUIRE_ALIGNED(dsw2);
    REQUIRE_ALIGNED(dsr1);
    REQUIRE_ALIGNED(dsr2);
    REQUIRE((dsw1 == nullptr) == (dsw2 == nullptr) && (dsr1 == nullptr) == (dsr2 == nullptr),
            SSLP_ERR_INVALID_ARG, "score-half gradients come in pairs (dsw1 with dsw2, dsr1 with dsr2)");
    REQUIRE_ALIGNED(workspace);
    const size_t need = sdm_backward_workspace_size(s);
    REQUIRE(workspace != nullptr && ws_bytes >= need, SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    const long long P = (long long)s->B * s->T * s->H;
    REQUIRE(P < (1ll << 31), SSLP_ERR_UNSUPPORTED, "too many problems");
    char* ws = static_cast<char*>(workspace);
    const size_t bp = bwd_part_bytes(s);
    const size_t bw = align_up((size_t)P * s->W * 4);
    const size_t br = align_up((size_t)P * s->R * 4);
    sslp::SdmBwdArgs a{};
    a.B = s->B;
    a.T = s->T;
    a.H = s->H;
    a.N = s->sqrtN * s->sqrtN;
    a.dv = s->d_v;
    a.W = s->W;
    a.R = s->R;
    a.dtype = dtype;
    a.residual_mode = residual_mode;
    a.idx_w = idx_w;
    a.wt_w = wt_w;
    a.idx_r = idx_r;
    a.wt_r = wt_r;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.M = M;
    a.saved = saved;
    a.dy = dy;
    a.dM = dM;
    a.dv_out = dv;
    a.part = reinterpret_cast<float*>(ws);
    a.dalpha = dalpha;
    a.dbeta = dbeta;
    a.dwt_w = dwt_w ? dwt_w : reinterpret_cast<float*>(ws + bp);
    a.dwt_r = dwt_r ? dwt_r : reinterpret_cast<float*>(ws + bp + bw);
    a.err = error_word();
    hipStream_t st = (hipStream_t)stream;
    if (backward_chunked(s)) {
        char* fplan = ws + bp + bw + br;
        char* bplan = fplan + align_up(sslp::sdm_chunk_plan_bytes(s->B, s->T, s->H, s->W));
        if (int rc = hip_status(sslp::launch_sdm_backward_chunked(a, fplan, bplan, st),
                                "sdm backward launch"))
            return rc;
    } else if (int rc = hip_status(sslp::launch_sdm_update_backward(a, st), "sdm backward launch")) {
        return rc;
    }
    if (dsw1 && dsr1)
        return hip_status(sslp::launch_sdm_address_backward_pair(
                              (int)P, s->sqrtN, s->W, idx_w, wt_w, a.dwt_w, dsw1, dsw2, s->R,
                              idx_r, wt_r, a.dwt_r, dsr1, dsr2, st),
                          "sdm address backward launch");
    if (dsw1)
        if (int rc = hip_status(sslp::launch_sdm_address_backward((int)P, s->sqrtN, s->W, idx_w,
                                                                  wt_w, a.dwt_w, dsw1, dsw2, st),
                                "sdm address backward launch"))
            return rc;
    if (dsr1)
        return hip_status(sslp::launch_sdm_address_backward((int)P, s->sqrtN, s->R, idx_r, wt_r,
                                                            a.dwt_r, dsr1, dsr2, st),
                          "sdm address backward launch");
    return SSLP_OK;
}

int sdm_norm_gate(long long rows, int d, int dtype, const void* y, const void* gate,
                  const float* gamma, float eps, int act, void* o, void* stream) {
    g_err[0] = 0;
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(rows >= 0 && d >= 1, SSLP_ERR_INVALID_ARG, "rows >= 0 and d >= 1 needed");
    REQUIRE(d % 4 == 0 && d <= kMaxDv, SSLP_ERR_UNSUPPORTED,
            "d must be a multiple of 4 and <= %d (got %d)", kMaxDv, d);
    REQUIRE(act >= SSLP_GATE_NONE && act <= SSLP_GATE_SIGMOID, SSLP_ERR_INVALID_ARG,
            "act must be SSLP_GATE_NONE, SSLP_GATE_SILU or SSLP_GATE_SIGMOID (got %d)", act);
    REQUIRE(eps >= 0.f, SSLP_ERR_INVALID_ARG, "eps must be >= 0");
    if (rows == 0) return SSLP_OK;
    REQUIRE_PTR(y);
    REQUIRE_PTR(gamma);
    REQUIRE_PTR(o);
    if (act != SSLP_GATE_NONE) REQUIRE_PTR(gate);
    REQUIRE_ALIGNED(gate);
    REQUIRE(rows <= (1ll << 40), SSLP_ERR_UNSUPPORTED, "too many rows");
    return hip_status(sslp::launch_norm_gate(rows, d, dtype, y, gate, gamma, eps, act, o,
                                             (hipStream_t)stream),
                      "sdm_norm_gate launch");
}

// ---------------------------------------------------------------------------
// GDN / KDA and SSE: argument checks (kernels follow)
// ---------------------------------------------------------------------------
static int check_gdn_shape(const sslp_gdn_shape* s) {
    REQUIRE(s != nullptr, SSLP_ERR_INVALID_ARG, "shape must not be NULL");
    REQUIRE(s->B >= 1 && s->H >= 1 && s->T >= 0, SSLP_ERR_INVALID_ARG, "bad B/T/H");
    REQUIRE(s->d_k >= 1 && s->d_v >= 1 && s->chunk >= 1, SSLP_ERR_INVALID_ARG,
            "d_k, d_v, chunk must be >= 1");
    REQUIRE(s->d_k == 128 && s->d_v == 128 && s->chunk == 64, SSLP_ERR_UNSUPPORTED,
            "only d_k = d_v = 128 and chunk = 64 are supported (got %d, %d, %d)", s->d_k, s->d_v,
            s->chunk);
    return SSLP_OK;
}

size_t gdn_workspace_size(const sslp_gdn_shape* s) {
    if (check_gdn_shape(s) != SSLP_OK) return 0;
    return align_up(sslp::gdn_record_bytes(s->B, s->T, s->H));
}

int gdn_chunk_forward(const sslp_gdn_shape* s, int dtype, int decay_mode, const void* q,
                      const void* k, const void* v, const float* alpha, const float* beta,
                      const float* S0, float* S_out, void* o, void* workspace, size_t ws_bytes,
                      void* stream) {
    g_err[0] = 0;
    if (int rc = check_gdn_shape(s)) return rc;
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(decay_mode == SSLP_DECAY_SCALAR || decay_mode == SSLP_DECAY_CHANNEL,
            SSLP_ERR_INVALID_ARG, "decay_mode must be 0 or 1 (got %d)", decay_mode);
    REQUIRE_ALIGNED(q);
    REQUIRE_ALIGNED(k);
    REQUIRE_ALIGNED(v);
    REQUIRE_ALIGNED(alpha);
    REQUIRE_ALIGNED(beta);
    REQUIRE_ALIGNED(o);
    REQUIRE_ALIGNED(S0);
    REQUIRE(dtype == SSLP_BF16, SSLP_ERR_UNSUPPORTED,
            "gdn_chunk_forward supports bf16 q/k/v only (got dtype %d)", dtype);
    REQUIRE_PTR(S_out);
    if (s->T > 0) {
        REQUIRE_PTR(q);
        REQUIRE_PTR(k);
        REQUIRE_PTR(v);
        REQUIRE_PTR(alpha);
        REQUIRE_PTR(beta);
        REQUIRE_PTR(o);
    }
    const size_t need = gdn_workspace_size(s);
    REQUIRE(ws_bytes >= need && (need == 0 || workspace != nullptr), SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    REQUIRE_ALIGNED(workspace);
    return hip_status(sslp::launch_gdn_chunk(s->B, s->T, s->H, s->d_v, dtype, decay_mode, q, k, v,
                                             alpha, beta, S0, S_out, o, workspace,
                                             (hipStream_t)stream),
                      "gdn_chunk_forward launch");
}

int gdn2_chunk_forward(const sslp_gdn_shape* s, int dtype, const void* q, const void* k,
                       const void* v, const float* alpha, const float* erase, const float* write,
                       const float* S0, float* S_out, void* o, void* workspace, size_t ws_bytes,
                       void* stream) {
    g_err[0] = 0;
    if (int rc = check_gdn_shape(s)) return rc;
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE_ALIGNED(q);
    REQUIRE_ALIGNED(k);
    REQUIRE_ALIGNED(v);
    REQUIRE_ALIGNED(alpha);
    REQUIRE_ALIGNED(erase);
    REQUIRE_ALIGNED(write);
    REQUIRE_ALIGNED(o);
    REQUIRE_ALIGNED(S0);
    REQUIRE(dtype == SSLP_BF16, SSLP_ERR_UNSUPPORTED,
            "gdn2_chunk_forward supports bf16 q/k/v only (got dtype %d)", dtype);
    REQUIRE_PTR(S_out);
    if (s->T > 0) {
        REQUIRE_PTR(q);
        REQUIRE_PTR(k);
        REQUIRE_PTR(v);
        REQUIRE_PTR(alpha);
        REQUIRE_PTR(erase);
        REQUIRE_PTR(write);
        REQUIRE_PTR(o);
    }
    const size_t need = gdn_workspace_size(s);
    REQUIRE(ws_bytes >= need && (need == 0 || workspace != nullptr), SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    REQUIRE_ALIGNED(workspace);
    return hip_status(sslp::launch_gdn_chunk(s->B, s->T, s->H, s->d_v, dtype, 2, q, k, v, alpha,
                                             nullptr, S0, S_out, o, workspace, (hipStream_t)stream,
                                             erase, write),
                      "gdn2_chunk_forward launch");
}

static int check_sse_shape(const sslp_sse_shape* s) {
    REQUIRE(s != nullptr, SSLP_ERR_INVALID_ARG, "shape must not be NULL");
    REQUIRE(s->B >= 1 && s->H >= 1 && s->T >= 0, SSLP_ERR_INVALID_ARG, "bad B/T/H");
    REQUIRE(s->N >= 1 && s->topk >= 1 && s->topk <= s->N, SSLP_ERR_INVALID_ARG,
            "need 1 <= topk <= N (topk=%d N=%d)", s->topk, s->N);
    REQUIRE(s->N <= 8 && s->topk <= 4, SSLP_ERR_UNSUPPORTED, "need N <= 8 and topk <= 4");
    REQUIRE(s->c >= 1 && s->d >= 1 && s->chunk >= 1, SSLP_ERR_INVALID_ARG,
            "c, d, chunk must be >= 1");
    REQUIRE(s->c == 128 && s->d == 128 && s->chunk == 64, SSLP_ERR_UNSUPPORTED,
            "only c = d = 128 and chunk = 64 are supported");
    return SSLP_OK;
}

// routing results (selected partitions, their gates) when the caller does not take them
static size_t sse_route_bytes(const sslp_sse_shape* s) {
    return align_up((size_t)s->B * s->T * s->H * s->topk * 4);
}

size_t sse_workspace_size(const sslp_sse_shape* s) {
    if (check_sse_shape(s) != SSLP_OK) return 0;
    return 2 * sse_route_bytes(s) + sslp::sse_scratch_bytes(s->B, s->T, s->H, s->N, s->topk, s->d);
}

static int sse_run(const char* name, int masking, const sslp_sse_shape* s, int dtype,
                   const float* gate_logits, const void* q, const void* k, const void* v,
                   const float* lambda, const void* q_sh, const void* k_sh, float* S, void* o,
                   int32_t* sel, float* e_sel, void* workspace, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (int rc = check_sse_shape(s)) return rc;
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(dtype == SSLP_BF16, SSLP_ERR_UNSUPPORTED,
            "%s supports bf16 q/k/v only (got dtype %d)", name, dtype);
    REQUIRE_PTR(S);
    REQUIRE_ALIGNED(q_sh);
    REQUIRE_ALIGNED(k_sh);
    REQUIRE_ALIGNED(sel);
    REQUIRE_ALIGNED(e_sel);
    if (s->T == 0) return SSLP_OK;
    REQUIRE_PTR(gate_logits);
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(lambda);
    REQUIRE_PTR(o);
    REQUIRE(workspace != nullptr && ws_bytes >= sse_workspace_size(s), SSLP_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", sse_workspace_size(s), ws_bytes);
    REQUIRE_ALIGNED(workspace);
    char* ws = static_cast<char*>(workspace);
    if (sel == nullptr) sel = reinterpret_cast<int32_t*>(ws);
    if (e_sel == nullptr) e_sel = reinterpret_cast<float*>(ws + sse_route_bytes(s));
    return hip_status(sslp::launch_sse(s->B, s->T, s->H, s->N, s->topk, s->d, dtype, gate_logits,
                                       q, k, v, lambda, q_sh, k_sh, S, o, sel, e_sel,
                                       ws + 2 * sse_route_bytes(s), (hipStream_t)stream, masking),
                      name);
}

int sse_forward(const sslp_sse_shape* s, int dtype, const float* gate_logits, const void* q,
                const void* k, const void* v, const float* lambda, const void* q_sh,
                const void* k_sh, float* S, void* o, int32_t* sel, float* e_sel, void* workspace,
                size_t ws_bytes, void* stream) {
    return sse_run("sse_forward", 0, s, dtype, gate_logits, q, k, v, lambda, q_sh, k_sh, S, o, sel,
                   e_sel, workspace, ws_bytes, stream);
}

int sse_forward_masking(const sslp_sse_shape* s, int dtype, const float* gate_logits,
                        const void* q, const void* k, const void* v, const float* lambda,
                        const void* q_sh, const void* k_sh, float* S, void* o, int32_t* sel,
                        float* e_sel, void* workspace, size_t ws_bytes, void* stream) {
    return sse_run("sse_forward_masking", 1, s, dtype, gate_logits, q, k, v, lambda, q_sh, k_sh, S,
                   o, sel, e_sel, workspace, ws_bytes, stream);
}

int sse_decode_step(const sslp_sse_shape* s, int dtype, const float* gate_logits, const void* q,
                    const void* k, const void* v, const float* lambda, const void* q_sh,
                    const void* k_sh, float* S, void* o, int32_t* sel, float* e_sel, void* stream) {
    g_err[0] = 0;
    if (int rc = check_sse_shape(s)) return rc;
    REQUIRE(s->T == 1, SSLP_ERR_INVALID_ARG, "sse_decode_step takes T = 1 (got %d)", s->T);
    if (int rc = check_dtype(dtype)) return rc;
    REQUIRE(dtype == SSLP_BF16, SSLP_ERR_UNSUPPORTED,
            "sse_decode_step supports bf16 q/k/v only (got dtype %d)", dtype);
    REQUIRE_PTR(S);
    REQUIRE_PTR(gate_logits);
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(lambda);
    REQUIRE_PTR(o);
    REQUIRE_ALIGNED(q_sh);
    REQUIRE_ALIGNED(k_sh);
    REQUIRE_ALIGNED(sel);
    REQUIRE_ALIGNED(e_sel);
    return hip_status(sslp::launch_sse_decode(s->B, s->H, s->N, s->topk, s->d, gate_logits, q, k,
                                              v, lambda, q_sh, k_sh, S, o, sel, e_sel,
                                              (hipStream_t)stream),
                      "sse_decode_step launch");
}

}  // extern "C"
