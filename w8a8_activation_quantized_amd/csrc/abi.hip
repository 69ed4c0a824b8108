// C-ABI layer of libw8a8: argument validation, device checks, status codes and
// dispatch to the kernel launchers. Every check runs on the host before anything is
// enqueued, so an invalid call leaves the stream untouched.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/w8a8.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return W8A8_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool forced_unavailable() {
    const char *e = getenv("W8A8_FORCE_UNAVAILABLE");
    return e && e[0] == '1' && e[1] == '\0';
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_force_cfg{-1};
std::atomic<int> g_force_slices{-1};

bool device_is_gfx950(int device) {
    if (device < 0 || device >= kMaxDevices) return false;
    int cached = g_arch_ok[device].load(std::memory_order_relaxed);
    if (cached == 0) {
        int count = 0;
        hipDeviceProp_t prop;
        bool good = hipGetDeviceCount(&count) == hipSuccess && device < count &&
                    hipGetDeviceProperties(&prop, device) == hipSuccess &&
                    strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        cached = good ? 1 : 2;
        g_arch_ok[device].store(cached, std::memory_order_relaxed);
    }
    return cached == 1;
}

// Checks the current device; returns W8A8_OK or an error status (message set).
int check_device() {
    if (forced_unavailable())
        return fail(W8A8_ERR_UNSUPPORTED_DEVICE, "W8A8_FORCE_UNAVAILABLE=1 is set");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(W8A8_ERR_UNSUPPORTED_DEVICE, "no HIP device available");
    }
    if (!device_is_gfx950(dev))
        return fail(W8A8_ERR_UNSUPPORTED_DEVICE, "device %d is not a gfx950 (MI355X) GPU", dev);
    return W8A8_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(W8A8_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool valid_out(int d) { return d == W8A8_F16 || d == W8A8_BF16 || d == W8A8_F32 || d == W8A8_I32; }

// Shape, dtype and stride checks shared by the GEMM entry points.
int check_gemm_shape(const char *fn, int gs, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                     bool per_group) {
    if (M < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: M = %lld < 0", fn, (long long)M);
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || N * K > ((int64_t)1 << 40) ||
        M * K > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    if (N < 16 || N % 16 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: N = %lld must be a positive multiple of 16", fn,
                    (long long)N);
    if (K < 64 || K % 64 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K = %lld must be a positive multiple of 64", fn,
                    (long long)K);
    if (per_group) {
        if (gs != 64 && gs != 128)
            return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: group_size = %d must be 64 or 128", fn, gs);
        if (K % gs != 0)
            return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K = %lld not a multiple of group_size %d", fn,
                        (long long)K, gs);
    }
    if (!valid_out(y_dtype)) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: bad y_dtype %d", fn, y_dtype);
    if (ldy < N || ldy % 4 != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: ldy = %lld must be >= N and a multiple of 4", fn,
                    (long long)ldy);
    return W8A8_OK;
}

// Shared validation of the GEMM entry points.
int check_gemm(const char *fn, const void *x_q, const float *s_x, const void *w, const float *s_w,
               int gs, const void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
               bool per_group) {
    const int rc = check_gemm_shape(fn, gs, y_dtype, M, N, K, ldy, per_group);
    if (rc != W8A8_OK) return rc;
    if (M == 0) return W8A8_OK;
    if (!x_q || !s_x || !w || !s_w || !y) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (!aligned16(x_q) || !aligned16(s_x) || !aligned16(w) || !aligned16(s_w) || !aligned16(y))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    return W8A8_OK;
}

w8a8::GemmProblem make_problem(const int8_t *x_q, const float *s_x, const void *w, const float *s_w, int gs,
                               int wkind, void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy) {
    w8a8::GemmProblem p;
    p.xq = x_q;
    p.sx = s_x;
    p.wq = w;
    p.sw = s_w;
    p.y = y;
    p.ldy = ldy;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.gs = gs;
    p.wkind = wkind;
    p.out = y_dtype;
    {
        const int64_t esize = (y_dtype == W8A8_F16 || y_dtype == W8A8_BF16) ? 2 : 4;
        p.y_rows16 = ((reinterpret_cast<uintptr_t>(y) & 15) == 0 && ((ldy * esize) & 15) == 0) ? 1 : 0;
    }
    p.x = nullptr;
    p.ldx = 0;
    p.x_bf16 = 0;
    p.xq_out = nullptr;
    p.sx_out = nullptr;
    p.ksplit = 1;
    p.ws = nullptr;
    return p;
}

int run_gemm(const char *fn, const int8_t *x_q, const float *s_x, const void *w, const float *s_w,
             int gs, int wkind, void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
             void *stream) {
    int rc = check_gemm(fn, x_q, s_x, w, s_w, gs, y, y_dtype, M, N, K, ldy, gs != 0);
    if (rc != W8A8_OK) return rc;
    if ((rc = check_device()) != W8A8_OK) return rc;
    if (M == 0) return ok();
    const w8a8::GemmProblem p = make_problem(x_q, s_x, w, s_w, gs, wkind, y, y_dtype, M, N, K, ldy);
    return launched(w8a8::launch_gemm(p, g_force_cfg.load(std::memory_order_relaxed),
                                      static_cast<hipStream_t>(stream)),
                    fn);
}

}  // namespace

namespace w8a8 {

int num_cus() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cached.store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace w8a8

extern "C" {

int w8a8_is_available(int device) {
    if (forced_unavailable()) return 0;
    return device_is_gfx950(device) ? 1 : 0;
}

const char *w8a8_status_string(int status) {
    switch (status) {
        case W8A8_OK: return "ok";
        case W8A8_ERR_INVALID_ARGUMENT: return "invalid argument";
        case W8A8_ERR_UNSUPPORTED_DEVICE: return "unsupported device";
        case W8A8_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case W8A8_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char *w8a8_last_error(void) { return g_last_error; }

int w8a8_abi_version(void) { return 1; }

int w8a8_debug_force_config(int config_id) {
    if (config_id < -1 || config_id >= w8a8::gemm_num_configs()) return -W8A8_ERR_INVALID_ARGUMENT;
    g_force_cfg.store(config_id, std::memory_order_relaxed);
    return w8a8::gemm_num_configs();
}

int quantize_per_token(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t *x_q,
                       float *s_x, void *stream) {
    const char *fn = "quantize_per_token";
    if (x_dtype != W8A8_F16 && x_dtype != W8A8_BF16)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: x_dtype must be F16 or BF16", fn);
    if (M < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: M = %lld < 0", fn, (long long)M);
    if (K < 8 || K % 8 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K = %lld must be a positive multiple of 8", fn,
                    (long long)K);
    if (M > INT32_MAX || K > INT32_MAX || M * K > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    if (ldx < K || ldx % 8 != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: ldx = %lld must be >= K and a multiple of 8", fn,
                    (long long)ldx);
    if (M > 0) {
        if (!x || !x_q || !s_x) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
        if (!aligned16(x) || !aligned16(x_q) || !aligned16(s_x))
            return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    }
    int rc = check_device();
    if (rc != W8A8_OK) return rc;
    if (M == 0) return ok();
    return launched(w8a8::launch_quantize_per_token(x, x_dtype == W8A8_BF16, ldx, (int)M, (int)K, x_q,
                                                    s_x, static_cast<hipStream_t>(stream)),
                    fn);
}

int rmsnorm_quantize(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const void *gamma,
                     int gamma_dtype, float eps, int8_t *x_q, float *s_x, void *stream) {
    const char *fn = "rmsnorm_quantize";
    if (x_dtype != W8A8_F16 && x_dtype != W8A8_BF16)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: x_dtype must be F16 or BF16", fn);
    if (gamma_dtype != W8A8_F16 && gamma_dtype != W8A8_BF16)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: gamma_dtype must be F16 or BF16", fn);
    if (!(eps >= 0.0f && eps <= 3.0e38f))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
    if (M < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: M = %lld < 0", fn, (long long)M);
    if (K < 8 || K % 8 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K = %lld must be a positive multiple of 8", fn,
                    (long long)K);
    if (M > INT32_MAX || K > INT32_MAX || M * K > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    if (ldx < K || ldx % 8 != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: ldx = %lld must be >= K and a multiple of 8", fn,
                    (long long)ldx);
    if (M > 0) {
        if (!x || !gamma || !x_q || !s_x) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
        if (!aligned16(x) || !aligned16(gamma) || !aligned16(x_q) || !aligned16(s_x))
            return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    }
    int rc = check_device();
    if (rc != W8A8_OK) return rc;
    if (M == 0) return ok();
    return launched(w8a8::launch_rmsnorm_quantize(x, x_dtype == W8A8_BF16, ldx, gamma, gamma_dtype == W8A8_BF16,
                                                  eps, (int)M, (int)K, x_q, s_x, static_cast<hipStream_t>(stream)),
                    fn);
}

int swiglu_quantize(const void *gate, const void *up, int dtype, int64_t M, int64_t I, int64_t ldg, int64_t ldu,
                    int8_t *x_q, float *s_x, void *stream) {
    const char *fn = "swiglu_quantize";
    if (dtype != W8A8_F16 && dtype != W8A8_BF16)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: dtype must be F16 or BF16", fn);
    if (M < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: M = %lld < 0", fn, (long long)M);
    if (I < 8 || I % 8 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: I = %lld must be a positive multiple of 8", fn, (long long)I);
    if (M > INT32_MAX || I > INT32_MAX || M * I > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    if (ldg < I || ldg % 8 != 0 || ldu < I || ldu % 8 != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: ldg = %lld, ldu = %lld must be >= I and multiples of 8", fn,
                    (long long)ldg, (long long)ldu);
    if (M > 0) {
        if (!gate || !up || !x_q || !s_x) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
        if (!aligned16(gate) || !aligned16(up) || !aligned16(x_q) || !aligned16(s_x))
            return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    }
    int rc = check_device();
    if (rc != W8A8_OK) return rc;
    if (M == 0) return ok();
    return launched(w8a8::launch_swiglu_quantize(gate, ldg, up, ldu, dtype == W8A8_BF16, (int)M, (int)I, x_q, s_x,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

int quantize_weight(const float *W, int64_t N, int64_t K, int bits, int group_size, void *w_q,
                    float *s_w, void *stream) {
    const char *fn = "quantize_weight";
    if (bits != 8 && bits != 4) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: bits must be 8 or 4", fn);
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: group_size must be 0, 64 or 128", fn);
    if (N < 1) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: N = %lld < 1", fn, (long long)N);
    if (K < 64 || K % 64 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K = %lld must be a positive multiple of 64", fn,
                    (long long)K);
    if (group_size && K % group_size != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K not a multiple of group_size", fn);
    if (N > INT32_MAX || K > INT32_MAX || N * K > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    if (!W || !w_q || !s_w) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (!aligned16(W) || !aligned16(w_q) || !aligned16(s_w))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    int rc = check_device();
    if (rc != W8A8_OK) return rc;
    return launched(w8a8::launch_quantize_weight(W, (int)N, (int)K, bits, group_size, w_q, s_w,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

int quantize_weight_clipped(const float *W, int64_t N, int64_t K, int bits, int group_size, float clip_percentile,
                            void *w_q, float *s_w, void *stream) {
    const char *fn = "quantize_weight_clipped";
    if (!(clip_percentile > 0.0f && clip_percentile <= 100.0f))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: clip_percentile must be in (0, 100]", fn);
    if (bits != 8 && bits != 4) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: bits must be 8 or 4", fn);
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: group_size must be 0, 64 or 128", fn);
    if (N < 1) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: N = %lld < 1", fn, (long long)N);
    if (K < 64 || K % 64 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K = %lld must be a positive multiple of 64", fn,
                    (long long)K);
    if (group_size && K % group_size != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K not a multiple of group_size", fn);
    if (N > INT32_MAX || K > INT32_MAX || N * K > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    if (!W || !w_q || !s_w) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (!aligned16(W) || !aligned16(w_q) || !aligned16(s_w))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    int rc = check_device();
    if (rc != W8A8_OK) return rc;
    return launched(w8a8::launch_quantize_weight_clipped(W, (int)N, (int)K, bits, group_size, clip_percentile, w_q,
                                                         s_w, static_cast<hipStream_t>(stream)),
                    fn);
}

int w8a8_gemm_pc(const int8_t *x_q, const float *s_x, const int8_t *w_q, const float *s_w, void *y,
                 int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy, void *stream) {
    return run_gemm("w8a8_gemm_pc", x_q, s_x, w_q, s_w, 0, w8a8::W_INT8, y, y_dtype, M, N, K, ldy, stream);
}

int w8a8_gemm_pg(const int8_t *x_q, const float *s_x, const int8_t *w_q, const float *s_w,
                 int group_size, void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                 void *stream) {
    if (group_size == 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "w8a8_gemm_pg: group_size must be 64 or 128");
    return run_gemm("w8a8_gemm_pg", x_q, s_x, w_q, s_w, group_size, w8a8::W_INT8, y, y_dtype, M, N, K,
                    ldy, stream);
}

int w4a8_gemm_pg(const int8_t *x_q, const float *s_x, const uint8_t *w_packed, const float *s_w,
                 int group_size, void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                 void *stream) {
    if (group_size == 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "w4a8_gemm_pg: group_size must be 64 or 128");
    return run_gemm("w4a8_gemm_pg", x_q, s_x, w_packed, s_w, group_size, w8a8::W_INT4, y, y_dtype, M, N,
                    K, ldy, stream);
}

int w4a8_gemm_pc(const int8_t *x_q, const float *s_x, const uint8_t *w_packed, const float *s_w, void *y,
                 int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy, void *stream) {
    return run_gemm("w4a8_gemm_pc", x_q, s_x, w_packed, s_w, 0, w8a8::W_INT4, y, y_dtype, M, N, K, ldy, stream);
}

// Validation shared by the split-K query and call: weight_bits / group_size as for w8a8_linear.
static int check_split_kind(const char *fn, int weight_bits, int group_size) {
    if (weight_bits != 8 && weight_bits != 4)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: weight_bits must be 8 or 4", fn);
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: group_size must be 0, 64 or 128", fn);
    return W8A8_OK;
}

static w8a8::SplitPlan current_split_plan(const w8a8::GemmProblem &p) {
    return w8a8::splitk_plan(p, g_force_cfg.load(std::memory_order_relaxed),
                             g_force_slices.load(std::memory_order_relaxed));
}

int w8a8_linear(const void *x, int x_dtype, int64_t ldx, const void *w, const float *s_w, int weight_bits,
                int group_size, int8_t *x_q, float *s_x, void *y, int y_dtype, int64_t M, int64_t N, int64_t K,
                int64_t ldy, void *stream) {
    const char *fn = "w8a8_linear";
    if (x_dtype != W8A8_F16 && x_dtype != W8A8_BF16)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: x_dtype must be F16 or BF16", fn);
    if (weight_bits != 8 && weight_bits != 4)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: weight_bits must be 8 or 4", fn);
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: group_size must be 0, 64 or 128", fn);
    if (y_dtype == W8A8_I32)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: y_dtype must be F16, BF16 or F32", fn);
    if (ldx < K || ldx % 8 != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: ldx = %lld must be >= K and a multiple of 8", fn,
                    (long long)ldx);
    int rc = check_gemm(fn, x_q, s_x, w, s_w, group_size, y, y_dtype, M, N, K, ldy, group_size != 0);
    if (rc != W8A8_OK) return rc;
    if (M > 0 && (!x || !aligned16(x)))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: x must be a non-null 16-byte aligned pointer", fn);
    if ((rc = check_device()) != W8A8_OK) return rc;
    if (M == 0) return ok();
    const int wkind = weight_bits == 4 ? w8a8::W_INT4 : w8a8::W_INT8;
    w8a8::GemmProblem p = make_problem(x_q, s_x, w, s_w, group_size, wkind, y, y_dtype, M, N, K, ldy);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int force = g_force_cfg.load(std::memory_order_relaxed);
    if (force < 0) {
        p.x = x;
        p.ldx = ldx;
        p.x_bf16 = x_dtype == W8A8_BF16 ? 1 : 0;
        p.xq_out = x_q;
        p.sx_out = s_x;
        const hipError_t e = w8a8::launch_linear_small(p, st);
        if (e != hipErrorNotSupported) return launched(e, fn);
        p.x = nullptr;
        p.xq_out = nullptr;
        p.sx_out = nullptr;
    }
    hipError_t e = w8a8::launch_quantize_per_token(x, x_dtype == W8A8_BF16, ldx, (int)M, (int)K, x_q, s_x, st);
    if (e != hipSuccess) return launched(e, fn);
    return launched(w8a8::launch_gemm(p, force, st), fn);
}

int int8_mv(const void *x, int x_dtype, int64_t ldx, const int8_t *w_q, const float *s_w, int group_size, void *y,
            int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy, void *stream) {
    const char *fn = "int8_mv";
    if (x_dtype != W8A8_F16 && x_dtype != W8A8_BF16)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: x_dtype must be F16 or BF16", fn);
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: group_size must be 0, 64 or 128", fn);
    if (y_dtype != W8A8_F16 && y_dtype != W8A8_BF16 && y_dtype != W8A8_F32)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: y_dtype must be F16, BF16 or F32", fn);
    if (M < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: M = %lld < 0", fn, (long long)M);
    if (M > 16) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: M = %lld > 16 (decode batches only)", fn, (long long)M);
    if (N > INT32_MAX || K > INT32_MAX || N * K > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    if (N < 16 || N % 16 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: N = %lld must be a positive multiple of 16", fn, (long long)N);
    if (K < 128 || K % 128 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: K = %lld must be a positive multiple of 128", fn, (long long)K);
    if (ldx < K || ldx % 8 != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: ldx = %lld must be >= K and a multiple of 8", fn, (long long)ldx);
    if (ldy < N || ldy % 4 != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: ldy = %lld must be >= N and a multiple of 4", fn, (long long)ldy);
    if (M > 0) {
        if (!x || !w_q || !s_w || !y) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
        if (!aligned16(x) || !aligned16(w_q) || !aligned16(s_w) || !aligned16(y))
            return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    }
    int rc = check_device();
    if (rc != W8A8_OK) return rc;
    if (M == 0) return ok();
    w8a8::GemmProblem p = make_problem(nullptr, nullptr, w_q, s_w, group_size, w8a8::W_INT8, y, y_dtype, M, N, K, ldy);
    p.x = x;
    p.ldx = ldx;
    p.x_bf16 = x_dtype == W8A8_BF16 ? 1 : 0;
    const hipError_t e = w8a8::launch_mv(p, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: shape does not fit the kernel's LDS plan", fn);
    return launched(e, fn);
}

namespace {

static int check_sdpa(const char *fn, int dtype, int o_dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t Ncap,
               int64_t D, float scale) {
    if (dtype != W8A8_F16 && dtype != W8A8_BF16)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: dtype must be F16 or BF16", fn);
    if (o_dtype != W8A8_F16 && o_dtype != W8A8_BF16 && o_dtype != W8A8_F32)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: o_dtype must be F16, BF16 or F32", fn);
    if (B < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: B = %lld < 0", fn, (long long)B);
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: Hq must be a positive multiple of Hkv", fn);
    if (Hq / Hkv > 16) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: Hq / Hkv = %lld > 16", fn, (long long)(Hq / Hkv));
    if (D != 64 && D != 128) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: D = %lld must be 64 or 128", fn, (long long)D);
    if (N < 1 || Ncap < N) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: need 1 <= N <= Ncap", fn);
    if (!(scale > 0.0f) || !(scale < INFINITY))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: scale must be positive and finite", fn);
    if (B > INT32_MAX || Hq > INT32_MAX || Ncap > INT32_MAX || B * Hkv * Ncap * D > ((int64_t)1 << 40))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "%s: sizes too large", fn);
    return W8A8_OK;
}

}  // namespace

int64_t sdpa_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D) {
    const int rc = check_sdpa("sdpa_decode_workspace", W8A8_F16, W8A8_F16, B, Hq, Hkv, N, N, D, 1.0f);
    if (rc != W8A8_OK) return -(int64_t)rc;
    ok();
    if (B == 0) return 0;
    return w8a8::sdpa_workspace_bytes((int)B, (int)Hq, (int)Hkv, (int)N, (int)D);
}

int sdpa_decode(const void *q, const void *k, const void *v, int dtype, void *o, int o_dtype, int64_t B, int64_t Hq,
                int64_t Hkv, int64_t N, int64_t Ncap, int64_t D, float scale, void *workspace, int64_t workspace_bytes,
                void *stream) {
    const char *fn = "sdpa_decode";
    int rc = check_sdpa(fn, dtype, o_dtype, B, Hq, Hkv, N, Ncap, D, scale);
    if (rc != W8A8_OK) return rc;
    if (workspace_bytes < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: workspace_bytes < 0", fn);
    if (workspace && !aligned16(workspace))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
    if (B > 0) {
        if (!q || !k || !v || !o) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
            return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    }
    if ((rc = check_device()) != W8A8_OK) return rc;
    if (B == 0) return ok();
    return launched(w8a8::launch_sdpa_decode(q, k, v, dtype == W8A8_BF16, o, o_dtype, (int)B, (int)Hq, (int)Hkv, (int)N,
                                             (int)Ncap, (int)D, scale, workspace, workspace_bytes,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

int sdpa_decode_autotune(const void *q, const void *k, const void *v, int dtype, void *o, int o_dtype, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t N, int64_t Ncap, int64_t D, float scale, void *workspace,
                         int64_t workspace_bytes, void *stream, int *slices_out) {
    const char *fn = "sdpa_decode_autotune";
    int rc = check_sdpa(fn, dtype, o_dtype, B, Hq, Hkv, N, Ncap, D, scale);
    if (rc != W8A8_OK) return rc;
    if (B < 1) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: B must be at least 1", fn);
    if (workspace_bytes < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: workspace_bytes < 0", fn);
    if (workspace && !aligned16(workspace))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
    if (!q || !k || !v || !o) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: pointers must be 16-byte aligned", fn);
    if ((rc = check_device()) != W8A8_OK) return rc;
    return launched(w8a8::sdpa_autotune(q, k, v, dtype == W8A8_BF16, o, o_dtype, (int)B, (int)Hq, (int)Hkv, (int)N,
                                        (int)Ncap, (int)D, scale, workspace, workspace_bytes,
                                        static_cast<hipStream_t>(stream), slices_out),
                    fn);
}

int sdpa_decode_tuned_slices(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D) {
    const char *fn = "sdpa_decode_tuned_slices";
    const int rc = check_sdpa(fn, dtype, W8A8_F16, B, Hq, Hkv, N, N, D, 1.0f);
    if (rc != W8A8_OK) return -rc;
    ok();
    return w8a8::sdpa_tuned_slices(dtype == W8A8_BF16, (int)B, (int)Hq, (int)Hkv, (int)N, (int)D);
}

int64_t w8a8_gemm_splitk_workspace(int weight_bits, int group_size, int y_dtype, int64_t M, int64_t N,
                                   int64_t K) {
    const char *fn = "w8a8_gemm_splitk_workspace";
    int rc = check_split_kind(fn, weight_bits, group_size);
    if (rc == W8A8_OK) rc = check_gemm_shape(fn, group_size, y_dtype, M, N, K, N, group_size != 0);
    if (rc != W8A8_OK) return -(int64_t)rc;
    ok();
    if (M == 0) return 0;
    const int wkind = weight_bits == 4 ? w8a8::W_INT4 : w8a8::W_INT8;
    const w8a8::GemmProblem p = make_problem(nullptr, nullptr, nullptr, nullptr, group_size, wkind, nullptr, y_dtype,
                                             M, N, K, N);
    return w8a8::splitk_workspace_bytes(p, current_split_plan(p));
}

int w8a8_gemm_splitk(const int8_t *x_q, const float *s_x, const void *w, const float *s_w, int weight_bits,
                     int group_size, void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                     void *workspace, int64_t workspace_bytes, void *stream) {
    const char *fn = "w8a8_gemm_splitk";
    int rc = check_split_kind(fn, weight_bits, group_size);
    if (rc != W8A8_OK) return rc;
    rc = check_gemm(fn, x_q, s_x, w, s_w, group_size, y, y_dtype, M, N, K, ldy, group_size != 0);
    if (rc != W8A8_OK) return rc;
    if (workspace_bytes < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: workspace_bytes < 0", fn);
    if (workspace && !aligned16(workspace))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
    if ((rc = check_device()) != W8A8_OK) return rc;
    if (M == 0) return ok();
    const int wkind = weight_bits == 4 ? w8a8::W_INT4 : w8a8::W_INT8;
    w8a8::GemmProblem p = make_problem(x_q, s_x, w, s_w, group_size, wkind, y, y_dtype, M, N, K, ldy);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const w8a8::SplitPlan plan = current_split_plan(p);
    const int64_t need = w8a8::splitk_workspace_bytes(p, plan);
    if (plan.slices > 1 && workspace && workspace_bytes >= need) {
        p.ws = workspace;
        return launched(w8a8::launch_gemm_splitk(p, plan, st), fn);
    }
    return launched(w8a8::launch_gemm(p, g_force_cfg.load(std::memory_order_relaxed), st), fn);
}

int w8a8_gemm_splitk_noalloc(const int8_t *x_q, const float *s_x, const void *w, const float *s_w, int weight_bits,
                             int group_size, void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                             void *stream) {
    const char *fn = "w8a8_gemm_splitk_noalloc";
    int rc = check_split_kind(fn, weight_bits, group_size);
    if (rc != W8A8_OK) return rc;
    rc = check_gemm(fn, x_q, s_x, w, s_w, group_size, y, y_dtype, M, N, K, ldy, group_size != 0);
    if (rc != W8A8_OK) return rc;
    if ((rc = check_device()) != W8A8_OK) return rc;
    if (M == 0) return ok();
    const int wkind = weight_bits == 4 ? w8a8::W_INT4 : w8a8::W_INT8;
    w8a8::GemmProblem p = make_problem(x_q, s_x, w, s_w, group_size, wkind, y, y_dtype, M, N, K, ldy);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const w8a8::SplitPlan plan = current_split_plan(p);
    if (plan.slices > 1) {
        const int64_t need = w8a8::splitk_workspace_bytes(p, plan);
        if (need > w8a8::kSplitScratchBytes)
            return fail(W8A8_ERR_UNSUPPORTED_SHAPE,
                        "%s: the split plan (%d slices) needs %lld bytes of scratch, more than the %lld bytes this "
                        "call holds per device; use w8a8_gemm_splitk with a workspace",
                        fn, plan.slices, (long long)need, (long long)w8a8::kSplitScratchBytes);
        void *ws = nullptr;
        const hipError_t e = w8a8::splitk_scratch(&ws);
        if (e != hipSuccess) return fail(W8A8_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
        p.ws = ws;
        return launched(w8a8::launch_gemm_splitk(p, plan, st), fn);
    }
    return launched(w8a8::launch_gemm(p, g_force_cfg.load(std::memory_order_relaxed), st), fn);
}

int w8a8_debug_clock_probe(uint64_t *out, void *stream) {
    const char *fn = "w8a8_debug_clock_probe";
    if (!out || !aligned16(out)) return fail(W8A8_ERR_INVALID_ARGUMENT, "%s: out must be a 16-byte aligned pointer", fn);
    const int rc = check_device();
    if (rc != W8A8_OK) return rc;
    return launched(w8a8::launch_clock_probe(out, 1024, static_cast<hipStream_t>(stream)), fn);
}

int w8a8_debug_force_splitk(int slices) {
    if (slices < -1 || slices == 0 || slices > 4096) return -W8A8_ERR_INVALID_ARGUMENT;
    g_force_slices.store(slices, std::memory_order_relaxed);
    return W8A8_OK;
}

}  // extern "C"
