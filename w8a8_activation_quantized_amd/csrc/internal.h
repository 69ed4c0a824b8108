// Internal launcher interface between the C-ABI layer (abi.hip) and the kernel
// translation units. Arguments reaching these launchers are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

enum OutType { OUT_F16 = 0, OUT_BF16 = 1, OUT_F32 = 2, OUT_I32 = 3 };
enum WeightKind { W_INT8 = 0, W_INT4 = 1 };

struct GemmProblem {
    const int8_t *xq;  // [M, K]
    const float *sx;   // [M]
    const void *wq;    // int8 [N, K] or packed uint8 [N, K/2]
    const float *sw;   // [N] (per-channel) or [N, K/gs]
    void *y;           // [M, N], row stride ldy
    int64_t ldy;
    int M, N, K;
    int gs;            // 0 = per-channel, else 64 | 128
    int wkind;         // WeightKind
    int out;           // OutType
    int y_rows16;      // 1 if y and the start of every output row are 16-byte aligned
    // fused small-M layer (activation quantization inside the GEMV kernel): x is read in
    // place of xq / sx, and workgroup 0 writes the codes and scales it computes
    const void *x;     // [M, K] fp16 / bf16, row stride ldx elements; null when unfused
    int64_t ldx;
    int x_bf16;
    int8_t *xq_out;    // [M, K]
    float *sx_out;     // [M]
    // split-K: K is cut into ksplit slices of whole 128-value K-tiles; slice s writes its
    // partial result to ws + s * M * N ([M, N], row stride N: int32 sums for per-channel and
    // I32 output, fp32 group folds for per-group); 1 and null for the single-pass kernels
    int ksplit;
    void *ws;
};

// Activation quantization (fp16 / bf16 rows -> int8 + fp32 scale).
hipError_t launch_quantize_per_token(const void *x, bool bf16, int64_t ldx, int M, int K,
                                     int8_t *xq, float *sx, hipStream_t stream);
hipError_t launch_rmsnorm_quantize(const void *x, bool x_bf16, int64_t ldx, const void *g, bool g_bf16, float eps,
                                   int M, int K, int8_t *xq, float *sx, hipStream_t stream);

// SwiGLU producer: codes and per-token scale of h = silu(gate) * up (fp16 / bf16 rows of I
// values, row strides ldg / ldu elements).
hipError_t launch_swiglu_quantize(const void *gate, int64_t ldg, const void *up, int64_t ldu, bool bf16, int M, int I,
                                  int8_t *xq, float *sx, hipStream_t stream);

// Offline weight quantization.
hipError_t launch_quantize_weight(const float *W, int N, int K, int bits, int gs, void *wq,
                                  float *sw, hipStream_t stream);
// quantize_weight with each run's magnitude from the pct-th percentile of |W| (pct in (0, 100];
// 100 is the maximum, i.e. launch_quantize_weight).
hipError_t launch_quantize_weight_clipped(const float *W, int N, int K, int bits, int gs, float pct, void *wq,
                                          float *sw, hipStream_t stream);

// GEMM + fused dequant. `force_cfg` < 0 lets the launcher choose by shape.
hipError_t launch_gemm(const GemmProblem &p, int force_cfg, hipStream_t stream);
// The whole layer for small M in one kernel (p.x set). Returns hipErrorNotSupported without
// launching when the shape does not fit it; the caller then quantizes and runs launch_gemm.
hipError_t launch_linear_small(const GemmProblem &p, hipStream_t stream);

// Decode matrix-vector product without activation quantization: y = x . (w_q * s_w)^T from
// fp16 / bf16 x (p.x, p.ldx, p.x_bf16), int8 weights, per channel or per group (p.gs);
// 1 <= M <= 16, K % 128 == 0. hipErrorNotSupported when the LDS plan does not fit.
hipError_t launch_mv(const GemmProblem &p, hipStream_t stream);

// Decode-step attention (one query token per head, grouped KV heads). q [B, Hq, D]; k, v
// [B, Hkv, Ncap, D] (first N rows used); fp16 or bf16; o [B, Hq, D] of out. Splits the keys
// over sdpa_slices(...) workgroups per KV head when ws holds sdpa_workspace_bytes(...), else
// runs one slice.
// The slice count is the autotuner's for this size class when it has run on this device
// (sdpa_autotune), else a fixed rule (sdpa_slices); the workspace size covers every count
// the autotuner may choose.
int sdpa_slices(int B, int Hkv, int N);
int64_t sdpa_workspace_bytes(int B, int Hq, int Hkv, int N, int D);
hipError_t launch_sdpa_decode(const void *q, const void *k, const void *v, bool bf16, void *o, int out, int B, int Hq,
                              int Hkv, int N, int Ncap, int D, float scale, void *ws, int64_t ws_bytes,
                              hipStream_t stream);
int sdpa_tuned_slices(bool bf16, int B, int Hq, int Hkv, int N, int D);
hipError_t sdpa_autotune(const void *q, const void *k, const void *v, bool bf16, void *o, int out, int B, int Hq,
                         int Hkv, int N, int Ncap, int D, float scale, void *ws, int64_t ws_bytes, hipStream_t stream,
                         int *best_out);

// Measurement aid: `blocks` workgroups each store, at out[4 b .. 4 b + 2], where they ran
// (XCC_ID << 32 | HW_ID), the shader-clock counter and the 100 MHz counter.
hipError_t launch_clock_probe(uint64_t *out, int blocks, hipStream_t stream);

// Compute units of the current device (cached after the first call; 256 when no device
// answers, which is the MI355X count).
int num_cus();

// Number of GEMM tile configurations selectable via force_cfg.
int gemm_num_configs();

// Split-K, for problems whose output tiles are too few to occupy the chip (narrow N, long K).
struct SplitPlan {
    int cfg;     // tile configuration of the slice kernel
    int slices;  // 1: no split (run launch_gemm)
};
// The plan for p (force_cfg / force_slices >= 0 override the automatic choice; a forced
// plan that the problem cannot take gives slices = 1).
SplitPlan splitk_plan(const GemmProblem &p, int force_cfg, int force_slices);
// Workspace bytes of a plan: slices * M * N * 4 (0 when slices == 1).
int64_t splitk_workspace_bytes(const GemmProblem &p, const SplitPlan &plan);
// Runs the slices into p.ws, then one kernel that adds them in slice order and writes y.
// Requires plan.slices > 1, p.ws with splitk_workspace_bytes(p, plan) bytes.
hipError_t launch_gemm_splitk(GemmProblem p, const SplitPlan &plan, hipStream_t stream);

// Size of the per-device scratch array of the allocation-free split-K call.
constexpr int64_t kSplitScratchBytes = (int64_t)32 << 20;
// Device address of the current device's scratch array (looked up once per device with
// hipGetSymbolAddress, then cached). Allocates nothing.
hipError_t splitk_scratch(void **ptr);

}  // namespace w8a8
