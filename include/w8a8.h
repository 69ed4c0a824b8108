/*
 * w8a8.h -- C ABI of libw8a8: fused per-token activation quantization, int8 GEMM
 * and dequantization (W8A8 / W4A8 linear layers) for AMD Instinct MI355X (gfx950).
 *
 * The method (Cider project pages):
 *  - juejin post "在Mac上跑大模型，MLX 不是终点", section "W8A8 对称量化：Cider 的选择":
 *    per-token symmetric scale s_x = max|x| / 127, x_q = round(x / s_x) clamped to
 *    [-128, 127]; y = (x_q . w_q) * s_x * s_w, dequantization fused into the GEMM store.
 *  - same post, "INT8 TensorOps 内核设计": int8 x int8 products accumulate in int32;
 *    "三种量化粒度的实现": weight scales per output channel, or per group of 64/128
 *    elements along K (a segmented multiplication).
 *  - Cider README, sections "模式" and "量化": W4A8 weights are symmetric int4 with
 *    zero point 8, packed two per uint8; "Metal Kernel 流水线": quantize_per_token
 *    then the fused int8 matmul with dequantization; for W4A8 the int4 -> int8
 *    unpack happens inside the GEMM's operand load.
 *
 * Rounding: "round" is read as IEEE round-half-to-even of the correctly rounded
 * fp32 quotient x / s (a true fp32 division). A row or group whose max is 0 has
 * scale 0 and all-zero codes.
 *
 * Conventions for every entry point below:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates and frees nothing and keeps no per-call state (reentrant). The one
 *    piece of device memory it holds is the static scratch array of
 *    w8a8_gemm_splitk_noalloc (see there).
 *  - All tensors are row-major with the last index contiguous. Base pointers must
 *    be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream) on the current device.
 *    Calls enqueue work and return; results are valid once the caller has
 *    synchronized with the stream.
 *  - Arguments are validated on the host BEFORE anything is enqueued; on any
 *    non-OK return nothing was enqueued (except W8A8_ERR_HIP, where the launch
 *    itself failed). w8a8_last_error() then gives a thread-local message.
 *  - Device faults surface at the caller's next synchronization (HIP semantics).
 *  - M = 0 (an empty batch) is valid and enqueues nothing.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W8A8_OK = 0,
    W8A8_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size/stride/alignment, bad enum */
    W8A8_ERR_UNSUPPORTED_DEVICE = 2, /* no device, not gfx950, or W8A8_FORCE_UNAVAILABLE=1 */
    W8A8_ERR_UNSUPPORTED_SHAPE = 3, /* shape outside the documented constraints */
    W8A8_ERR_HIP = 4 /* a HIP runtime call or kernel launch failed */
} w8a8_status;

typedef enum {
    W8A8_F16 = 0,
    W8A8_BF16 = 1,
    W8A8_F32 = 2,
    W8A8_I32 = 3 /* GEMM output only: the raw int32 accumulator sum_k x_q*w_q (testing) */
} w8a8_dtype;

/* 1 iff `device` exists, is a gfx950 GPU, and W8A8_FORCE_UNAVAILABLE is not set to 1.
 * Mirrors the pages' is_available() (README "条件编译"): callers fall back when 0. */
int w8a8_is_available(int device);

/* Static string for a status code. */
const char *w8a8_status_string(int status);

/* Thread-local detail for the last non-OK return on this thread ("" if none). */
const char *w8a8_last_error(void);

/* Library ABI version (increments on incompatible changes). */
int w8a8_abi_version(void);

/*
 * quantize_per_token -- online per-token activation quantization
 * (juejin post, "W8A8 对称量化：Cider 的选择"; README "Metal Kernel 流水线" step 1).
 *   x       [M, K] fp16 or bf16 (x_dtype = W8A8_F16 | W8A8_BF16), row stride ldx elements
 *   x_q     [M, K] int8 output, row stride K
 *   s_x     [M]    fp32 output: s_x[m] = max_k |x[m,k]| / 127
 * Codes: x_q = clamp(rne(x / s_x), -128, 127); 0 where s_x == 0.
 * Constraints: M >= 0, K >= 8, K % 8 == 0, ldx >= K, ldx % 8 == 0. Inputs finite.
 */
int quantize_per_token(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                       int8_t *x_q, float *s_x, void *stream);

/*
 * rmsnorm_quantize -- the producer of a linear layer's input writes the codes itself, so
 * the per-token quantization (README "Metal Kernel 流水线" step 1; juejin post, "W8A8 对称量化":
 * it must stay cheap) needs no pass of its own. The producer is RMSNorm with weight gamma:
 *     n[m,k] = x[m,k] * gamma[k] / sqrt(mean_k x[m,k]^2 + eps).
 * The row factor cancels in the per-token quantization of n, so the outputs are
 *   x_q   [M, K] int8, row stride K: the per-token codes of u = x * gamma (one fp32 multiply
 *         per element), exactly as quantize_per_token would compute them for u
 *   s_x   [M] fp32: (max_k |u[m,k]| / 127) / sqrt(mean_k x[m,k]^2 + eps); 0 for a zero row
 * so s_x[m] * x_q[m,k] approximates n[m,k] within half a quantization step, and x_q, s_x feed
 * w8a8_gemm_pc / w8a8_gemm_pg / w4a8_gemm_pg as the outputs of quantize_per_token do. The
 * codes are exact; s_x carries the fp32 rounding of the row's sum of squares.
 *   x      [M, K] fp16 or bf16 (x_dtype), row stride ldx elements
 *   gamma  [K] fp16 or bf16 (gamma_dtype)
 *   eps    finite, >= 0
 * Constraints: M >= 0, K >= 8, K % 8 == 0, ldx >= K, ldx % 8 == 0, all pointers 16-byte
 * aligned. Inputs finite; the sum of x^2 and every product x * gamma finite in fp32.
 */
int rmsnorm_quantize(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const void *gamma,
                     int gamma_dtype, float eps, int8_t *x_q, float *s_x, void *stream);

/*
 * swiglu_quantize -- the producer of a gated MLP's down-projection input writes that input's
 * codes itself, so the per-token quantization (README "Metal Kernel 流水线" step 1; juejin
 * post, "W8A8 对称量化": it must stay cheap) needs no pass of its own. The input is
 * h = silu(gate) * up, gate and up being the two halves of the gate/up projection's output:
 *   e = exp(-g) (the fixed fp32 evaluation below);  s = g / (1 + e) (IEEE);  h = s * u  (fp32)
 *   x_q [M, I] int8, row stride I, and s_x [M] fp32: the per-token quantization of h exactly as
 *   quantize_per_token computes it (h is not rounded to fp16 / bf16 first).
 * exp(x) is evaluated as: x clamped to [-87, 88]; k = rint(x * RN(log2 e)); r = fma(-k, RN(ln 2),
 * x), r = fma(-k, RN(ln 2 - RN(ln 2)), r); p = the Taylor polynomial of degree 7 in r with the
 * coefficients RN(1 / n!), by Horner's rule with fmas; result p * 2^k (RN = fp32 rounding).
 * With that, the codes and scales are bit-reproducible; h is within 2^-20 relative of
 * silu(g) * u for g >= -87.
 *   gate, up  [M, I] fp16 or bf16 (dtype), row strides ldg, ldu elements (they may be views
 *             into one [M, 2 I] array)
 * Constraints: M >= 0, I >= 8, I % 8 == 0, ldg, ldu >= I and multiples of 8, all pointers
 * 16-byte aligned. Inputs finite, and every h finite in fp32 (bf16 gate and up can overflow it).
 */
int swiglu_quantize(const void *gate, const void *up, int dtype, int64_t M, int64_t I, int64_t ldg, int64_t ldu,
                    int8_t *x_q, float *s_x, void *stream);

/*
 * quantize_weight -- offline min-max weight quantization (README "说明": min-max
 * by default; "量化": symmetric int8 per channel / per group, int4 zero point 8).
 *   W      [N, K] fp32 (row n = output channel n)
 *   bits 8, group_size 0      : w_q int8 [N, K],        s_w [N]       = max_k |W[n,:]| / 127
 *   bits 8, group_size 64|128 : w_q int8 [N, K],        s_w [N, K/gs] = max |W[n, group]| / 127
 *   bits 4, group_size 64|128 : w_q uint8 [N, K/2],     s_w [N, K/gs] = max |W[n, group]| / 7
 *   bits 4, group_size 0      : w_q uint8 [N, K/2],     s_w [N]       = max_k |W[n,:]| / 7
 *       (the README's per-column INT4, section "量化": one scale per output channel)
 *       int4 codes q = clamp(rne(W / s), -8, 7) stored as u = q + 8, byte j of row n
 *       = u[n, 2j] | u[n, 2j+1] << 4 (even k in the low nibble).
 * Constraints: N >= 1, K >= 64, K % 64 == 0, K % group_size == 0. Inputs finite.
 */
int quantize_weight(const float *W, int64_t N, int64_t K, int bits, int group_size, void *w_q,
                    float *s_w, void *stream);

/*
 * quantize_weight_clipped -- quantize_weight with a clipped scale (Cider README "说明": the
 * scale comes from min-max by default, or from a percentile of the weights, clip_percentile).
 * Per run (row for group_size 0, else group of group_size along K) the magnitude used in
 * place of max|W| is the clip_percentile-th percentile of |W| over the run, with linear
 * interpolation between order statistics: with u_0 <= ... <= u_{n-1} the sorted
 * magnitudes, h = (clip_percentile * (n - 1)) / 100 and i = floor(h) in fp64,
 *   a = u_{n-1} if i >= n - 1, else (float)(u_i + (h - i) * (u_{i+1} - u_i)) (fp64, one rounding)
 * then s = a / 127 (int8) or a / 7 (int4) and the codes as quantize_weight computes them, so
 * weights beyond the percentile saturate at the clamp. clip_percentile = 100 gives exactly
 * quantize_weight's output.
 * Constraints: those of quantize_weight, and 0 < clip_percentile <= 100.
 */
int quantize_weight_clipped(const float *W, int64_t N, int64_t K, int bits, int group_size,
                            float clip_percentile, void *w_q, float *s_w, void *stream);

/*
 * w8a8_gemm_pc -- int8 GEMM with per-channel dequant fused into the store
 * (juejin post, "W8A8 对称量化" and "INT8 TensorOps 内核设计"; README "量化":
 * C = C_int32 * s_act * s_weight).
 *   x_q [M, K] int8, s_x [M] fp32, w_q [N, K] int8, s_w [N] fp32
 *   y   [M, N] of y_dtype with row stride ldy elements:
 *       acc = sum_k x_q[m,k] * w_q[n,k]  (exact int32)
 *       y   = rne_out((fp32(acc) * s_x[m]) * s_w[n])       (fp32 arithmetic)
 *       W8A8_I32 writes acc itself.
 * Constraints: M >= 0, N >= 16, N % 16 == 0, K >= 64, K % 64 == 0, ldy >= N, ldy % 4 == 0.
 */
int w8a8_gemm_pc(const int8_t *x_q, const float *s_x, const int8_t *w_q, const float *s_w,
                 void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                 void *stream);

/*
 * w8a8_gemm_pg -- int8 GEMM with per-group weight scales (juejin post
 * "三种量化粒度的实现": each K-group has its own scale; dequant is segmented).
 *   s_w [N, G] fp32 with G = K / group_size, group_size in {64, 128}
 *   acc_g = sum over k in group g of x_q[m,k] * w_q[n,k]  (exact int32)
 *   t = 0; for g = 0..G-1: t = fma(fp32(acc_g), s_w[n,g], t);  y = rne_out(t * s_x[m])
 *   W8A8_I32 writes sum_g acc_g (= the full integer product).
 * Constraints: as w8a8_gemm_pc, plus K % group_size == 0.
 */
int w8a8_gemm_pg(const int8_t *x_q, const float *s_x, const int8_t *w_q, const float *s_w,
                 int group_size, void *y, int y_dtype, int64_t M, int64_t N, int64_t K,
                 int64_t ldy, void *stream);

/*
 * w4a8_gemm_pg -- W4A8 GEMM: int4 weights packed two per byte, unpacked to int8
 * inside the GEMM's weight-tile load (README "Metal Kernel 流水线", W4A8 note),
 * then the per-group path of w8a8_gemm_pg on the codes q = u - 8.
 *   w_packed [N, K/2] uint8 (layout of quantize_weight with bits = 4)
 *   s_w      [N, K/group_size] fp32, group_size in {64, 128}
 * Constraints: as w8a8_gemm_pg.
 */
int w4a8_gemm_pg(const int8_t *x_q, const float *s_x, const uint8_t *w_packed, const float *s_w,
                 int group_size, void *y, int y_dtype, int64_t M, int64_t N, int64_t K,
                 int64_t ldy, void *stream);

/*
 * w4a8_gemm_pc -- W4A8 GEMM with per-column int4 weights (Cider README "量化": W4A8 weights are
 * symmetric INT4, zero point 8, per column): one scale per output channel, the int4 codes
 * unpacked inside the GEMM's weight-tile load as for w4a8_gemm_pg, then the per-channel path:
 *   w_packed [N, K/2] uint8 (quantize_weight with bits = 4, group_size = 0), s_w [N] fp32
 *   acc = sum_k x_q[m,k] * q[n,k]  (q = u - 8, exact int32);  y = rne_out((fp32(acc) * s_x[m]) * s_w[n])
 *   W8A8_I32 writes acc itself.
 * Constraints: as w8a8_gemm_pc.
 */
int w4a8_gemm_pc(const int8_t *x_q, const float *s_x, const uint8_t *w_packed, const float *s_w, void *y,
                 int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy, void *stream);

/*
 * w8a8_linear -- the whole layer in one call: per-token activation quantization of x
 * followed by the int8 GEMM with fused dequant (juejin post, "INT8 TensorOps 内核设计":
 * quantize_per_token, then matmul_fused_dequant). The weight arguments select the GEMM:
 *   weight_bits 8, group_size 0      -> w8a8_gemm_pc (w = w_q [N, K] int8, s_w [N])
 *   weight_bits 8, group_size 64|128 -> w8a8_gemm_pg (s_w [N, K/group_size])
 *   weight_bits 4, group_size 64|128 -> w4a8_gemm_pg (w = w_packed [N, K/2])
 *   weight_bits 4, group_size 0      -> w4a8_gemm_pc (w = w_packed [N, K/2], s_w [N])
 *   x [M, K] fp16 or bf16 (x_dtype), row stride ldx elements (ldx >= K, ldx % 8 == 0).
 *   x_q [M, K] int8 and s_x [M] fp32 (caller-owned) receive the codes and scales exactly as
 *   quantize_per_token writes them; y [M, N] as for the GEMM calls (not W8A8_I32).
 * Results are bit-identical to quantize_per_token followed by the matching GEMM call for
 * per-channel weights. For M <= 16 one kernel does both steps (each workgroup quantizes
 * the rows it needs, saving the second launch); the per-group sum over a row's K range
 * may then be split differently, within the GEMM's fp32 tolerance. Larger M, or a
 * configuration forced with w8a8_debug_force_config, runs the two launches.
 * Constraints: those of quantize_per_token and of the selected GEMM call.
 */
int w8a8_linear(const void *x, int x_dtype, int64_t ldx, const void *w, const float *s_w,
                int weight_bits, int group_size, int8_t *x_q, float *s_x, void *y, int y_dtype,
                int64_t M, int64_t N, int64_t K, int64_t ldy, void *stream);

/*
 * int8_mv -- the decode path without activation quantization (Cider README "Metal Kernel
 * 流水线", decode: the int8 matrix-vector kernel dequantizes the weights on the fly; juejin
 * post "INT8 TensorOps 内核设计": seq_len = 1 takes a dedicated matrix-vector kernel).
 *   x    [M, K] fp16 or bf16 (x_dtype), row stride ldx elements, 1 <= M <= 16 (M = 0: no-op)
 *   w_q  [N, K] int8, s_w [N] (group_size 0) or [N, K / group_size] (64 | 128), as
 *        quantize_weight writes them with bits = 8
 *   y    [M, N] of y_dtype (F16, BF16 or F32), row stride ldy elements:
 *        y[m, n] = sum_k x[m, k] * (w_q[n, k] * s_w[n, k / group_size])
 *   evaluated with fp32 products and sums (the codes are converted exactly to the
 *   activation format; per channel the K-sum is scaled by s_w[n] at the end, per group each
 *   group's sum is folded in fp32, groups ascending within a K-segment), then rounded once
 *   to y_dtype. The fp32 sums follow no fixed order: results are within the fp32 evaluation
 *   bound (K + 2) * 2^-24 * sum_k |terms| of the exact value, plus the output rounding.
 * Constraints: N >= 16, N % 16 == 0, K >= 128, K % 128 == 0, ldx >= K, ldx % 8 == 0,
 * ldy >= N, ldy % 4 == 0; inputs finite.
 */
int int8_mv(const void *x, int x_dtype, int64_t ldx, const int8_t *w_q, const float *s_w, int group_size,
            void *y, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy, void *stream);

/*
 * Split-K form of the three GEMM calls, for problems whose output has too few tiles to
 * occupy the chip (narrow N with long K at M in the hundreds or low thousands): K is cut
 * into slices of whole 128-value K-tiles that run side by side, each writing its partial
 * result to a caller-provided workspace, and a second kernel adds the slices in slice order
 * and applies the dequantization of juejin post "W8A8 对称量化" (per-channel) or
 * "三种量化粒度的实现" (per-group).
 *
 * w8a8_gemm_splitk_workspace: bytes of workspace the split form uses for this problem,
 *   slices * M * N * 4; 0 when the library would not split it (M <= 16, K % 128 != 0, int4
 *   weights with per-channel scales or with W8A8_I32 output, or a single pass estimated
 *   faster). The value depends only on the arguments, the device's compute-unit count and
 *   the debug knobs below.
 *   Negative: -status for invalid arguments (the checks of the GEMM calls).
 *
 * w8a8_gemm_splitk: the GEMM selected as in w8a8_linear (weight_bits 8 / group_size 0:
 *   w8a8_gemm_pc; 8 / 64|128: w8a8_gemm_pg; 4 / 64|128: w4a8_gemm_pg, w = w_packed;
 *   4 / 0: w4a8_gemm_pc, which has no split form and always runs its single pass),
 *   same operands, layouts and constraints, plus
 *   workspace        device memory, 16-byte aligned, owned by the caller, not overlapping
 *                    any operand; contents on return are unspecified. It must stay
 *                    allocated until the stream has run the call; two calls in flight at
 *                    once need two workspaces.
 *   workspace_bytes  its size. With workspace NULL, or smaller than the query's value,
 *                    the call runs the single-pass kernels of the matching GEMM call.
 * Results: per-channel (and W8A8_I32) bit-identical to the matching GEMM call, since
 * int32 sums are exact in any order; per-group within the same fp32 tolerance, the group
 * terms being summed per slice and then across slices.
 */
int64_t w8a8_gemm_splitk_workspace(int weight_bits, int group_size, int y_dtype, int64_t M, int64_t N,
                                   int64_t K);
int w8a8_gemm_splitk(const int8_t *x_q, const float *s_x, const void *w, const float *s_w,
                     int weight_bits, int group_size, void *y, int y_dtype, int64_t M, int64_t N,
                     int64_t K, int64_t ldy, void *workspace, int64_t workspace_bytes,
                     void *stream);

/*
 * w8a8_gemm_splitk_noalloc -- w8a8_gemm_splitk for callers that cannot allocate device
 * memory (code under stream / graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the slices' partial results go to a scratch array that the library holds in
 * each device's memory from its first use there until the process ends (32 MiB per device,
 * a file-scope device array), so the call takes no workspace and allocates nothing.
 * Operands, layouts, constraints and results are those of w8a8_gemm_splitk with a
 * sufficient workspace (the same plan and kernels, so the same bits). When the plan for the
 * problem does not split, the single-pass kernels run and the scratch is not touched.
 * Errors: W8A8_ERR_UNSUPPORTED_SHAPE, with nothing enqueued, when the plan's partial results
 * need more than the 32 MiB scratch (slices * M * N * 4 bytes; w8a8_gemm_splitk_workspace
 * gives that size): call w8a8_gemm_splitk with a workspace instead.
 * Every call on one device shares that device's scratch: two calls whose executions
 * overlap on a device (different streams, no ordering between them) race on it and give
 * undefined results. Calls ordered on one stream are safe.
 */
int w8a8_gemm_splitk_noalloc(const int8_t *x_q, const float *s_x, const void *w, const float *s_w,
                             int weight_bits, int group_size, void *y, int y_dtype, int64_t M, int64_t N,
                             int64_t K, int64_t ldy, void *stream);

/*
 * sdpa_decode -- attention for one decode step (Cider README "优化 SDPA（解码注意力）": one
 * query token per head, no mask; the query heads that share a KV head are served together so
 * each K / V row is read once; long caches are split over workgroups and merged in a second
 * pass, two-pass FlashDecoding).
 *   q [B, Hq, D], k and v [B, Hkv, Ncap, D] of dtype (F16 or BF16), row-major; the first N
 *   rows of each head's cache are used. Query head h reads KV head h / (Hq / Hkv).
 *   o [B, Hq, D] of o_dtype (F16, BF16 or F32):
 *     o[b, h, :] = sum_n p_n v[b, h / G, n, :],  p = softmax_n(scale * q[b, h, :] . k[b, h / G, n, :])
 *   evaluated in fp32 (exact products on the matrix cores, fp32 sums, exp2 on pre-scaled
 *   scores) and rounded once to o_dtype.
 *   workspace / workspace_bytes: device memory for the per-slice partial results, at least
 *   sdpa_decode_workspace(B, Hq, Hkv, N, D) bytes (0 means one pass suffices; the size holds
 *   every slice count sdpa_decode_autotune may pick); NULL or less than the chosen count needs
 *   runs a single slice per KV head (correct, slower for long caches). Caller-owned, 16-byte
 *   aligned, contents unspecified on return; one per call in flight. The slice count is the
 *   autotuned one for this size class if sdpa_decode_autotune has run, else a fixed rule
 *   (about one workgroup per compute unit, at least 128 keys per slice).
 * Constraints: B >= 0 (0: no-op), Hq % Hkv == 0, Hq / Hkv <= 16, D in {64, 128},
 * 1 <= N <= Ncap, 0 < scale < inf (usually 1 / sqrt(D)); inputs finite.
 * sdpa_decode_workspace returns -status for invalid arguments.
 */
int64_t sdpa_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D);
int sdpa_decode(const void *q, const void *k, const void *v, int dtype, void *o, int o_dtype, int64_t B,
                int64_t Hq, int64_t Hkv, int64_t N, int64_t Ncap, int64_t D, float scale, void *workspace,
                int64_t workspace_bytes, void *stream);

/*
 * sdpa_decode_autotune -- the split's autotuning (Cider README "优化 SDPA（解码注意力）",
 * AutoTune: block sizes swept per GQA ratio, head count and sequence length, the fastest
 * cached). Runs sdpa_decode on the given tensors with each candidate number of key slices per
 * KV head -- one slice, and the fixed rule's count r times 1/4, 1/2, 1, 2 and 4, each slice at
 * least 128 keys, the partials within the workspace -- times each as a captured HIP graph of
 * 20 calls, replayed on a private stream (created and destroyed here, ordered after the work
 * already on `stream`), and records the fastest for (current device, dtype, B, Hq, Hkv, D,
 * N rounded up to a power of two) in a process-wide table, keeping the rule's count unless
 * another is at least 3 % faster; later sdpa_decode calls of that size class use it (at most
 * N / 128 slices at their N) instead of the rule. *slices_out (may be NULL) receives the count
 * chosen. Arguments as sdpa_decode (B >= 1); o holds the last launch's result; a workspace of
 * sdpa_decode_workspace(...) bytes fits every candidate. Returns after the timed launches have
 * finished: not for use under graph capture. The table is guarded by a mutex.
 * sdpa_decode_tuned_slices returns the recorded count for the size class of these arguments on
 * the current device, 0 if none, or -status for invalid arguments.
 */
int sdpa_decode_autotune(const void *q, const void *k, const void *v, int dtype, void *o, int o_dtype, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t N, int64_t Ncap, int64_t D, float scale, void *workspace,
                         int64_t workspace_bytes, void *stream, int *slices_out);
int sdpa_decode_tuned_slices(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D);

/*
 * Debug knob: force the number of K-slices of w8a8_gemm_splitk (-1 = automatic, 1 = never
 * split, n >= 2: n slices, at most K / 128). Combined with w8a8_debug_force_config a
 * configuration with a split form (per-channel 7, 12, 14; per-group 11, 12) is used for the
 * slices; forcing any other configuration runs the single-pass kernels. Returns W8A8_OK, or
 * -W8A8_ERR_INVALID_ARGUMENT for 0, < -1 or > 4096. Process-wide.
 */
int w8a8_debug_force_splitk(int slices);

/*
 * Measurement aid: enqueues 1024 small workgroups; workgroup b stores where it ran,
 * (XCC_ID << 32) | HW_ID (the XCD, and the compute unit, shader array and engine), the
 * shader-clock counter (s_memtime, counting at the current engine clock) and the constant
 * 100 MHz counter (s_memrealtime) to out[4 b], out[4 b + 1], out[4 b + 2] (out: device memory,
 * 4096 uint64, 16-byte aligned, caller-owned; out[4 b + 3] is not written). Two probes on
 * one stream around some work give the mean engine clock over it on each compute unit that
 * both visited: 100 MHz * (shader-clock difference) / (100 MHz counter difference).
 */
int w8a8_debug_clock_probe(uint64_t *out, void *stream);

/*
 * Debug knob: force the GEMM tile configuration (-1 = automatic choice by shape).
 * Every configuration computes identical results; tests use this to run each one.
 * Returns the number of configurations, or W8A8_ERR_INVALID_ARGUMENT (negated)
 * for an unknown id. Process-wide.
 */
int w8a8_debug_force_config(int config_id);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
