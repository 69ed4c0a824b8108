// Activation and weight quantization kernels for gfx950.
//
// Per-token symmetric int8 quantization (juejin post "在Mac上跑大模型，MLX 不是终点",
// section "W8A8 对称量化：Cider 的选择"): s = max|x| / 127, q = clamp(round(x / s)).
// "round" is IEEE round-half-to-even of the correctly rounded fp32 quotient x / s. The
// scale is one IEEE fp32 division per row; the per-element quotient is computed with a
// corrected reciprocal that gives the same value (see the activation section below).
// This file must never be built with fast-math, approximate division or flushed fp32
// denormals.
//
// Activation kernel layout: one wavefront per token row, 4 rows per 256-thread
// workgroup. Each lane loads 16-byte chunks (8 halves) at chunk index lane + 64*j,
// so every load instruction of the wave covers 1 KiB of contiguous row data. The
// row is cached in registers between the absmax pass and the quantize pass (up to
// CPL chunks per lane), so HBM sees exactly one read of x and one write of x_q.
// The absmax works on the magnitude bit patterns (bits & 0x7fff), which order
// like the magnitudes for finite fp16/bf16 values.
#include <cmath>
#include <type_traits>

#include "act_quant.h"
#include "internal.h"

namespace w8a8 {
namespace {

// One code: clamp(rne(v / s), lo, hi); 0 when s == 0 (IEEE division; offline weights).
__device__ __forceinline__ int quant_one(float v, float s, float lo, float hi) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

using namespace act;

// ---- activation quantization (arithmetic in act_quant.h) -------------------------------

template <bool BF16, bool FAST, int CPL>
__device__ __forceinline__ void quant_row_store(const uint4 (&cache)[CPL], const uint16_t *row, int8_t *qrow,
                                                int lane, int nch, float s, float r) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) *reinterpret_cast<uint2 *>(qrow + 8 * c) = quant8<BF16, FAST>(cache[j], s, r);
    }
    for (int c = lane + 64 * CPL; c < nch; c += 64)
        *reinterpret_cast<uint2 *>(qrow + 8 * c) =
            quant8<BF16, FAST>(*reinterpret_cast<const uint4 *>(row + 8 * c), s, r);
}

// Rows of at least this many values go to the workgroup-per-row kernel (measured on MI355X,
// x streamed from HBM: K = 10240, M = 4096: 21.3 against 26.2 us; K = 12288, M = 2048: 14.7
// against 17.6; K = 4096: 7.2 against 7.6; at K = 2560 four waves per row are slower than
// one, 8.8 against 8.3 us at M = 4096).
constexpr int kRowsPerWorkgroupK = 4096;
// Rows of 2048 .. 4095 values: a workgroup of two waves per row (M = 4096, K = 2560: 8.2
// against 8.4 us; M = 8192: 12.8 against 13.8 us); shorter rows keep a wave per row.
constexpr int kRowsPerPairK = 2048;

// CPL = chunks per lane kept in registers; rows with more chunks than 64*CPL take
// a second read pass for the remainder.
template <int CPL, bool BF16>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t *__restrict__ x,
                                                             int64_t ldx, int M, int K,
                                                             int8_t *__restrict__ xq,
                                                             float *__restrict__ sx) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const uint16_t *row = x + (int64_t)m * ldx;
    int8_t *qrow = xq + (int64_t)m * K;
    const int nch = K >> 3;

    uint4 cache[CPL];
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        int c = lane + 64 * j;
        cache[j] = c < nch ? *reinterpret_cast<const uint4 *>(row + 8 * c) : make_uint4(0, 0, 0, 0);
        m2 = absmax8(cache[j], m2);
    }
    for (int c = lane + 64 * CPL; c < nch; c += 64) m2 = absmax8(*reinterpret_cast<const uint4 *>(row + 8 * c), m2);
    uint32_t amax = m2.x > m2.y ? m2.x : m2.y;
    amax = wave_max_u32(amax);

    const float s = row_scale<BF16>(amax);
    if (lane == 0) sx[m] = s;
    if (s == 0.0f) {
        // all-zero row: zero codes
        for (int c = lane; c < nch; c += 64) *reinterpret_cast<uint2 *>(qrow + 8 * c) = make_uint2(0, 0);
        return;
    }
    if (s >= kMinFastScale) {
        const float r = 1.0f / s;
        quant_row_store<BF16, true, CPL>(cache, row, qrow, lane, nch, s, r);
    } else {
        quant_row_store<BF16, false, CPL>(cache, row, qrow, lane, nch, s, 0.f);
    }
}

// Codes of one row from the workgroup's threads (thread t: chunks t + NT j).
template <bool BF16, bool FAST, int CPT, int NT>
__device__ __forceinline__ void wg_row_store(const uint4 (&cache)[CPT], const uint16_t *row, int8_t *qrow, int tid,
                                             int nch, float s, float r) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + NT * j;
        if (c < nch) *reinterpret_cast<uint2 *>(qrow + 8 * c) = quant8<BF16, FAST>(cache[j], s, r);
    }
    for (int c = tid + NT * CPT; c < nch; c += NT)
        *reinterpret_cast<uint2 *>(qrow + 8 * c) = quant8<BF16, FAST>(*reinterpret_cast<const uint4 *>(row + 8 * c), s, r);
}

// Long rows: a row per 256-thread workgroup (thread t takes the chunks t + 256 j, up to CPT
// of them held in registers), the four waves' maxima combined through LDS; the same codes.
template <int CPT, bool BF16, int NT>
__global__ __launch_bounds__(NT) void quantize_rows_wg_kernel(const uint16_t *__restrict__ x, int64_t ldx, int K,
                                                               int8_t *__restrict__ xq, float *__restrict__ sx) {
    __shared__ uint32_t wmax[NT / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = blockIdx.x;
    const uint16_t *row = x + (int64_t)m * ldx;
    int8_t *qrow = xq + (int64_t)m * K;
    const int nch = K >> 3;

    uint4 cache[CPT];
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + NT * j;
        cache[j] = c < nch ? *reinterpret_cast<const uint4 *>(row + 8 * c) : make_uint4(0, 0, 0, 0);
        m2 = absmax8(cache[j], m2);
    }
    for (int c = tid + NT * CPT; c < nch; c += NT) m2 = absmax8(*reinterpret_cast<const uint4 *>(row + 8 * c), m2);
    uint32_t amax = wave_max_u32(m2.x > m2.y ? m2.x : m2.y);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) amax = max(amax, wmax[w]);

    const float s = row_scale<BF16>(amax);
    if (tid == 0) sx[m] = s;
    if (s == 0.0f) {
        for (int c = tid; c < nch; c += NT) *reinterpret_cast<uint2 *>(qrow + 8 * c) = make_uint2(0, 0);
        return;
    }
    if (s >= kMinFastScale)
        wg_row_store<BF16, true, CPT, NT>(cache, row, qrow, tid, nch, s, 1.0f / s);
    else
        wg_row_store<BF16, false, CPT, NT>(cache, row, qrow, tid, nch, s, 0.f);
}

template <bool BF16>
hipError_t launch_rows(const void *x, int64_t ldx, int M, int K, int8_t *xq, float *sx,
                       hipStream_t stream) {
    const int nch = K / 8;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    if (K >= kRowsPerWorkgroupK) {
        const int per_thread = (nch + 255) / 256;
        if (per_thread <= 4)
            hipLaunchKernelGGL((quantize_rows_wg_kernel<4, BF16, 256>), dim3(M), dim3(256), 0, stream, xp, ldx, K, xq, sx);
        else if (per_thread <= 6)
            hipLaunchKernelGGL((quantize_rows_wg_kernel<6, BF16, 256>), dim3(M), dim3(256), 0, stream, xp, ldx, K, xq, sx);
        else
            hipLaunchKernelGGL((quantize_rows_wg_kernel<8, BF16, 256>), dim3(M), dim3(256), 0, stream, xp, ldx, K, xq, sx);
        return hipGetLastError();
    }
    if (K >= kRowsPerPairK) {
        // two waves per row
        hipLaunchKernelGGL((quantize_rows_wg_kernel<4, BF16, 128>), dim3(M), dim3(128), 0, stream, xp, ldx, K, xq, sx);
        return hipGetLastError();
    }
    const int per_lane = (nch + 63) / 64;
    dim3 grid((M + 3) / 4), block(256);
    if (per_lane <= 1)
        hipLaunchKernelGGL((quantize_rows_kernel<1, BF16>), grid, block, 0, stream, xp, ldx, M, K, xq, sx);
    else if (per_lane <= 2)
        hipLaunchKernelGGL((quantize_rows_kernel<2, BF16>), grid, block, 0, stream, xp, ldx, M, K, xq, sx);
    else if (per_lane <= 4)
        hipLaunchKernelGGL((quantize_rows_kernel<4, BF16>), grid, block, 0, stream, xp, ldx, M, K, xq, sx);
    else if (per_lane <= 8)
        hipLaunchKernelGGL((quantize_rows_kernel<8, BF16>), grid, block, 0, stream, xp, ldx, M, K, xq, sx);
    else if (per_lane <= 16)
        hipLaunchKernelGGL((quantize_rows_kernel<16, BF16>), grid, block, 0, stream, xp, ldx, M, K, xq, sx);
    else
        hipLaunchKernelGGL((quantize_rows_kernel<32, BF16>), grid, block, 0, stream, xp, ldx, M, K, xq, sx);
    return hipGetLastError();
}

// ---- RMSNorm with the per-token quantization folded in -------------------------------
// The producer of a linear layer's input writes its codes directly (Cider README
// "Metal Kernel 流水线" runs the quantization as a dispatch of its own in front of the
// GEMM; juejin post, "W8A8 对称量化": that online step must stay cheap). The producer is
// RMSNorm with a per-channel weight g: n[k] = x[k] g[k] / sqrt(mean x^2 + eps). Its row
// factor is positive and common to the row, so it cancels in n / (max|n| / 127): the
// codes are those of u = x g (one fp32 multiply) and the factor goes into the scale,
// s_x = (max|u| / 127) / sqrt(mean x^2 + eps). The row's products u = x g are held in
// registers between the pass that finds max|u| and sum x^2 and the pass that writes
// codes, so x and g are read once (rows longer than the registers hold recompute the
// rest). The per-element quotient u / s uses
// the corrected reciprocal of the quantize kernel: with r = RN(1 / s) and the residual
// taken exactly by an fma, Markstein's theorem gives the correctly rounded quotient for
// any fp32 u (checked on the CPU against IEEE division on 2.5e8 products of two halves,
// a quarter of them with quotients at and next to a half-integer; the only difference is
// the sign of a zero quotient, which makes no difference to the code).

// u = x g for the eight values of one 16-byte chunk of x and of g (element e = 2 i + h of
// dword i), one fp32 product each, written fma(x, g, -0) (the same value: the product of two
// halves or two bf16 values is exact in fp32, and -0 is the additive identity, also for the
// sign of a zero) so that halves are read directly by v_fma_mix, with no conversion.
template <bool XBF, bool GBF>
__device__ __forceinline__ void norm_u8(uint4 xc, uint4 gc, float (&u)[8], float (&xv)[8]) {
    const uint32_t xw[4] = {xc.x, xc.y, xc.z, xc.w}, gw[4] = {gc.x, gc.y, gc.z, gc.w};
    const float nz = opaque_f32(-0.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            xv[2 * i + h] = to_float<XBF>(h ? xw[i] >> 16 : xw[i] & 0xffffu);
            u[2 * i + h] = __builtin_fmaf(xv[2 * i + h], to_float<GBF>(h ? gw[i] >> 16 : gw[i] & 0xffffu), nz);
        }
}

// Sum of squares: fp32 for fp16 rows (x^2 of any half stays within the fp32 normal range,
// 2^-48 .. 2^32); fp64 for bf16 rows, whose squares leave the fp32 range for |x| > 2^64 or
// |x| < 2^-75 (inf or 0 sums, so an infinite or zero scale beside nonzero codes).
template <typename SS>
__device__ __forceinline__ void norm_stats8(const float (&u)[8], const float (&xv)[8], float &amax, SS &ss) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        amax = __builtin_fmaxf(amax, __builtin_fabsf(u[e]));  // |u| as a source modifier
        if constexpr (std::is_same<SS, double>::value)
            ss = __builtin_fma((double)xv[e], (double)xv[e], ss);
        else
            ss = __builtin_fmaf(xv[e], xv[e], ss);
    }
}

// FAST: finite s >= 2^-100 (|u| <= max|u| then keeps every quotient inside (-127.5, 127.5),
// so no clamp), codes placed by the rounding adds; otherwise IEEE division and the clamp.
template <bool FAST>
__device__ __forceinline__ uint2 norm_quant8(const float (&u)[8], float s, float r) {
    uint32_t out[2] = {0, 0};
    if constexpr (FAST) {
        const float magic = opaque_f32(kMagic);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float q[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) q[h] = quotient<true>(u[4 * i + h], s, r);
            put_code<0>(out[i], q[0], magic);
            put_code<1>(out[i], q[1], magic);
            put_code<2>(out[i], q[2], magic);
            put_code<3>(out[i], q[3], magic);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e >> 2] |= code_byte(quotient<false>(u[e], s, r)) << (8 * (e & 3));
    }
    return make_uint2(out[0], out[1]);
}

// The fast path needs a finite scale: u = x g (or silu(gate) up) of finite bf16 inputs can
// overflow fp32, and an infinite row maximum gives s = inf.
__device__ __forceinline__ bool fast_scale(float s) { return s >= kMinFastScale && s <= 0x1.fffffep127f; }

// A row per 256-thread workgroup: thread t takes the 16-byte chunks t + 256 j, holds u = x g
// of the first CPT of them in registers between the two passes and recomputes the rest;
// the four waves combine max|u| and sum x^2 through LDS.
constexpr int NORM_THREADS = 256;

template <bool XBF, bool GBF, bool FAST, int CPT>
__device__ __forceinline__ void norm_row_store(const float (&uc)[CPT][8], const uint16_t *row, const uint16_t *g,
                                               int8_t *qrow, int tid, int nch, float s, float r) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + NORM_THREADS * j;
        if (c < nch) *reinterpret_cast<uint2 *>(qrow + 8 * c) = norm_quant8<FAST>(uc[j], s, r);
    }
    for (int c = tid + NORM_THREADS * CPT; c < nch; c += NORM_THREADS) {
        float u[8], xv[8];
        norm_u8<XBF, GBF>(*reinterpret_cast<const uint4 *>(row + 8 * c), *reinterpret_cast<const uint4 *>(g + 8 * c), u, xv);
        *reinterpret_cast<uint2 *>(qrow + 8 * c) = norm_quant8<FAST>(u, s, r);
    }
}

template <int CPT, bool XBF, bool GBF>
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_quantize_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                                         const uint16_t *__restrict__ g, float eps,
                                                                         int K, int8_t *__restrict__ xq,
                                                                         float *__restrict__ sx) {
    using SS = typename std::conditional<XBF, double, float>::type;
    __shared__ uint32_t wmax[NORM_THREADS / 64];
    __shared__ SS wsum[NORM_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = blockIdx.x;
    const uint16_t *row = x + (int64_t)m * ldx;
    int8_t *qrow = xq + (int64_t)m * K;
    const int nch = K >> 3;

    float uc[CPT][8];
    float amaxf = 0.0f;  // max |u| (u finite: the same value as a max over magnitude bit patterns)
    SS ss = 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + NORM_THREADS * j;
        float xv[8];
        if (c < nch) {
            norm_u8<XBF, GBF>(*reinterpret_cast<const uint4 *>(row + 8 * c), *reinterpret_cast<const uint4 *>(g + 8 * c),
                              uc[j], xv);
            norm_stats8(uc[j], xv, amaxf, ss);
        }
    }
    for (int c = tid + NORM_THREADS * CPT; c < nch; c += NORM_THREADS) {
        float u[8], xv[8];
        norm_u8<XBF, GBF>(*reinterpret_cast<const uint4 *>(row + 8 * c), *reinterpret_cast<const uint4 *>(g + 8 * c), u, xv);
        norm_stats8(u, xv, amaxf, ss);
    }
    uint32_t amax = wave_max_u32(__builtin_bit_cast(uint32_t, amaxf));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if (lane == 0) {
        wmax[wave] = amax;
        wsum[wave] = ss;
    }
    __syncthreads();
    amax = wmax[0];
    ss = wsum[0];
#pragma unroll
    for (int w = 1; w < NORM_THREADS / 64; ++w) {
        amax = amax > wmax[w] ? amax : wmax[w];
        ss += wsum[w];
    }

    const float s = __builtin_bit_cast(float, amax) / 127.0f;
    if (tid == 0) {
        if constexpr (XBF)
            sx[m] = s == 0.0f ? 0.0f : (float)((double)s * (1.0 / __builtin_sqrt(ss / (double)K + (double)eps)));
        else
            sx[m] = s == 0.0f ? 0.0f : s * (1.0f / __builtin_sqrtf(ss / (float)K + eps));
    }
    if (s == 0.0f) {
        for (int c = tid; c < nch; c += NORM_THREADS) *reinterpret_cast<uint2 *>(qrow + 8 * c) = make_uint2(0, 0);
        return;
    }
    if (fast_scale(s))
        norm_row_store<XBF, GBF, true, CPT>(uc, row, g, qrow, tid, nch, s, 1.0f / s);
    else
        norm_row_store<XBF, GBF, false, CPT>(uc, row, g, qrow, tid, nch, s, 0.f);
}

template <bool XBF, bool GBF>
hipError_t launch_norm_rows(const void *x, int64_t ldx, const void *g, float eps, int M, int K, int8_t *xq,
                            float *sx, hipStream_t stream) {
    const int per_thread = (K / 8 + NORM_THREADS - 1) / NORM_THREADS;
    dim3 grid(M), block(NORM_THREADS);
    const uint16_t *xp = static_cast<const uint16_t *>(x), *gp = static_cast<const uint16_t *>(g);
#define W8A8_NORM_LAUNCH(C) \
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<C, XBF, GBF>), grid, block, 0, stream, xp, ldx, gp, eps, K, xq, sx)
    if (per_thread <= 1) W8A8_NORM_LAUNCH(1);
    else if (per_thread <= 2) W8A8_NORM_LAUNCH(2);
    else if (per_thread <= 4) W8A8_NORM_LAUNCH(4);
    else if (per_thread <= 6) W8A8_NORM_LAUNCH(6);
    else W8A8_NORM_LAUNCH(8);
#undef W8A8_NORM_LAUNCH
    return hipGetLastError();
}

// ---- SwiGLU with the per-token quantization folded in ---------------------------------
// The producer of the down projection's input in a gated MLP writes that input's codes
// directly (Cider README "Metal Kernel 流水线": the quantization is otherwise a dispatch of
// its own; juejin post, "W8A8 对称量化": it must stay cheap): h = silu(gate) * up in fp32,
// then the per-token quantization of h, with h held in registers between the pass that finds
// max|h| and the pass that writes the codes. silu(g) = g / (1 + e^-g) uses one fixed fp32
// evaluation of e^x, so that the codes are reproducible bit for bit by any implementation of
// the same steps: the argument clamped to [-87, 88]; Cody-Waite reduction x = k ln 2 + r,
// k = rint(x log2 e), r by two fmas against ln 2 split into its fp32 rounding and the
// rounding of the remainder; e^r by the degree-7 Taylor polynomial (1 / n! in fp32), Horner
// with fmas; times 2^k (one rounding). Division g / (1 + e) is IEEE; the
// quotient h / s of the codes is the corrected reciprocal of the quantize kernel.

__device__ __forceinline__ float exp_fixed(float x) {
    x = __builtin_amdgcn_fmed3f(x, -87.0f, 88.0f);
    const float k = __builtin_rintf(x * 0x1.715476p+0f);   // log2 e
    float r = __builtin_fmaf(-k, 0x1.62e43p-1f, x);         // ln 2, high part
    r = __builtin_fmaf(-k, -0x1.05c61p-29f, r);             // ln 2, low part
    float p = 0x1.a01a02p-13f;                              // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);              // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);               // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);               // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);               // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    // p 2^k (k in [-126, 127]) by v_ldexp: the same value as p times the fp32 power 2^k (one
    // rounding either way, subnormal results included; equal for every fp16 and bf16 gate value)
    return __builtin_amdgcn_ldexpf(p, (int)k);
}

// h = silu(g) * u for the eight values of one 16-byte chunk of gate and of up.
template <bool BF16>
__device__ __forceinline__ void swiglu_h8(uint4 gc, uint4 uc, float (&h)[8]) {
    const uint32_t gw[4] = {gc.x, gc.y, gc.z, gc.w}, uw[4] = {uc.x, uc.y, uc.z, uc.w};
    const float nz = opaque_f32(-0.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float g = to_float<BF16>(e ? gw[i] >> 16 : gw[i] & 0xffffu);
            const float u = to_float<BF16>(e ? uw[i] >> 16 : uw[i] & 0xffffu);
            const float silu = g / (1.0f + exp_fixed(-g));
            h[2 * i + e] = __builtin_fmaf(silu, u, nz);  // silu * u; -0 keeps an fp16 u unconverted (v_fma_mix)
        }
}

template <bool BF16, bool FAST, int CPT>
__device__ __forceinline__ void swiglu_row_store(const float (&hc)[CPT][8], const uint16_t *grow, const uint16_t *urow,
                                                 int8_t *qrow, int tid, int nch, float s, float r) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + NORM_THREADS * j;
        if (c < nch) *reinterpret_cast<uint2 *>(qrow + 8 * c) = norm_quant8<FAST>(hc[j], s, r);
    }
    for (int c = tid + NORM_THREADS * CPT; c < nch; c += NORM_THREADS) {
        float h[8];
        swiglu_h8<BF16>(*reinterpret_cast<const uint4 *>(grow + 8 * c), *reinterpret_cast<const uint4 *>(urow + 8 * c), h);
        *reinterpret_cast<uint2 *>(qrow + 8 * c) = norm_quant8<FAST>(h, s, r);
    }
}

// A row per 256-thread workgroup: thread t takes the 16-byte chunks t + 256 j and holds h of
// the first CPT of them in registers (recomputing the rest); the four waves combine max|h|
// through LDS.
template <int CPT, bool BF16>
__global__ __launch_bounds__(NORM_THREADS) void swiglu_quantize_kernel(const uint16_t *__restrict__ gate, int64_t ldg,
                                                                        const uint16_t *__restrict__ up, int64_t ldu,
                                                                        int I, int8_t *__restrict__ xq,
                                                                        float *__restrict__ sx) {
    __shared__ uint32_t wmax[NORM_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = blockIdx.x;
    const uint16_t *grow = gate + (int64_t)m * ldg, *urow = up + (int64_t)m * ldu;
    int8_t *qrow = xq + (int64_t)m * I;
    const int nch = I >> 3;

    float hc[CPT][8];
    float amaxf = 0.0f;  // max |h| (h is never NaN: the same value as a max over magnitude bit patterns)
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + NORM_THREADS * j;
        if (c < nch) {
            swiglu_h8<BF16>(*reinterpret_cast<const uint4 *>(grow + 8 * c), *reinterpret_cast<const uint4 *>(urow + 8 * c),
                            hc[j]);
#pragma unroll
            for (int e = 0; e < 8; ++e) amaxf = __builtin_fmaxf(amaxf, __builtin_fabsf(hc[j][e]));
        }
    }
    for (int c = tid + NORM_THREADS * CPT; c < nch; c += NORM_THREADS) {
        float h[8];
        swiglu_h8<BF16>(*reinterpret_cast<const uint4 *>(grow + 8 * c), *reinterpret_cast<const uint4 *>(urow + 8 * c), h);
#pragma unroll
        for (int e = 0; e < 8; ++e) amaxf = __builtin_fmaxf(amaxf, __builtin_fabsf(h[e]));
    }
    uint32_t amax = wave_max_u32(__builtin_bit_cast(uint32_t, amaxf));
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int w = 1; w < NORM_THREADS / 64; ++w) amax = amax > wmax[w] ? amax : wmax[w];

    const float s = __builtin_bit_cast(float, amax) / 127.0f;
    if (tid == 0) sx[m] = s;
    if (s == 0.0f) {
        for (int c = tid; c < nch; c += NORM_THREADS) *reinterpret_cast<uint2 *>(qrow + 8 * c) = make_uint2(0, 0);
        return;
    }
    if (fast_scale(s))
        swiglu_row_store<BF16, true, CPT>(hc, grow, urow, qrow, tid, nch, s, 1.0f / s);
    else
        swiglu_row_store<BF16, false, CPT>(hc, grow, urow, qrow, tid, nch, s, 0.f);
}

template <bool BF16>
hipError_t launch_swiglu_rows(const void *gate, int64_t ldg, const void *up, int64_t ldu, int M, int I, int8_t *xq,
                              float *sx, hipStream_t stream) {
    const int per_thread = (I / 8 + NORM_THREADS - 1) / NORM_THREADS;
    dim3 grid(M), block(NORM_THREADS);
    const uint16_t *gp = static_cast<const uint16_t *>(gate), *up_ = static_cast<const uint16_t *>(up);
#define W8A8_SWIGLU_LAUNCH(C) \
    hipLaunchKernelGGL((swiglu_quantize_kernel<C, BF16>), grid, block, 0, stream, gp, ldg, up_, ldu, I, xq, sx)
    if (per_thread <= 1) W8A8_SWIGLU_LAUNCH(1);
    else if (per_thread <= 2) W8A8_SWIGLU_LAUNCH(2);
    else if (per_thread <= 4) W8A8_SWIGLU_LAUNCH(4);
    else if (per_thread <= 6) W8A8_SWIGLU_LAUNCH(6);
    else W8A8_SWIGLU_LAUNCH(8);
#undef W8A8_SWIGLU_LAUNCH
    return hipGetLastError();
}

// ---- offline weight quantization ------------------------------------------------------
// One wavefront per run (a weight row for per-channel, one K-group for per-group).
// Min-max symmetric (Cider README "说明"): s = max|W| / qdiv, q = clamp(rne(W / s)).
// int4: s = max / 7, codes in [-8, 7] stored as u = q + 8, even k in the low nibble
// (README "模式" / "量化").
//
// Clipped scale (README "说明", clip_percentile): the run's magnitude is the percentile
// u_i + f (u_{i+1} - u_i) of the sorted magnitudes u instead of the maximum, with i and f
// from the host (the same for every run: i = floor(h), f = h - i, h = pct (n - 1) / 100 in
// fp64), interpolated in fp64 and rounded once to fp32. u_i is found by radix selection on
// the magnitudes' fp32 bit patterns (non-negative floats order like their bit patterns):
// four passes over 8-bit digits, most significant first, each counting the run's values
// that match the digits chosen so far into a 256-bin histogram of this wave in LDS.

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor(v, d, 64));
    return v;
}

// Bit pattern of the rank-k (0-based, ascending) magnitude of src[0, n). Every lane returns it.
__device__ uint32_t run_select(const float *src, int n, uint32_t k, uint32_t *hist, int lane) {
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        // the wave's LDS operations run in issue order: the clears land before the counts
#pragma unroll
        for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0;
        __builtin_amdgcn_wave_barrier();
        for (int i = lane; i < n; i += 64) {
            const uint32_t key = __float_as_uint(src[i]) & 0x7fffffffu;
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
        }
        __builtin_amdgcn_wave_barrier();
        // lane l holds bins 4l .. 4l + 3; the lane whose bins hold rank k picks the digit
        const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                       c3 = hist[4 * lane + 3];
        const uint32_t own = c0 + c1 + c2 + c3;
        uint32_t incl = own;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t t = __shfl_up(incl, d, 64);
            if (lane >= d) incl += t;
        }
        const uint32_t excl = incl - own;
        const bool mine = excl <= k && k < incl;
        uint32_t below = excl;
        int bin = 0;
        if (mine) {
            if (k < below + c0) {
                bin = 0;
            } else if (k < below + c0 + c1) {
                bin = 1;
                below += c0;
            } else if (k < below + c0 + c1 + c2) {
                bin = 2;
                below += c0 + c1;
            } else {
                bin = 3;
                below += c0 + c1 + c2;
            }
        }
        const int owner = __ffsll((unsigned long long)__ballot(mine)) - 1;
        const uint32_t digit = (uint32_t)__shfl(4 * lane + bin, owner, 64);
        k -= (uint32_t)__shfl((int)below, owner, 64);
        prefix |= digit << shift;
        mask |= 0xffu << shift;
        __builtin_amdgcn_wave_barrier();
    }
    return prefix;
}

template <int BITS, bool CLIP>
__global__ __launch_bounds__(256) void quantize_weight_kernel(const float *__restrict__ W, int N,
                                                               int K, int run,
                                                               void *__restrict__ wq,
                                                               float *__restrict__ sw, int sel_i,
                                                               double sel_f) {
    __shared__ uint32_t hist[CLIP ? 4 * 256 : 1];
    const int lane = threadIdx.x & 63;
    const int runs_per_row = K / run;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= (int64_t)N * runs_per_row) return;
    const int64_t n = r / runs_per_row;
    const int g = (int)(r % runs_per_row);
    const float *src = W + n * K + (int64_t)g * run;

    float a = 0.f;
    if constexpr (CLIP) {
        // u_i, then u_{i+1}: u_i again when more than i + 1 magnitudes are <= u_i, else the
        // smallest magnitude above it
        const uint32_t ui = run_select(src, run, (uint32_t)sel_i, hist + (threadIdx.x >> 6) * 256, lane);
        uint32_t le = 0, above = 0xffffffffu;
        for (int i = lane; i < run; i += 64) {
            const uint32_t key = __float_as_uint(src[i]) & 0x7fffffffu;
            le += key <= ui ? 1u : 0u;
            if (key > ui) above = min(above, key);
        }
        le = wave_sum_u32(le);
        above = wave_min_u32(above);
        const uint32_t ui1 = le >= (uint32_t)sel_i + 2 ? ui : above;
        const double d0 = (double)__uint_as_float(ui), d1 = (double)__uint_as_float(ui1);
        a = (float)(d0 + sel_f * (d1 - d0));
    } else {
        for (int i = lane; i < run; i += 64) a = fmaxf(a, fabsf(src[i]));
        a = wave_max_f32(a);
    }
    const float qdiv = BITS == 8 ? 127.0f : 7.0f;
    const float s = a / qdiv;
    if (lane == 0) sw[r] = s;

    if (BITS == 8) {
        int8_t *dst = static_cast<int8_t *>(wq) + n * K + (int64_t)g * run;
        for (int i = lane; i < run; i += 64) dst[i] = (int8_t)quant_one(src[i], s, -128.f, 127.f);
    } else {
        uint8_t *dst = static_cast<uint8_t *>(wq) + n * (K / 2) + (int64_t)g * (run / 2);
        for (int p = lane; p < run / 2; p += 64) {
            int q0 = quant_one(src[2 * p], s, -8.f, 7.f);
            int q1 = quant_one(src[2 * p + 1], s, -8.f, 7.f);
            dst[p] = (uint8_t)((q0 + 8) | ((q1 + 8) << 4));
        }
    }
}

}  // namespace

hipError_t launch_quantize_per_token(const void *x, bool bf16, int64_t ldx, int M, int K,
                                     int8_t *xq, float *sx, hipStream_t stream) {
    return bf16 ? launch_rows<true>(x, ldx, M, K, xq, sx, stream)
                : launch_rows<false>(x, ldx, M, K, xq, sx, stream);
}

hipError_t launch_rmsnorm_quantize(const void *x, bool x_bf16, int64_t ldx, const void *g, bool g_bf16, float eps,
                                   int M, int K, int8_t *xq, float *sx, hipStream_t stream) {
    if (x_bf16) return g_bf16 ? launch_norm_rows<true, true>(x, ldx, g, eps, M, K, xq, sx, stream)
                              : launch_norm_rows<true, false>(x, ldx, g, eps, M, K, xq, sx, stream);
    return g_bf16 ? launch_norm_rows<false, true>(x, ldx, g, eps, M, K, xq, sx, stream)
                  : launch_norm_rows<false, false>(x, ldx, g, eps, M, K, xq, sx, stream);
}

hipError_t launch_swiglu_quantize(const void *gate, int64_t ldg, const void *up, int64_t ldu, bool bf16, int M, int I,
                                  int8_t *xq, float *sx, hipStream_t stream) {
    return bf16 ? launch_swiglu_rows<true>(gate, ldg, up, ldu, M, I, xq, sx, stream)
                : launch_swiglu_rows<false>(gate, ldg, up, ldu, M, I, xq, sx, stream);
}

hipError_t launch_quantize_weight(const float *W, int N, int K, int bits, int gs, void *wq,
                                  float *sw, hipStream_t stream) {
    return launch_quantize_weight_clipped(W, N, K, bits, gs, 100.0f, wq, sw, stream);
}

hipError_t launch_quantize_weight_clipped(const float *W, int N, int K, int bits, int gs, float pct, void *wq,
                                          float *sw, hipStream_t stream) {
    const int run = gs ? gs : K;
    const int64_t runs = (int64_t)N * (K / run);
    dim3 grid((unsigned)((runs + 3) / 4)), block(256);
    // position of the percentile among the run's sorted magnitudes (the maximum at 100)
    const double h = ((double)pct * (double)(run - 1)) / 100.0;
    const int64_t i = (int64_t)floor(h);
    const double f = h - (double)i;
    if (i >= run - 1) {
        if (bits == 8)
            hipLaunchKernelGGL((quantize_weight_kernel<8, false>), grid, block, 0, stream, W, N, K, run, wq, sw, 0, 0.0);
        else
            hipLaunchKernelGGL((quantize_weight_kernel<4, false>), grid, block, 0, stream, W, N, K, run, wq, sw, 0, 0.0);
    } else {
        if (bits == 8)
            hipLaunchKernelGGL((quantize_weight_kernel<8, true>), grid, block, 0, stream, W, N, K, run, wq, sw, (int)i, f);
        else
            hipLaunchKernelGGL((quantize_weight_kernel<4, true>), grid, block, 0, stream, W, N, K, run, wq, sw, (int)i, f);
    }
    return hipGetLastError();
}

}  // namespace w8a8
