// Per-token activation code arithmetic for gfx950, shared by the quantize kernel and the
// fused small-M linear kernel so that both produce the same codes and scales.
//
// Per-token symmetric int8 quantization (juejin post "在Mac上跑大模型，MLX 不是终点",
// section "W8A8 对称量化：Cider 的选择"): s = max|x| / 127, q = clamp(round(x / s)), with
// "round" read as IEEE round-half-to-even of the correctly rounded fp32 quotient x / s.
// Never build users of this header with fast-math, approximate division or flushed fp32
// denormals.
#pragma once

#include "internal.h"

namespace w8a8 {
namespace act {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __builtin_bit_cast(float, h << 16);
}

template <bool BF16>
__device__ __forceinline__ float to_float(uint32_t bits) {
    return BF16 ? bf16_bits_to_float(bits) : half_bits_to_float(bits);
}

// max(v, v of the lane that the DPP pattern CTRL selects), in the rows that ROWS enables
// (other rows keep v).
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xf, false);
    return v > o ? v : o;
}

// Maximum over the 64 lanes of a wave (all lanes active), returned to every lane. DPP moves
// within and across 16-lane rows and one lane read, instead of six LDS-crossbar permutes
// (__shfl_xor): a few cycles per step on the critical path of a row's quantization.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_dpp<0xb1>(v);        // quad_perm [1, 0, 3, 2]
    v = max_dpp<0x4e>(v);        // quad_perm [2, 3, 0, 1]: max of each quad
    v = max_dpp<0x141>(v);       // row_half_mirror: max of each half-row
    v = max_dpp<0x140>(v);       // row_mirror: max of each row
    v = max_dpp<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3: rows (0, 1) and (2, 3)
    v = max_dpp<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3: row 3 holds all four
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Per-element quotient. Quantization is VALU-bound, not HBM-bound, if every element pays
// for an IEEE division (about ten instructions, four cycles each for a wave64 on a 16-lane
// SIMD). Instead each row divides once, r = 1 / s (correctly rounded), and each element
// takes Markstein's corrected quotient
//     q0 = x * r,   e = fma(-q0, s, x),   q = fma(e, r, q0),
// which equals the IEEE quotient x / s: checked exhaustively on the CPU for every pair of
// an fp16 row maximum and an fp16 element (1.0e9 pairs, no difference), and for bf16 every
// pair gives the same rounded code when s >= 2^-100 (rows with a smaller scale, possible
// only for bf16 input, keep the true division). The quotient is clamped to [-128, 127] and
// rounded half-to-even by adding 1.5 * 2^23: in that binade the fp32 spacing is 1, so the
// addition itself rounds to the nearest integer (ties to even) and the code is the low
// byte of the sum's bit pattern.
//
// On the fast path (finite input, s >= 2^-100) the clamp is never active and is left out:
// s = RN(max|x| / 127) is a normal number within 2^-24 relative of max|x| / 127, so
// |x / s| <= 127 (1 + 2^-24) / (1 - 2^-24) < 127.5 and every code already lies in
// [-127, 127].

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kMinFastScale = 0x1p-100f;

// Row scale from the largest magnitude bit pattern of the row: one IEEE fp32 division.
template <bool BF16>
__device__ __forceinline__ float row_scale(uint32_t amax_bits) {
    return to_float<BF16>(amax_bits) / 127.0f;
}

__device__ __forceinline__ uint32_t code_byte(float t) {
    t = __builtin_amdgcn_fmed3f(t, -128.0f, 127.0f);
    return __builtin_bit_cast(uint32_t, t + kMagic) & 0xffu;
}

template <bool FAST>
__device__ __forceinline__ float quotient(float x, float s, float r) {
    if (FAST) {
        const float q0 = x * r;
        const float e = __builtin_fmaf(-q0, s, x);
        return __builtin_fmaf(e, r, q0);
    }
    return x / s;
}

// A value the compiler cannot see through (so fma(x, r, -0) is not folded into a multiply).
__device__ __forceinline__ float opaque_f32(float v) {
    asm("" : "+v"(v));
    return v;
}

// acc byte B = low byte of the bits of q + magic (the rounded code), the other bytes kept
// (B = 0: cleared). One SDWA add per code: the rounding add also places the byte.
template <int B>
__device__ __forceinline__ void put_code(uint32_t &acc, float q, float magic) {
    static_assert(B >= 0 && B < 4, "byte index");
    if constexpr (B == 0)
        asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD"
            : "=v"(acc) : "v"(q), "v"(magic));
    else if constexpr (B == 1)
        asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
            : "+v"(acc) : "v"(q), "v"(magic));
    else if constexpr (B == 2)
        asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
            : "+v"(acc) : "v"(q), "v"(magic));
    else
        asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
            : "+v"(acc) : "v"(q), "v"(magic));
}

// Eight elements (one 16-byte chunk) -> eight codes (8 bytes).
// FAST (s >= 2^-100, finite input): the corrected quotient with no clamp (see above); for
// fp16 the product x r is written fma(x, r, -0) (the same value, -0 being the additive
// identity) so that both products read the half directly (v_fma_mix, no conversion).
// Otherwise: IEEE division and the clamp.
template <bool BF16, bool FAST>
__device__ __forceinline__ uint2 quant8(uint4 c, float s, float r) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t out[2];
    if constexpr (FAST) {
        const float nz = opaque_f32(-0.0f), magic = opaque_f32(kMagic);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float q[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t word = w[2 * i + (h >> 1)];
                const float x = to_float<BF16>((h & 1) ? word >> 16 : word & 0xffffu);
                const float q0 = BF16 ? x * r : __builtin_fmaf(x, r, nz);
                const float e = __builtin_fmaf(-q0, s, x);
                q[h] = __builtin_fmaf(e, r, q0);
            }
            uint32_t acc;
            put_code<0>(acc, q[0], magic);
            put_code<1>(acc, q[1], magic);
            put_code<2>(acc, q[2], magic);
            put_code<3>(acc, q[3], magic);
            out[i] = acc;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t b0 = code_byte(quotient<false>(to_float<BF16>(w[2 * i] & 0xffffu), s, r));
            const uint32_t b1 = code_byte(quotient<false>(to_float<BF16>(w[2 * i] >> 16), s, r));
            const uint32_t b2 = code_byte(quotient<false>(to_float<BF16>(w[2 * i + 1] & 0xffffu), s, r));
            const uint32_t b3 = code_byte(quotient<false>(to_float<BF16>(w[2 * i + 1] >> 16), s, r));
            out[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
    }
    return make_uint2(out[0], out[1]);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Max of the magnitude bit patterns of eight fp16 / bf16 values, as two packed u16 lanes.
__device__ __forceinline__ u16x2 absmax8(uint4 c, u16x2 m) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
    return m;
}

}  // namespace act
}  // namespace w8a8
