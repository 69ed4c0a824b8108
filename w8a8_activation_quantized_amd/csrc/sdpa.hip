// Decode-step attention for gfx950 (sdpa_decode): one query token per head, no mask, query
// heads grouped over shared KV heads (Cider README "优化 SDPA（解码注意力）").
//
// Layout: q [B, Hq, D], k and v [B, Hkv, Ncap, D] (the first N rows of each head are used),
// fp16 or bf16; query head h reads KV head h / G with G = Hq / Hkv.
//
// Design (the pages' ideas on CDNA4):
//  * One workgroup serves all G query heads of one KV head over one slice of the keys, so each
//    K and V row is read from HBM once for the whole group (the pages' contiguous-chunk GQA
//    scheduling), not G times.
//  * Long caches are split over workgroups (two-pass FlashDecoding): each slice keeps its own
//    running maximum, sum and weighted value sum, written to a caller-provided workspace and
//    merged by a second kernel; with one slice the first kernel writes the output directly.
//  * Scores on the matrix cores: S^T = K_block . q^T with v_mfma_f32_16x16x32_{f16,bf16}, the
//    block's 16 keys as A rows and the (up to 16) query heads as B columns, so K rows are
//    loaded straight from HBM into the A operand (16 bytes of one row per lane). Products are
//    exact in fp32; scores, the softmax and every sum are fp32.
//  * P . V on the vector units: V's contiguous dimension is d, not the summed key dimension
//    the MFMA operands want, so each lane owns 8 consecutive d of one key residue class and
//    accumulates all G heads; the probabilities pass through a small per-wave LDS tile.
//  * Online softmax per 32-key block in base 2: scores are scaled by scale * log2(e) once,
//    p = exp2(s - m), and the running sums are rescaled by exp2(m_old - m_new) per block.
#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef _Float16 sd_v8h __attribute__((ext_vector_type(8)));
typedef __bf16 sd_v8bf __attribute__((ext_vector_type(8)));
typedef float sd_v4f __attribute__((ext_vector_type(4)));

constexpr int SD_WAVES = 4;  // waves per workgroup
constexpr int SD_BK = 32;    // keys per block (two MFMA row tiles)

template <bool BF16>
__device__ __forceinline__ float half_to_f32(uint32_t bits16) {
    if constexpr (BF16)
        return __builtin_bit_cast(float, bits16 << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <bool BF16>
__device__ __forceinline__ sd_v4f mfma_qk(v4u a, v4u b, sd_v4f c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sd_v8bf, a), __builtin_bit_cast(sd_v8bf, b), c, 0,
                                                       0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(sd_v8h, a), __builtin_bit_cast(sd_v8h, b), c, 0, 0,
                                                      0);
}

struct SdpaArgs {
    const uint16_t *q, *k, *v;
    void *o;      // final output (slices == 1)
    float *part;  // per (b, h, slice): m, l, 0, 0, o[0 .. D) (slices > 1)
    int B, Hq, Hkv, G, N, Ncap, slices, out;
    float c;  // scale * log2(e)
};

// Workgroup (slice, b * Hkv + kvh). GMAX >= G bounds the per-lane accumulators.
template <int D, int GMAX, bool BF16>
__global__ __launch_bounds__(64 * SD_WAVES) void sdpa_kernel(SdpaArgs a) {
    constexpr int T = D / 32;          // MFMAs per 16-key tile
    constexpr int LPR = D / 8;         // lanes per value row (8 d each)
    constexpr int KG = 64 / LPR;       // key residue classes per wave
    constexpr int KPL = SD_BK / KG;    // keys per lane per block
    constexpr int GV = (GMAX + 3) / 4; // float4 reads per probability row
    __shared__ __attribute__((aligned(16))) float p_lds[SD_WAVES][SD_BK][16];
    __shared__ __attribute__((aligned(16))) float al_lds[SD_WAVES][16];
    __shared__ __attribute__((aligned(16))) float red_o[SD_WAVES][GMAX][D];
    __shared__ float red_ml[SD_WAVES][2][16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.Hkv, kvh = bk % a.Hkv;
    const int G = a.G, N = a.N;
    // keys of this slice, then of this wave
    const int s0 = (int)((int64_t)slice * N / a.slices), s1 = (int)((int64_t)(slice + 1) * N / a.slices);
    const int w0 = s0 + (int)((int64_t)wave * (s1 - s0) / SD_WAVES);
    const int w1 = s0 + (int)((int64_t)(wave + 1) * (s1 - s0) / SD_WAVES);
    const uint16_t *K = a.k + ((int64_t)b * a.Hkv + kvh) * a.Ncap * D;
    const uint16_t *V = a.v + ((int64_t)b * a.Hkv + kvh) * a.Ncap * D;

    // MFMA lane roles: row / column r16 = lane % 16, quarter q4 = lane / 16
    const int r16 = lane & 15, q4 = lane >> 4;
    // q^T columns: head r16 of the group (zero past G), d in [32 t + 8 q4, + 8)
    v4u qf[T];
    {
        const uint16_t *qh = a.q + ((int64_t)b * a.Hq + (int64_t)kvh * G + min(r16, G - 1)) * D;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const v4u x = *reinterpret_cast<const v4u *>(qh + 32 * t + 8 * q4);
            qf[t] = r16 < G ? x : v4u{0, 0, 0, 0};
        }
    }
    // value roles: 8 d starting at 8 dq, keys kq, kq + KG, ... of each block
    const int dq = lane % LPR, kq = lane / LPR;

    float m = -INFINITY, l = 0.f;  // of head r16 (copies in the 4 lanes of a column)
    float o[GMAX][8];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = 0.f;

    for (int n0 = w0; n0 < w1; n0 += SD_BK) {
        // loads: K rows of both tiles (A operands) and this lane's V pieces
        v4u kf[2][T], vf[KPL];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int row = min(n0 + 16 * tile + r16, w1 - 1);
#pragma unroll
            for (int t = 0; t < T; ++t) kf[tile][t] = *reinterpret_cast<const v4u *>(K + (int64_t)row * D + 32 * t + 8 * q4);
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int row = min(n0 + kq + KG * i, w1 - 1);
            vf[i] = *reinterpret_cast<const v4u *>(V + (int64_t)row * D + 8 * dq);
        }
        // scores: lane holds keys 16 tile + 4 q4 + e of head r16
        sd_v4f sc[2];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            sd_v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < T; ++t) acc = mfma_qk<BF16>(kf[tile][t], qf[t], acc);
            sc[tile] = acc;
        }
        float s[8];
        float bm = -INFINITY;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = n0 + 16 * tile + 4 * q4 + e;
                const float x = key < w1 ? sc[tile][e] * a.c : -INFINITY;
                s[4 * tile + e] = x;
                bm = fmaxf(bm, x);
            }
        bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
        bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
        const float mn = fmaxf(m, bm);  // finite: every block has a key below w1
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = __builtin_amdgcn_exp2f(s[i] - mn);
            ps += s[i];
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l = l * alpha + ps;
        m = mn;
        // probabilities and rescale factors to LDS: P[key][head]
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int e = 0; e < 4; ++e) p_lds[wave][16 * tile + 4 * q4 + e][r16] = s[4 * tile + e];
        if (q4 == 0) al_lds[wave][r16] = alpha;
        __builtin_amdgcn_wave_barrier();
        // (this wave's LDS writes and reads run in issue order)
        float al[GMAX];
#pragma unroll
        for (int j = 0; j < GV; ++j) {
            const float4 x = *reinterpret_cast<const float4 *>(&al_lds[wave][4 * j]);
            al[4 * j] = x.x;
            if (4 * j + 1 < GMAX) al[4 * j + 1] = x.y;
            if (4 * j + 2 < GMAX) al[4 * j + 2] = x.z;
            if (4 * j + 3 < GMAX) al[4 * j + 3] = x.w;
        }
#pragma unroll
        for (int g = 0; g < GMAX; ++g)
#pragma unroll
            for (int j = 0; j < 8; ++j) o[g][j] *= al[g];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int r = kq + KG * i;
            float pr[GMAX];
#pragma unroll
            for (int j = 0; j < GV; ++j) {
                const float4 x = *reinterpret_cast<const float4 *>(&p_lds[wave][r][4 * j]);
                pr[4 * j] = x.x;
                if (4 * j + 1 < GMAX) pr[4 * j + 1] = x.y;
                if (4 * j + 2 < GMAX) pr[4 * j + 2] = x.z;
                if (4 * j + 3 < GMAX) pr[4 * j + 3] = x.w;
            }
            float vv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vv[2 * j] = half_to_f32<BF16>(vf[i][j] & 0xffffu);
                vv[2 * j + 1] = half_to_f32<BF16>(vf[i][j] >> 16);
            }
#pragma unroll
            for (int g = 0; g < GMAX; ++g)
#pragma unroll
                for (int j = 0; j < 8; ++j) o[g][j] = __builtin_fmaf(pr[g], vv[j], o[g][j]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // the wave's key classes -> one sum per (head, d): butterfly over the lanes of a d range
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float x = o[g][j];
#pragma unroll
            for (int sh = LPR; sh < 64; sh <<= 1) x += __shfl_xor(x, sh, 64);
            o[g][j] = x;
        }
    // merge the waves: wave w's (m, l, o) to LDS, then each thread combines one (head, d) set
    if (kq == 0) {
#pragma unroll
        for (int g = 0; g < GMAX; ++g)
#pragma unroll
            for (int j = 0; j < 8; ++j) red_o[wave][g][8 * dq + j] = o[g][j];
    }
    if (q4 == 0) {
        red_ml[wave][0][r16] = m;  // -inf for a wave without keys
        red_ml[wave][1][r16] = l;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += 64 * SD_WAVES) {
        const int g = e / D, d = e - g * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < SD_WAVES; ++w) M = fmaxf(M, red_ml[w][0][g]);
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < SD_WAVES; ++w) {
            const float mw = red_ml[w][0][g];
            const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            L += red_ml[w][1][g] * f;
            acc += red_o[w][g][d] * f;
        }
        const int h = kvh * G + g;
        if (a.slices == 1) {
            const float y = acc / L;
            const int64_t off = ((int64_t)b * a.Hq + h) * D + d;
            if (a.out == OUT_F32)
                static_cast<float *>(a.o)[off] = y;
            else if (a.out == OUT_BF16)
                static_cast<uint16_t *>(a.o)[off] = (uint16_t)bf16_rne(y);
            else
                static_cast<uint16_t *>(a.o)[off] = (uint16_t)f16_bits(y);
        } else {
            float *pp = a.part + (((int64_t)b * a.Hq + h) * a.slices + slice) * (D + 4);
            if (d == 0) {
                pp[0] = M;
                pp[1] = L;
            }
            pp[4 + d] = acc;
        }
    }
}

// Second pass: merge the slices of one (b, h), thread d.
template <int D>
__global__ __launch_bounds__(D) void sdpa_combine_kernel(const float *part, void *o, int slices, int out) {
    const int bh = blockIdx.x, d = threadIdx.x;
    const float *pp = part + (int64_t)bh * slices * (D + 4);
    float M = -INFINITY;
    for (int s = 0; s < slices; ++s) M = fmaxf(M, pp[s * (D + 4)]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < slices; ++s) {
        const float f = __builtin_amdgcn_exp2f(pp[s * (D + 4)] - M);
        L += pp[s * (D + 4) + 1] * f;
        acc += pp[s * (D + 4) + 4 + d] * f;
    }
    const float y = acc / L;
    const int64_t off = (int64_t)bh * D + d;
    if (out == OUT_F32)
        static_cast<float *>(o)[off] = y;
    else if (out == OUT_BF16)
        static_cast<uint16_t *>(o)[off] = (uint16_t)bf16_rne(y);
    else
        static_cast<uint16_t *>(o)[off] = (uint16_t)f16_bits(y);
}

template <int D, int GMAX, bool BF16>
hipError_t launch_sdpa_t(const SdpaArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((sdpa_kernel<D, GMAX, BF16>), dim3(a.slices, a.B * a.Hkv), dim3(64 * SD_WAVES), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.slices == 1) return e;
    hipLaunchKernelGGL((sdpa_combine_kernel<D>), dim3(a.B * a.Hq), dim3(D), 0, stream, a.part, a.o, a.slices, a.out);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_sdpa_d(const SdpaArgs &a, hipStream_t stream) {
    if (a.G <= 4) return launch_sdpa_t<D, 4, BF16>(a, stream);
    if (a.G <= 8) return launch_sdpa_t<D, 8, BF16>(a, stream);
    return launch_sdpa_t<D, 16, BF16>(a, stream);
}

}  // namespace

int sdpa_slices(int B, int Hkv, int N) {
    // about two workgroups per CU, each slice at least 256 keys (two blocks per wave)
    const int64_t groups = (int64_t)B * Hkv;
    int s = (int)((2 * (int64_t)num_cus() + groups - 1) / groups);
    s = std::min(s, std::max(1, N / 256));
    return std::max(1, std::min(s, 1024));
}

int64_t sdpa_workspace_bytes(int B, int Hq, int Hkv, int N, int D) {
    const int s = sdpa_slices(B, Hkv, N);
    return s > 1 ? (int64_t)B * Hq * s * (D + 4) * 4 : 0;
}

hipError_t launch_sdpa_decode(const void *q, const void *k, const void *v, bool bf16, void *o, int out, int B, int Hq,
                              int Hkv, int N, int Ncap, int D, float scale, void *ws, int64_t ws_bytes,
                              hipStream_t stream) {
    SdpaArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = o;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.N = N;
    a.Ncap = Ncap;
    a.out = out;
    a.c = (float)((double)scale * 1.4426950408889634);  // scale * log2(e), rounded once
    a.slices = sdpa_slices(B, Hkv, N);
    if (a.slices > 1 && (ws == nullptr || ws_bytes < sdpa_workspace_bytes(B, Hq, Hkv, N, D))) a.slices = 1;
    a.part = static_cast<float *>(ws);
    if (D == 64) return bf16 ? launch_sdpa_d<64, true>(a, stream) : launch_sdpa_d<64, false>(a, stream);
    return bf16 ? launch_sdpa_d<128, true>(a, stream) : launch_sdpa_d<128, false>(a, stream);
}

}  // namespace w8a8
