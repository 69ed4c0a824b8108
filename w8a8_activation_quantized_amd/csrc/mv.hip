// Decode path of libw8a8 (gfx950): int8 weights times fp16 / bf16 activations, with no
// activation quantization (int8_mv).
#include "device_common.h"
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int MV_MAX_WAVES = 8;  // waves per workgroup (max)

// ---- decode: int8 weights times fp16 / bf16 activations ---------------------------------
//
// The pages' decode path (Cider README "Metal Kernel 流水线", decode; juejin post "INT8
// TensorOps 内核设计", the two paths): the weights are dequantized as they stream and meet
// the activations as they are, with no per-token quantization:
//   y[m, n] = sum_k x[m, k] * (w_q[n, k] * s_w[n, g(k)])
// computed here as fp32 products and sums on the matrix cores: the codes are converted to
// the activation format (exact: |q| <= 128 fits both fp16 and bf16) and multiplied with
// v_mfma_f32_16x16x32_{f16,bf16}; per channel the sum over K is scaled by s_w[n] at the end,
// per group each group's sum is folded, t = fma(sum_g, s_w[n, g], t). Up to 16 tokens are the
// 16 columns of the B operand (M = 1 uses one).
//
// Streaming is that of gemv_dma_kernel: a workgroup owns 16 output rows, its waves split K
// into segments of whole 128-value chunks (whole groups), and each wave runs a private ring
// of slots filled by global_load_lds: 16 weight rows x 128 bytes (the 16-byte pieces of row r
// at position piece ^ ((r >> 1) & 7)), then the chunk's activations, M rows x 256 bytes
// (row r's 16-byte piece P at position P ^ r, so that the 16 rows read at one position hit
// 16 different bank groups). A lane (row / token l % 16, quarter f = l / 16) reads weight
// pieces f and 4 + f of its row: piece 4h + f holds k in [16(4h + f), 16(4h + f) + 16) of the
// chunk, whose two halves are the lane's operands of MFMA 2h and 2h + 1; the activation
// operand of MFMA t is the 8 values at the same k. The products pair A and B lanes of the
// same quarter, so any such assignment of k to quarters gives the full dot product, and this
// one reads each weight byte once with 16-byte loads and keeps MFMAs 0-1 in the chunk's first
// 64 values and MFMAs 2-3 in the second (the group boundaries for a group size of 64).
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Eight int8 codes (two dwords) -> eight fp16 values, exactly: byte b ^ 0x80 = q + 128 is the
// low mantissa byte of the half 0x64xx = 1024 + (q + 128), and subtracting 1152 leaves q.
__device__ __forceinline__ v8h codes_to_f16(uint32_t d0, uint32_t d1) {
    const uint32_t u0 = d0 ^ 0x80808080u, u1 = d1 ^ 0x80808080u;
    const v2h off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const v2h h0 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) + off;
    const v2h h1 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) + off;
    const v2h h2 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) + off;
    const v2h h3 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) + off;
    return v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Eight int8 codes -> eight bf16 values, exactly: each code through fp32 (exact), whose upper
// half is the bf16 value (a code has at most 8 significant bits).
__device__ __forceinline__ v8bf codes_to_bf16(uint32_t d0, uint32_t d1) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d = i < 2 ? d0 : d1, sh = 16 * (i & 1);
        const float lo = (float)(int)(int8_t)(d >> sh), hi = (float)(int)(int8_t)(d >> (sh + 8));
        o[i] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
    }
    return __builtin_bit_cast(v8bf, v4u{o[0], o[1], o[2], o[3]});
}

template <int OPS, int N>
__device__ __forceinline__ void mv_wait_tail(int after) {
    // vmcnt wait allowing `after` chunks (OPS instructions each) issued after the one needed
    if constexpr (N > 0) {
        if (after >= N) {
            wait_vmcnt<OPS * N>();
            return;
        }
        mv_wait_tail<OPS, N - 1>(after);
    } else {
        wait_vmcnt<0>();
    }
}

constexpr int MV_RING = 8;  // ring slots per wave (max)

// GS: 0 (per channel), 64 or 128; XR = ceil(M / 4): 1 KiB activation pieces per slot.
template <int GS, bool BF16X, int XR>
__global__ __launch_bounds__(64 * MV_MAX_WAVES) void mv_kernel(GemmProblem p, int seg_chunks, int slots,
                                                                  int table_groups) {
    constexpr bool GROUPED = GS > 0;
    constexpr int GPC = GROUPED ? 128 / GS : 1;  // groups per chunk
    constexpr int OPS = 2 + XR;                   // DMA instructions per chunk
    constexpr int SLOT = 2048 + XR * 1024;
    static_assert(OPS * (MV_RING - 1) < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(1024))) int8_t mv_lds[];

    const int NW = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int frow = lane & 15, fq = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int M = p.M, N = p.N, K = p.K;
    const int G = GROUPED ? K / GS : 1;
    const int NCH = K / 128;
    const int c0 = wave * seg_chunks, nch = max(min(NCH, c0 + seg_chunks) - c0, 0);

    int8_t *ring = mv_lds + wave * slots * SLOT;
    float *table = reinterpret_cast<float *>(mv_lds + NW * slots * SLOT) + wave * table_groups * 16;

    // per-channel scales of the lane's four output rows, fetched ahead of the weight stream
    float4 e_sw = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (!GROUPED)
        if (wave == 0) e_sw = *reinterpret_cast<const float4 *>(p.sw + min(n0 + 4 * fq, N - 4));

    // group scales of the segment: table[(g - g0) * 16 + r] = s_w[n0 + r, g] (4-byte DMA,
    // 64 entries per instruction; table_groups is a multiple of 4)
    const int g0 = c0 * GPC;
    if constexpr (GROUPED) {
        const int ng = min(G - g0, table_groups);
        for (int b = 0; b * 64 < ng * 16; ++b) {
            const int e = b * 64 + lane;
            const int gg = min(e >> 4, ng - 1), r = e & 15;
            dma_4B(p.sw + (int64_t)min(n0 + r, N - 1) * G + g0 + gg, table + b * 64);
        }
    }

    // weight pieces: lane i covers row (half * 8 + i / 8) at slot position i % 8
    const int dr = lane >> 3, dpos = lane & 7;
    const int8_t *W = static_cast<const int8_t *>(p.wq);
    const int8_t *src_lo = W + (int64_t)min(n0 + dr, N - 1) * K + 16 * (dpos ^ ((dr >> 1) & 7));
    const int8_t *src_hi = W + (int64_t)min(n0 + 8 + dr, N - 1) * K + 16 * (dpos ^ (((8 + dr) >> 1) & 7));
    // activation pieces: piece i = 64 b + lane of the chunk's block is row i / 16 at position
    // i % 16, holding the row's 8 values (i % 16) ^ row; lanes past 16 M stay idle
    const uint16_t *X = static_cast<const uint16_t *>(p.x);
    auto issue = [&](int j, int8_t *slot) __attribute__((always_inline)) {
        const int ck = c0 + j;
        dma_16B(src_lo + ck * 128, slot);
        dma_16B(src_hi + ck * 128, slot + 1024);
#pragma unroll
        for (int b = 0; b < XR; ++b) {
            const int xi = 64 * b + lane, xr = xi >> 4;
            if (xi < 16 * M)
                dma_16B(X + (int64_t)xr * p.ldx + ck * 128 + 8 * ((xi & 15) ^ xr), slot + 2048 + b * 1024);
        }
    };

    v4f acc = {0.f, 0.f, 0.f, 0.f};
    float facc[4] = {0.f, 0.f, 0.f, 0.f};
    const int xm = min(frow, M - 1);
    const int R = min(slots, nch);
    for (int j = 0; j < R; ++j) issue(j, ring + j * SLOT);
    int sl = 0;
    for (int j = 0; j < nch; ++j) {
        mv_wait_tail<OPS, MV_RING - 1>(min(nch, j + R) - j - 1);
        const int8_t *slot = ring + sl * SLOT;
        const v4u w0 = *reinterpret_cast<const v4u *>(slot + frow * 128 + ((fq ^ ((frow >> 1) & 7)) << 4));
        const v4u w1 = *reinterpret_cast<const v4u *>(slot + frow * 128 + (((4 + fq) ^ ((frow >> 1) & 7)) << 4));
        const int8_t *xs = slot + 2048 + xm * 256;
        v4u xb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int L = 2 * (4 * (t >> 1) + fq) + (t & 1);
            xb[t] = *reinterpret_cast<const v4u *>(xs + ((L ^ xm) << 4));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v4u w = t < 2 ? w0 : w1;
            const uint32_t d0 = (t & 1) ? w[2] : w[0], d1 = (t & 1) ? w[3] : w[1];
            const bool restart = GROUPED && (GS == 64 ? (t & 1) == 0 : t == 0);
            const v4f c = restart ? v4f{0.f, 0.f, 0.f, 0.f} : acc;
            if constexpr (BF16X)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(d0, d1), __builtin_bit_cast(v8bf, xb[t]), c, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes_to_f16(d0, d1), __builtin_bit_cast(v8h, xb[t]), c, 0, 0, 0);
            if constexpr (GROUPED) {
                if (GS == 64 ? (t & 1) == 1 : t == 3) {
                    const int g = (c0 + j) * GPC + (GS == 64 ? (t >> 1) : 0);
                    // (the table's DMA was retired by the first chunk wait)
                    const float4 sw = lds_read_f4_now(table + (g - g0) * 16 + 4 * fq);
                    facc[0] = __builtin_fmaf(acc[0], sw.x, facc[0]);
                    facc[1] = __builtin_fmaf(acc[1], sw.y, facc[1]);
                    facc[2] = __builtin_fmaf(acc[2], sw.z, facc[2]);
                    facc[3] = __builtin_fmaf(acc[3], sw.w, facc[3]);
                }
            }
        }
        if (j + R < nch) {
            wait_lgkmcnt0();  // this slot's LDS reads are done before it is refilled
            issue(j + R, ring + sl * SLOT);
        }
        sl = sl + 1 == R ? 0 : sl + 1;
    }

    // partial sums -> LDS (ring space, once every wave is done with it), added in segment order
    __syncthreads();
    float4 *red = reinterpret_cast<float4 *>(mv_lds);
    if constexpr (GROUPED)
        red[wave * 64 + lane] = make_float4(facc[0], facc[1], facc[2], facc[3]);
    else
        red[wave * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (wave != 0) return;
    const int m = frow, n = n0 + 4 * fq;
    if (m >= M || n >= N) return;
    float4 t = red[lane];
    for (int w = 1; w < NW; ++w) {
        const float4 u = red[w * 64 + lane];
        t.x += u.x;
        t.y += u.y;
        t.z += u.z;
        t.w += u.w;
    }
    const int64_t off = (int64_t)m * p.ldy + n;
    if constexpr (GROUPED)
        store4(p.y, off, p.out, t.x, t.y, t.z, t.w);
    else
        store4(p.y, off, p.out, t.x * e_sw.x, t.y * e_sw.y, t.z * e_sw.z, t.w * e_sw.w);
}

template <int GS, bool BF16X, int XR>
hipError_t launch_mv_x(const GemmProblem &p, hipStream_t stream) {
    constexpr int SLOT = 2048 + XR * 1024;
    const int NCH = p.K / 128;
    const int blocks = (p.N + 15) / 16;
    // waves per workgroup as in the GEMV: segments of at most MV_RING chunks where possible,
    // at least about 2048 waves in the grid while each wave keeps 2 chunks or more
    int NW = min(MV_MAX_WAVES, max(1, (NCH + MV_RING - 1) / MV_RING));
    while (NW < MV_MAX_WAVES && (int64_t)blocks * NW < 2048 && NCH / (NW + 1) >= 2) ++NW;
    int seg = (NCH + NW - 1) / NW;
    NW = (NCH + seg - 1) / seg;
    const int table_groups = GS > 0 ? (seg * (128 / GS) + 3) & ~3 : 0;
    const size_t fixed = (size_t)NW * table_groups * 16 * sizeof(float);
    // ring slots: as many as fit while every workgroup of the grid is resident at once, else
    // as many as fit one workgroup per CU (at least 2, or the whole segment)
    const int per_cu = (blocks + num_cus() - 1) / num_cus();
    const int need = min(2, seg);
    int fit = (int)(((size_t)160 * 1024 / per_cu - min(fixed, (size_t)160 * 1024 / per_cu)) / ((size_t)NW * SLOT));
    if (fit < need) fit = (int)(((size_t)160 * 1024 - fixed) / ((size_t)NW * SLOT));
    // ring depth: about 40 KiB of weight slots per CU in flight. Deeper rings stream slower
    // (measured at M = 1: 7.1 against 7.5 us at N=10240 K=2560 with 2 instead of 4 slots,
    // 8.0 against 9.0 us at N=2560 K=10240 with 3 instead of 6)
    const int target = (20 + per_cu * NW - 1) / (per_cu * NW);
    const int slots = min(min(MV_RING, seg), min(fit, max(need, target)));
    if (slots < need) return hipErrorNotSupported;
    const size_t lds = (size_t)NW * slots * SLOT + fixed;
    if (lds < (size_t)NW * 64 * 16) return hipErrorNotSupported;  // room for the partial sums
    hipLaunchKernelGGL((mv_kernel<GS, BF16X, XR>), dim3(blocks), dim3(64 * NW), lds, stream, p, seg, slots,
                       table_groups);
    return hipGetLastError();
}

template <int GS, bool BF16X>
hipError_t launch_mv_gs(const GemmProblem &p, hipStream_t stream) {
    switch ((p.M + 3) / 4) {
        case 1: return launch_mv_x<GS, BF16X, 1>(p, stream);
        case 2: return launch_mv_x<GS, BF16X, 2>(p, stream);
        case 3: return launch_mv_x<GS, BF16X, 3>(p, stream);
        default: return launch_mv_x<GS, BF16X, 4>(p, stream);
    }
}

template <bool BF16X>
hipError_t launch_mv_t(const GemmProblem &p, hipStream_t stream) {
    if (p.gs == 64) return launch_mv_gs<64, BF16X>(p, stream);
    if (p.gs == 128) return launch_mv_gs<128, BF16X>(p, stream);
    return launch_mv_gs<0, BF16X>(p, stream);
}

}  // namespace

hipError_t launch_mv(const GemmProblem &p, hipStream_t stream) {
    if (p.x == nullptr || p.M < 1 || p.M > 16 || p.K % 128 != 0 || p.wkind != W_INT8 || p.out == OUT_I32)
        return hipErrorInvalidValue;
    return p.x_bf16 ? launch_mv_t<true>(p, stream) : launch_mv_t<false>(p, stream);
}

}  // namespace w8a8
