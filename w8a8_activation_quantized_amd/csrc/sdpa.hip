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
//  * Both products on the matrix cores (v_mfma_f32_16x16x32_{f16,bf16}): scores S^T =
//    K_block . q^T with the block's 16 keys as A rows (K rows loaded straight from HBM into the
//    operand) and the (up to 16) query heads as B columns; then o^T = P . V with V staged in
//    LDS and read transposed, P split into input-format parts so that the result keeps fp32
//    precision (see sdpa_kernel). Scores, the softmax and every sum are fp32.
//  * Online softmax per 32-key block in base 2: scores are scaled by scale * log2(e) once,
//    p = exp2(s - m), and the running sums are rescaled by exp2(m_old - m_new) per block.
#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>

#include "device_common.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef _Float16 sd_v8h __attribute__((ext_vector_type(8)));
typedef __bf16 sd_v8bf __attribute__((ext_vector_type(8)));
typedef float sd_v4f __attribute__((ext_vector_type(4)));

constexpr int SD_WAVES = 4;  // waves per workgroup
constexpr int SD_BK = 32;    // keys per block (two MFMA row tiles)

// v combined with the value of lane l ^ 16 (xor16) or l ^ 32 (xor32) by a commutative op:
// v_permlane16_swap / v_permlane32_swap on two copies of v leave each lane holding its own
// value and its partner's (swap16: rows (0, 1) and (2, 3) exchanged; swap32: the halves), a
// VALU lane exchange instead of an LDS-crossbar shuffle. Commutativity makes the result
// the same bits as op(v, partner) in every lane.
template <typename Op>
__device__ __forceinline__ float xor16_combine(float v, Op op) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto sw = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return op(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}
template <typename Op>
__device__ __forceinline__ float xor32_combine(float v, Op op) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto sw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return op(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}

// v_mfma_f32_16x16x32 on 8 values of the input format per lane (both products use it)
template <bool BF16>
__device__ __forceinline__ sd_v4f mma16x16x32(v4u a, v4u b, sd_v4f c) {
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

// Workgroup (slice, b * Hkv + kvh): four waves, each a contiguous quarter of the slice's keys,
// merged at the end.
//
// Per 32-key block of a wave: the K rows go straight from HBM into MFMA A operands (one block
// ahead in registers); the V rows go to a per-wave LDS buffer by global_load_lds (one block
// ahead, two buffers), 16-byte pieces of key row r at position piece ^ 2 ((r >> 3) & 3), so
// that the transposed reads of the P . V operands (16 lanes: 16 consecutive d of one key; 4
// lane groups: keys 8 apart) fall in different banks.
//
// P . V on the matrix cores: o^T tiles of 16 heads x 16 d, A = P [heads x 32 keys], B =
// V [32 keys x 16 d] read transposed from LDS. P (fp32) is split into parts of the input
// format whose sum is P to about fp32 precision (fp16: hi + lo; bf16: hi + mid + lo), each
// part one MFMA; the products with V are exact and accumulate in fp32. The probabilities are
// scaled by 2^12 (p = exp2(s - m + 12)) so the fp16 residual parts stay normal down to
// p = 2^-15 of the block maximum; the scale cancels in o / l.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * SD_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void sdpa_kernel(SdpaArgs a) {
    constexpr int T = D / 32;              // QK MFMAs per 16-key tile
    constexpr int DT = D / 16;             // P . V output tiles (16 d each)
    constexpr int PARTS = BF16 ? 3 : 2;    // pieces of P in the input format
    constexpr int VROW = 2 * D;            // bytes per V row
    constexpr int VBUF = SD_BK * VROW;     // bytes per V block
    constexpr int VDMA = VBUF / 1024;      // 1 KiB DMA instructions per V block
    constexpr int RPD = 1024 / VROW;       // V rows per DMA instruction
    constexpr int CPR = VROW / 16;         // 16-byte pieces per V row
    constexpr int PBUF = PARTS * 16 * SD_BK * 2;  // P parts [part][head][key], 2 bytes each
    static_assert(VBUF % 1024 == 0, "V block in whole DMA instructions");
    // separate arrays, so that the compiler sees the DMA-written V buffers and the P tiles as
    // distinct memory
    __shared__ __attribute__((aligned(1024))) int8_t vlds[SD_WAVES * 2 * VBUF];
    __shared__ __attribute__((aligned(16))) uint16_t plds[SD_WAVES * PBUF / 2];
    __shared__ float red_ml[SD_WAVES][2][16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.Hkv, kvh = bk % a.Hkv;
    const int G = a.G, N = a.N;
    const int s0 = (int)((int64_t)slice * N / a.slices), s1 = (int)((int64_t)(slice + 1) * N / a.slices);
    const int w0 = s0 + (int)((int64_t)wave * (s1 - s0) / SD_WAVES);
    const int w1 = s0 + (int)((int64_t)(wave + 1) * (s1 - s0) / SD_WAVES);
    const uint16_t *K = a.k + ((int64_t)b * a.Hkv + kvh) * a.Ncap * D;
    const uint16_t *V = a.v + ((int64_t)b * a.Hkv + kvh) * a.Ncap * D;
    int8_t *vbuf = vlds + wave * 2 * VBUF;  // two V blocks
    uint16_t *pbuf = plds + wave * PBUF / 2;

    // MFMA lane roles: row / column r16 = lane % 16, quarter q4 = lane / 16
    const int r16 = lane & 15, q4 = lane >> 4;
    // q^T columns (QK B operand): head r16 of the group (zero past G), d in [32 t + 8 q4, + 8)
    v4u qf[T];
    {
        const uint16_t *qh = a.q + ((int64_t)b * a.Hq + (int64_t)kvh * G + min(r16, G - 1)) * D;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const v4u x = *reinterpret_cast<const v4u *>(qh + 32 * t + 8 * q4);
            qf[t] = r16 < G ? x : v4u{0, 0, 0, 0};
        }
    }

    float m = -INFINITY, l = 0.f;  // of head r16 (QK layout; copies in the 4 quarters)
    sd_v4f o[DT];                  // o^T tiles: lane holds heads 4 q4 + e, d = 16 dt + r16
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = sd_v4f{0.f, 0.f, 0.f, 0.f};

    auto load_k = [&](int n0, v4u (&kf)[2][T]) __attribute__((always_inline)) {
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int row = min(n0 + 16 * tile + r16, w1 - 1);
#pragma unroll
            for (int t = 0; t < T; ++t) kf[tile][t] = *reinterpret_cast<const v4u *>(K + (int64_t)row * D + 32 * t + 8 * q4);
        }
    };
    auto load_v = [&](int n0, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VDMA; ++i) {
            const int r = RPD * i + lane / CPR, pc = lane % CPR;
            const int lc = pc ^ (2 * ((r >> 3) & 3));
            const int row = min(n0 + r, w1 - 1);
            dma_16B(V + (int64_t)row * D + 8 * lc, vbuf + buf * VBUF + i * 1024);
        }
    };
    auto block = [&](int n0, int buf, const v4u (&kf)[2][T]) __attribute__((always_inline)) {
        // scores: lane holds keys 16 tile + 4 q4 + e of head r16
        sd_v4f sc[2];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            sd_v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < T; ++t) acc = mma16x16x32<BF16>(kf[tile][t], qf[t], acc);
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
        bm = xor16_combine(bm, [](float u, float v) { return fmaxf(u, v); });
        bm = xor32_combine(bm, [](float u, float v) { return fmaxf(u, v); });
        const float mn = fmaxf(m, bm);  // finite: every block has a key below w1
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = __builtin_amdgcn_exp2f(s[i] - mn + 12.0f);  // 2^12 p
            ps += s[i];
        }
        ps = xor16_combine(ps, [](float u, float v) { return u + v; });
        ps = xor32_combine(ps, [](float u, float v) { return u + v; });
        l = l * alpha + ps;
        m = mn;
        // P parts to LDS, [part][head][key]: this lane's 4 consecutive keys of each tile
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            uint32_t w[PARTS][2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                float r0 = s[4 * tile + 2 * h2], r1 = s[4 * tile + 2 * h2 + 1];
#pragma unroll
                for (int pt = 0; pt < PARTS; ++pt) {
                    uint32_t b0, b1;
                    if constexpr (BF16) {
                        b0 = bf16_rne(r0);
                        b1 = bf16_rne(r1);
                        r0 -= __builtin_bit_cast(float, b0 << 16);
                        r1 -= __builtin_bit_cast(float, b1 << 16);
                    } else {
                        b0 = f16_bits(r0);
                        b1 = f16_bits(r1);
                        r0 -= (float)__builtin_bit_cast(_Float16, (uint16_t)b0);
                        r1 -= (float)__builtin_bit_cast(_Float16, (uint16_t)b1);
                    }
                    w[pt][h2] = b0 | (b1 << 16);
                }
            }
#pragma unroll
            for (int pt = 0; pt < PARTS; ++pt)
                *reinterpret_cast<uint2 *>(pbuf + (pt * 16 + r16) * SD_BK + 16 * tile + 4 * q4) =
                    make_uint2(w[pt][0], w[pt][1]);
        }
        // rescale o: heads 4 q4 + e take alpha from lane 4 q4 + e (head r16 = that lane)
        float al[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * q4 + e, 64);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dt][e] *= al[e];
        // this block's V has landed (only the next block's K loads and V DMA may be in flight)
        wait_lgkmcnt0();
        // P A operands: head r16, keys 8 q4 .. 8 q4 + 8
        v4u pa[PARTS];
#pragma unroll
        for (int pt = 0; pt < PARTS; ++pt) pa[pt] = *reinterpret_cast<const v4u *>(pbuf + (pt * 16 + r16) * SD_BK + 8 * q4);
        const int8_t *vb = vbuf + buf * VBUF;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            // V^T B operand: d = 16 dt + r16, keys 8 q4 + j (2-byte reads, transposed)
            const int d = 16 * dt + r16, lc = d >> 3, off = 2 * (d & 7);
            uint32_t hv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 8 * q4 + j;
                hv[j] = *reinterpret_cast<const uint16_t *>(vb + r * VROW + 16 * (lc ^ (2 * ((r >> 3) & 3))) + off);
            }
            const v4u vfrag = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
#pragma unroll
            for (int pt = 0; pt < PARTS; ++pt) o[dt] = mma16x16x32<BF16>(pa[pt], vfrag, o[dt]);
        }
    };

    // pipeline: block j + 1's K loads and V DMA go out before block j computes
    v4u ka[2][T], kb[2][T];
    int nblk = (w1 - w0 + SD_BK - 1) / SD_BK;
    if (nblk > 0) {
        load_k(w0, ka);
        load_v(w0, 0);
    }
    for (int j = 0; j < nblk; j += 2) {
        const int n0 = w0 + j * SD_BK;
        wait_lgkmcnt0();  // the other V buffer's reads (block j - 1) are done
        if (j + 1 < nblk) {
            load_k(n0 + SD_BK, kb);
            load_v(n0 + SD_BK, 1);
            wait_vmcnt<2 * T + VDMA>();
        } else {
            wait_vmcnt<0>();
        }
        block(n0, 0, ka);
        if (j + 1 >= nblk) break;
        wait_lgkmcnt0();
        if (j + 2 < nblk) {
            load_k(n0 + 2 * SD_BK, ka);
            load_v(n0 + 2 * SD_BK, 0);
            wait_vmcnt<2 * T + VDMA>();
        } else {
            wait_vmcnt<0>();
        }
        block(n0 + SD_BK, 1, kb);
    }

    // merge the waves: (m, l) per head and o^T tiles to LDS (the V buffers, now free)
    __syncthreads();
    float *red_o = reinterpret_cast<float *>(vlds);  // [wave][16 heads][D]
    static_assert(SD_WAVES * 16 * D * 4 <= SD_WAVES * 2 * VBUF, "merge buffer");
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) red_o[(wave * 16 + 4 * q4 + e) * D + 16 * dt + r16] = o[dt][e];
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
            acc += red_o[(w * 16 + g) * D + d] * f;
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

constexpr int SD_COMBINE_THREADS = 1024;
constexpr int SD_COMBINE_SPLIT = 8;  // workgroups per head in the merge (4: GQA 32/4, N = 32768: 17.7 against 18.6 us with 1; 8 against 4: 0.2-2.3 % faster over GQA 32/4 .. 32/32, N = 1024 .. 32768)

// Second pass: merge the slices of one (b, h). Thread (d, part) of 1024 merges every PARTS-th
// slice's (m, l, o[d]) into a running (M, L, A), eight slices at a time: their loads go out
// together, then the running sums are rescaled once to the new maximum. The PARTS states then
// meet in LDS.
template <int D, int SPLIT>
__global__ __launch_bounds__(SD_COMBINE_THREADS / SPLIT) void sdpa_combine_kernel(const float *part, void *o,
                                                                                  int slices, int out) {
    // SPLIT workgroups per head, each merging D / SPLIT columns with PARTS slice streams
    constexpr int PARTS = SD_COMBINE_THREADS / D, DC = D / SPLIT;
    __shared__ float st[3][PARTS][DC];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int dc = tid % DC, pt = tid / DC, d = blockIdx.y * DC + dc;
    const float *pp = part + (int64_t)bh * slices * (D + 4);
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int s0 = pt; s0 < slices; s0 += 8 * PARTS) {
        // eight slices' values, all loads issued before any is used (clamped addresses)
        float ms[8], ls[8], os[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int sv = s0 + i * PARTS;
            const bool ok = sv < slices;
            const float *q = pp + (int64_t)(ok ? sv : pt) * (D + 4);
            ms[i] = q[0];
            ls[i] = q[1];
            os[i] = q[4 + d];
            if (!ok) ms[i] = -INFINITY;
        }
        float mx = M;
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, ms[i]);
        // mx is finite: slice s0 exists
        const float f = __builtin_amdgcn_exp2f(M - mx);  // 0 while M = -inf
        L *= f;
        A *= f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float w = __builtin_amdgcn_exp2f(ms[i] - mx);  // 0 for the missing slices
            L += ls[i] * w;
            A += os[i] * w;
        }
        M = mx;
    }
    st[0][pt][dc] = M;
    st[1][pt][dc] = L;
    st[2][pt][dc] = A;
    __syncthreads();
    if (pt != 0) return;
    float Mx = M;
#pragma unroll
    for (int q = 1; q < PARTS; ++q) Mx = fmaxf(Mx, st[0][q][dc]);
    float Lt = 0.f, At = 0.f;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) {
        const float mq = st[0][q][dc];
        const float f = mq == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq - Mx);
        Lt += st[1][q][dc] * f;
        At += st[2][q][dc] * f;
    }
    const float y = At / Lt;
    const int64_t off = (int64_t)bh * D + d;
    if (out == OUT_F32)
        static_cast<float *>(o)[off] = y;
    else if (out == OUT_BF16)
        static_cast<uint16_t *>(o)[off] = (uint16_t)bf16_rne(y);
    else
        static_cast<uint16_t *>(o)[off] = (uint16_t)f16_bits(y);
}

template <int D, bool BF16>
hipError_t launch_sdpa_t(const SdpaArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((sdpa_kernel<D, BF16>), dim3(a.slices, a.B * a.Hkv), dim3(64 * SD_WAVES), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.slices == 1) return e;
    hipLaunchKernelGGL((sdpa_combine_kernel<D, SD_COMBINE_SPLIT>), dim3(a.B * a.Hq, SD_COMBINE_SPLIT),
                       dim3(SD_COMBINE_THREADS / SD_COMBINE_SPLIT), 0, stream, a.part, a.o, a.slices, a.out);
    return hipGetLastError();
}

}  // namespace

int sdpa_slices(int B, int Hkv, int N) {
    // about one workgroup per CU, each slice at least 128 keys (one block per wave); swept on
    // the box over 8 .. 256 slices for 4, 8 and 32 KV heads at N = 4096 and 32768
    const int64_t groups = (int64_t)B * Hkv;
    int s = (int)(((int64_t)num_cus() + groups - 1) / groups);
    s = std::min(s, std::max(1, N / 128));
    return std::max(1, std::min(s, 1024));
}

// Most slices any call may use: four times the rule's count (the autotuner's largest
// candidate), at least 128 keys per slice. The workspace query sizes for it, so a tuned
// count always fits a workspace of the queried size.
int sdpa_max_slices(int B, int Hkv, int N) {
    return std::max(1, std::min(std::min(4 * sdpa_slices(B, Hkv, N), std::max(1, N / 128)), 1024));
}

static int64_t part_bytes(int B, int Hq, int slices, int D) {
    return slices > 1 ? (int64_t)B * Hq * slices * (D + 4) * 4 : 0;
}

int64_t sdpa_workspace_bytes(int B, int Hq, int Hkv, int N, int D) {
    return part_bytes(B, Hq, sdpa_max_slices(B, Hkv, N), D);
}

// Tuned slice counts (the pages' AutoTune table): per device, input format, B, Hq, Hkv, D
// and the cache length rounded up to a power of two.
namespace {
using TuneKey = std::tuple<int, bool, int, int, int, int, int>;
std::mutex g_tune_mutex;
std::map<TuneKey, int> g_tuned;

int n_bucket(int N) {
    int b = 0;
    while ((1 << b) < N && b < 30) ++b;
    return b;
}

TuneKey tune_key(bool bf16, int B, int Hq, int Hkv, int N, int D) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    return TuneKey(dev, bf16, B, Hq, Hkv, D, n_bucket(N));
}

SdpaArgs make_args(const void *q, const void *k, const void *v, void *o, int out, int B, int Hq, int Hkv, int N,
                   int Ncap, float scale, void *ws, int slices) {
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
    a.slices = slices;
    a.part = static_cast<float *>(ws);
    return a;
}

hipError_t launch_args(const SdpaArgs &a, bool bf16, int D, hipStream_t stream) {
    if (D == 64) return bf16 ? launch_sdpa_t<64, true>(a, stream) : launch_sdpa_t<64, false>(a, stream);
    return bf16 ? launch_sdpa_t<128, true>(a, stream) : launch_sdpa_t<128, false>(a, stream);
}
}  // namespace

int sdpa_tuned_slices(bool bf16, int B, int Hq, int Hkv, int N, int D) {
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    const auto it = g_tuned.find(tune_key(bf16, B, Hq, Hkv, N, D));
    return it == g_tuned.end() ? 0 : it->second;
}

hipError_t launch_sdpa_decode(const void *q, const void *k, const void *v, bool bf16, void *o, int out, int B, int Hq,
                              int Hkv, int N, int Ncap, int D, float scale, void *ws, int64_t ws_bytes,
                              hipStream_t stream) {
    // the tuned count for this size class if there is one (at most N / 128 slices at this N),
    // else the rule; one slice when the workspace cannot hold the partials
    int slices = sdpa_tuned_slices(bf16, B, Hq, Hkv, N, D);
    slices = slices > 0 ? std::max(1, std::min(slices, std::max(1, N / 128))) : sdpa_slices(B, Hkv, N);
    if (slices > 1 && (ws == nullptr || ws_bytes < part_bytes(B, Hq, slices, D))) slices = 1;
    return launch_args(make_args(q, k, v, o, out, B, Hq, Hkv, N, Ncap, scale, ws, slices), bf16, D, stream);
}

hipError_t sdpa_autotune(const void *q, const void *k, const void *v, bool bf16, void *o, int out, int B, int Hq,
                         int Hkv, int N, int Ncap, int D, float scale, void *ws, int64_t ws_bytes, hipStream_t stream,
                         int *best_out) {
    // candidates: one slice, and the rule's count times 1/4, 1/2, 1, 2, 4 (at least 128 keys
    // each, partials within the workspace). Each is timed as a captured graph of 20 calls,
    // replayed once untimed and once timed on a private stream that first waits for the
    // caller's: issued one by one, a short call is bound by how fast the host launches its
    // two kernels, and the timing then ranks the candidates by noise. The rule's count is
    // kept unless another one is at least 3 % faster.
    constexpr int kCalls = 20;
    const int r = sdpa_slices(B, Hkv, N), smax = sdpa_max_slices(B, Hkv, N);
    int cand[6] = {1, std::max(1, r / 4), std::max(1, r / 2), r, 2 * r, 4 * r};
    hipStream_t ts = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr, ready = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&ts, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ready, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(ts, ready, 0);
    int best = 0;
    float best_ms = 0.f, rule_ms = -1.f;
    for (int i = 0; i < 6 && e == hipSuccess; ++i) {
        const int s = cand[i];
        if (s > smax || (s > 1 && (ws == nullptr || ws_bytes < part_bytes(B, Hq, s, D)))) continue;
        bool seen = false;
        for (int j = 0; j < i; ++j) seen = seen || cand[j] == s;
        if (seen) continue;
        const SdpaArgs a = make_args(q, k, v, o, out, B, Hq, Hkv, N, Ncap, scale, ws, s);
        hipGraph_t g = nullptr;
        hipGraphExec_t ge = nullptr;
        if ((e = hipStreamBeginCapture(ts, hipStreamCaptureModeThreadLocal)) != hipSuccess) break;
        hipError_t el = hipSuccess;
        for (int rep = 0; rep < kCalls && el == hipSuccess; ++rep) el = launch_args(a, bf16, D, ts);
        e = hipStreamEndCapture(ts, &g);  // always ends the capture, also after a failed launch
        if (e == hipSuccess) e = el;
        if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
        if (e == hipSuccess) e = hipGraphLaunch(ge, ts);
        if (e == hipSuccess) e = hipEventRecord(e0, ts);
        if (e == hipSuccess) e = hipGraphLaunch(ge, ts);
        if (e == hipSuccess) e = hipEventRecord(e1, ts);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (ge) (void)hipGraphExecDestroy(ge);
        if (g) (void)hipGraphDestroy(g);
        if (e != hipSuccess) break;
        if (s == r) rule_ms = ms;
        if (best == 0 || ms < best_ms) {
            best = s;
            best_ms = ms;
        }
    }
    if (e == hipSuccess && rule_ms > 0.f && best != r && best_ms > 0.97f * rule_ms) best = r;
    if (e == hipSuccess) e = hipStreamSynchronize(ts);
    if (ready) (void)hipEventDestroy(ready);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (ts) (void)hipStreamDestroy(ts);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lock(g_tune_mutex);
        g_tuned[tune_key(bf16, B, Hq, Hkv, N, D)] = best;
    }
    if (best_out) *best_out = best;
    return hipSuccess;
}

}  // namespace w8a8
