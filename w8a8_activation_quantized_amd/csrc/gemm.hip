// int8 GEMM with fused dequantization for gfx950 (CDNA4) matrix cores.
//
// Computes, for x_q [M, K] int8 (row-major) and w_q [N, K] int8 (row-major, one row
// per output channel):
//   acc[m, n] = sum_k x_q[m, k] * w_q[n, k]             exact int32 (MFMA i8 -> i32)
// and then, in the store stage, one of (juejin post "在Mac上跑大模型，MLX 不是终点",
// sections "W8A8 对称量化" and "三种量化粒度的实现"; Cider README "量化"):
//   per-channel:  y = (fp32(acc) * s_x[m]) * s_w[n]
//   per-group:    t = 0; for each K-group g ascending: t = fma(fp32(acc_g), s_w[n, g], t);
//                 y = t * s_x[m]
// For W4A8 the weight tile arrives as packed nibbles (u = q + 8, even k low) and is
// unpacked to int8 codes while it is written to LDS (README "Metal Kernel 流水线":
// the unpack is part of the operand load); the rest is the per-group path.
//
// Design (MI355X-first):
//  * v_mfma_i32_16x16x64_i8: each lane feeds 16 contiguous K-bytes of one row of
//    each operand. Both operands are K-contiguous in HBM, so tiles are copied to
//    LDS row-major and read back as 16-byte fragments (ds_read_b128).
//  * The weight tile is the MFMA "A" operand and the activation tile the "B"
//    operand, so each lane's four accumulator values are four consecutive output
//    channels n of one token m: the epilogue writes 8 (fp16/bf16) or 16 (fp32)
//    contiguous bytes per lane.
//  * LDS rows are BK bytes; 16-byte chunks are XOR-swizzled by row: chunk ^ ((row >> 1)
//    & 7) for 128-byte rows, chunk ^ ((row >> 1) & 3) for 64-byte rows. Measured on
//    gfx950 with SQ_LDS_BANK_CONFLICT: these fragment-read patterns (16 rows x one
//    logical chunk per 16 lanes) run without conflicts, where an unswizzled 128-byte
//    layout takes 4x the cycles; for 64-byte rows, (row >> 2) & 3, (row >> 3) & 3,
//    row & 3 and no swizzle all lose a quarter of the LDS cycles to conflicts.
//  * Two LDS stages: global loads for tile k+1 are issued into registers before the
//    MFMAs of tile k and written to the other stage afterwards; one barrier per
//    K-tile.
//  * Workgroup -> tile mapping is XCD-aware: the hardware deals workgroups to the
//    8 XCDs round-robin, so the block id is remapped to give each XCD a contiguous
//    run of tiles, which are then walked in groups of GROUP_M tile-rows so the
//    tiles that run together on one XCD share activation and weight panels in
//    that XCD's L2.
//  * Ragged M and N: out-of-range rows are clamped to the last valid row for
//    loads (always in bounds) and masked at the store. A K that is a multiple of 64
//    but not of the 128-byte K-tile ends in a half tile whose missing chunks are
//    loaded from a clamped address and replaced by zero codes (int4: nibble 8),
//    which add nothing to the integer sums.
#include <atomic>
#include <type_traits>

#include "act_quant.h"
#include "device_common.h"
#include "internal.h"

namespace w8a8 {
namespace {

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a swizzled [rows][BK] tile.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
    if constexpr (BK == 128)
        return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
    else
        return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4);
}

// Largest K for int32 sums of 16 q (int4 weights unpacked as 16 q, see unpack_nibbles_x16)
// over all of K: |16 sum| <= 16 K 128 8 < 2^31 needs K < 131072 (codes -128 are accepted),
// and the kernels that use it take K in whole 128-value K-tiles.
constexpr int kInt4X16MaxK = 131072 - 128;

// Eight packed bytes (two dwords; 16 nibbles, even k in the low nibble) -> sixteen int8
// codes q = u - 8 in k order.
__device__ __forceinline__ uint32_t interleave_lo(uint32_t lo, uint32_t hi) {
    // bytes [lo0, hi0, lo1, hi1]
    return (lo & 0xFFu) | ((hi & 0xFFu) << 8) | ((lo & 0xFF00u) << 8) | ((hi & 0xFF00u) << 16);
}
__device__ __forceinline__ uint32_t interleave_hi(uint32_t lo, uint32_t hi) {
    // bytes [lo2, hi2, lo3, hi3]
    return ((lo >> 16) & 0xFFu) | (((hi >> 16) & 0xFFu) << 8) | ((lo >> 8) & 0xFF0000u) | (hi & 0xFF000000u);
}
__device__ __forceinline__ uint32_t recentre(uint32_t u4) {
    // per byte u - 8 without borrows: u + 0x78 stays below 0x100, xor 0x80 recentres
    return (u4 + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ v4u unpack_nibbles(uint32_t d0, uint32_t d1) {
    const uint32_t lo0 = d0 & 0x0F0F0F0Fu, hi0 = (d0 >> 4) & 0x0F0F0F0Fu;
    const uint32_t lo1 = d1 & 0x0F0F0F0Fu, hi1 = (d1 >> 4) & 0x0F0F0F0Fu;
    return v4u{recentre(interleave_lo(lo0, hi0)), recentre(interleave_hi(lo0, hi0)),
               recentre(interleave_lo(lo1, hi1)), recentre(interleave_hi(lo1, hi1))};
}

// Eight packed bytes -> sixteen int8 values 16 q in k order, q = u - 8. u ^ 8 is the 4-bit
// two's complement of q; placed in the high half of a byte it reads as the int8 16 q. Per
// dword: one xor, two masks (one after a shift) and two byte permutes; the MFMA sums are
// then 16 x the int4 sums, exactly.
__device__ __forceinline__ v4u unpack_nibbles_x16(uint32_t d0, uint32_t d1) {
    const uint32_t e0 = d0 ^ 0x88888888u, e1 = d1 ^ 0x88888888u;
    const uint32_t h0 = e0 & 0xF0F0F0F0u, l0 = (e0 << 4) & 0xF0F0F0F0u;  // odd k, even k
    const uint32_t h1 = e1 & 0xF0F0F0F0u, l1 = (e1 << 4) & 0xF0F0F0F0u;
    // v_perm_b32: selector byte i picks byte i of {h (bytes 4-7), l (bytes 0-3)}
    return v4u{__builtin_amdgcn_perm(h0, l0, 0x05010400u), __builtin_amdgcn_perm(h0, l0, 0x07030602u),
               __builtin_amdgcn_perm(h1, l1, 0x05010400u), __builtin_amdgcn_perm(h1, l1, 0x07030602u)};
}

struct TileMap {
    int tiles_m, tiles_n, group_m;
};

// Logical tile index -> (tile_m, tile_n): group_m M-tiles side by side, N-tiles in order
// within a group, so consecutive logical tiles share activation and weight panels.
__device__ __forceinline__ void logical_tile(const TileMap &t, int logical, int &tm, int &tn) {
    const int per_group = t.group_m * t.tiles_n;
    const int grp = logical / per_group;
    const int first_m = grp * t.group_m;
    const int gsize = min(t.tiles_m - first_m, t.group_m);
    const int in_grp = logical - grp * per_group;
    tm = first_m + in_grp % gsize;
    tn = in_grp / gsize;
}

// XCD-aware block -> (tile_m, tile_n). Workgroups are dealt to the 8 XCDs round-robin
// (block b runs on XCD b % 8), so XCD x is given one contiguous run of logical tiles and
// its L2 sees the panels of that run only.
__device__ __forceinline__ void map_tile(const TileMap &t, int &tm, int &tn) {
    const int T = t.tiles_m * t.tiles_n;
    const int b = blockIdx.x;
    const int x = b & 7, i = b >> 3;
    const int q = T >> 3, r = T & 7;
    logical_tile(t, x * q + min(x, r) + i, tm, tn);
}

// Split-K: block -> (tile_m, tile_n, K-slice). The units are the tiles times the slices,
// slice-major: the run of units that one XCD is given covers neighbouring tiles of one
// slice, which share that slice's activation and weight panels in the XCD's L2.
__device__ __forceinline__ void map_unit(const TileMap &t, int slices, int &tm, int &tn, int &ks) {
    const int T = t.tiles_m * t.tiles_n, U = T * slices;
    const int b = blockIdx.x;
    const int x = b & 7, i = b >> 3;
    const int q = U >> 3, r = U & 7;
    const int L = x * q + min(x, r) + i;
    ks = L / T;
    logical_tile(t, L - ks * T, tm, tn);
}

// K-tiles [kt0, kt0 + KT) of slice ks: the KTT K-tiles dealt as evenly as whole tiles allow.
__device__ __forceinline__ void slice_range(int KTT, int slices, int ks, int &kt0, int &KT) {
    kt0 = ks * KTT / slices;
    KT = (ks + 1) * KTT / slices - kt0;
}

// Compile-time shape of one kernel instantiation.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int GS_, int WK_>
struct Shape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, GS = GS_, WK = WK_;
    static constexpr int NT = 64 * WGM * WGN;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int CPR = BK / 16;  // 16-byte chunks per LDS row
    static constexpr int KSTEPS = BK / 64;
    static constexpr bool GROUPED = GS > 0;
    static constexpr int GPT = GROUPED ? BK / GS : 1;  // groups per K-tile
    static constexpr int KS_PER_G = GROUPED ? GS / 64 : 1;
    static constexpr int W_TILE = BN * BK, X_TILE = BM * BK, STAGE = W_TILE + X_TILE;
    static constexpr int W_LOADS = (WK == W_INT4 ? BN * CPR / 2 : BN * CPR);
    static constexpr int X_LOADS = BM * CPR;
    static constexpr int WL = W_LOADS / NT, XL = X_LOADS / NT;
    static constexpr int SW_N = GROUPED ? BN * GPT : 0;
    static constexpr int SWL = GROUPED ? (SW_N + NT - 1) / NT : 1;
    static_assert(!GROUPED || BK % GS == 0, "a K-tile must hold whole groups");
    static_assert(W_LOADS % NT == 0 && X_LOADS % NT == 0, "loader shape");
};

// Issue the global loads of K-tile kt into registers.
template <class S>
__device__ __forceinline__ void tile_gload(const GemmProblem &p, int kt, int tid, int m0, int n0,
                                           v4u (&wreg)[S::WL], v4u (&xreg)[S::XL],
                                           float (&swreg)[S::SWL]) {
    const int k0 = kt * S::BK;
    const int M = p.M, N = p.N, K = p.K;
#pragma unroll
    for (int i = 0; i < S::WL; ++i) {
        const int c = tid + i * S::NT;
        if constexpr (S::WK == W_INT4) {
            const int row = c / (S::CPR / 2), pc = c % (S::CPR / 2);
            const int n = min(n0 + row, N - 1);
            const int kk = k0 + pc * 32;  // first code of this 16-byte packed chunk
            const v4u v = *reinterpret_cast<const v4u *>(static_cast<const uint8_t *>(p.wq) +
                                                         (int64_t)n * (K / 2) + min(kk, K - 32) / 2);
            wreg[i] = kk < K ? v : v4u{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
        } else {
            const int row = c / S::CPR, cc = c % S::CPR;
            const int n = min(n0 + row, N - 1);
            const int kk = k0 + cc * 16;
            const v4u v = *reinterpret_cast<const v4u *>(static_cast<const int8_t *>(p.wq) +
                                                         (int64_t)n * K + min(kk, K - 16));
            wreg[i] = kk < K ? v : v4u{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int i = 0; i < S::XL; ++i) {
        const int c = tid + i * S::NT;
        const int row = c / S::CPR, cc = c % S::CPR;
        const int m = min(m0 + row, M - 1);
        const int kk = k0 + cc * 16;
        const v4u v = *reinterpret_cast<const v4u *>(p.xq + (int64_t)m * K + min(kk, K - 16));
        xreg[i] = kk < K ? v : v4u{0u, 0u, 0u, 0u};
    }
    if constexpr (S::GROUPED) {
        const int G = K / S::GS;
#pragma unroll
        for (int i = 0; i < S::SWL; ++i) {
            const int idx = tid + i * S::NT;
            if (idx < S::SW_N) {
                const int j = idx / S::BN, nn = idx % S::BN;
                const int n = min(n0 + nn, N - 1);
                const int g = kt * S::GPT + j;
                swreg[i] = g < G ? p.sw[(int64_t)n * G + g] : 0.f;
            }
        }
    }
}

// Write the registers of one K-tile into LDS stage `stage` (int4 weights unpacked here).
template <class S>
__device__ __forceinline__ void tile_lstore(int8_t *smem, float *s_sw, int stage, int tid,
                                            const v4u (&wreg)[S::WL], const v4u (&xreg)[S::XL],
                                            const float (&swreg)[S::SWL]) {
    int8_t *Ws = smem + stage * S::STAGE;
    int8_t *Xs = Ws + S::W_TILE;
#pragma unroll
    for (int i = 0; i < S::WL; ++i) {
        const int c = tid + i * S::NT;
        if constexpr (S::WK == W_INT4) {
            const int row = c / (S::CPR / 2), pc = c % (S::CPR / 2);
            const v4u v = wreg[i];
            const v4u lo = unpack_nibbles(v[0], v[1]), hi = unpack_nibbles(v[2], v[3]);
            *reinterpret_cast<v4u *>(Ws + swz<S::BK>(row, 2 * pc)) = lo;
            *reinterpret_cast<v4u *>(Ws + swz<S::BK>(row, 2 * pc + 1)) = hi;
        } else {
            const int row = c / S::CPR, cc = c % S::CPR;
            *reinterpret_cast<v4u *>(Ws + swz<S::BK>(row, cc)) = wreg[i];
        }
    }
#pragma unroll
    for (int i = 0; i < S::XL; ++i) {
        const int c = tid + i * S::NT;
        const int row = c / S::CPR, cc = c % S::CPR;
        *reinterpret_cast<v4u *>(Xs + swz<S::BK>(row, cc)) = xreg[i];
    }
    if constexpr (S::GROUPED) {
#pragma unroll
        for (int i = 0; i < S::SWL; ++i) {
            const int idx = tid + i * S::NT;
            if (idx < S::SW_N) s_sw[stage * S::SW_N + idx] = swreg[i];
        }
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, int GS, int WK>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmProblem p, TileMap tmap) {
    using S = Shape<BM, BN, BK, WGM, WGN, GS, WK>;
    constexpr int FM = S::FM, FN = S::FN, WM = S::WM, WN = S::WN;
    constexpr bool GROUPED = S::GROUPED;

    __shared__ __attribute__((aligned(16))) int8_t smem[2 * S::STAGE];
    __shared__ __attribute__((aligned(16))) float s_sw[GROUPED ? 2 * S::SW_N : 4];

    int tm, tn;
    map_tile(tmap, tm, tn);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WGM, wn = wave / WGM;
    const int m0 = tm * BM, n0 = tn * BN;

    v4u wreg[S::WL], xreg[S::XL];
    float swreg[S::SWL];

    v4i acc[FN][FM];
    float facc[GROUPED ? FN : 1][GROUPED ? FM : 1][4];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    if constexpr (GROUPED) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) facc[i][j][e] = 0.f;
    }

    const int KT = (p.K + BK - 1) / BK;  // K % 64 == 0: a last half tile is zero-filled
    const int frow = lane & 15, fchunk = lane >> 4;
    tile_gload<S>(p, 0, tid, m0, n0, wreg, xreg, swreg);
    tile_lstore<S>(smem, s_sw, 0, tid, wreg, xreg, swreg);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) tile_gload<S>(p, kt + 1, tid, m0, n0, wreg, xreg, swreg);
        const int8_t *Ws = smem + cur * S::STAGE;
        const int8_t *Xs = Ws + S::W_TILE;
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) {
            v4i a[FN], b[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                a[fn] = *reinterpret_cast<const v4i *>(Ws + swz<BK>(wn * WN + fn * 16 + frow, ks * 4 + fchunk));
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                b[fm] = *reinterpret_cast<const v4i *>(Xs + swz<BK>(wm * WM + fm * 16 + frow, ks * 4 + fchunk));
            if constexpr (GROUPED) {
                const bool first = (ks % S::KS_PER_G) == 0;
                const bool last = (ks % S::KS_PER_G) == S::KS_PER_G - 1;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
                        acc[fn][fm] = mfma_i8(a[fn], b[fm], first ? v4i{0, 0, 0, 0} : acc[fn][fm]);
                if (last) {
                    const int j = ks / S::KS_PER_G;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const float4 s4 = *reinterpret_cast<const float4 *>(
                            s_sw + cur * S::SW_N + j * BN + wn * WN + fn * 16 + 4 * fchunk);
#pragma unroll
                        for (int fm = 0; fm < FM; ++fm) {
                            facc[fn][fm][0] = __builtin_fmaf((float)acc[fn][fm][0], s4.x, facc[fn][fm][0]);
                            facc[fn][fm][1] = __builtin_fmaf((float)acc[fn][fm][1], s4.y, facc[fn][fm][1]);
                            facc[fn][fm][2] = __builtin_fmaf((float)acc[fn][fm][2], s4.z, facc[fn][fm][2]);
                            facc[fn][fm][3] = __builtin_fmaf((float)acc[fn][fm][3], s4.w, facc[fn][fm][3]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_i8(a[fn], b[fm], acc[fn][fm]);
            }
        }
        if (kt + 1 < KT) tile_lstore<S>(smem, s_sw, cur ^ 1, tid, wreg, xreg, swreg);
        __syncthreads();
    }

    // ---- epilogue: dequant + store -------------------------------------------------
    const int out = p.out;
    const int M = p.M, N = p.N;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * WM + fm * 16 + frow;
        const bool mok = m < M;
        const float sxm = mok ? p.sx[m] : 0.f;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + wn * WN + fn * 16 + 4 * fchunk;
            if (!mok || n >= N) continue;
            const int64_t off = (int64_t)m * p.ldy + n;
            if constexpr (GROUPED) {
                store4(p.y, off, out, facc[fn][fm][0] * sxm, facc[fn][fm][1] * sxm, facc[fn][fm][2] * sxm,
                       facc[fn][fm][3] * sxm);
            } else {
                const v4i v = acc[fn][fm];
                if (out == OUT_I32) {
                    *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = make_int4(v[0], v[1], v[2], v[3]);
                } else {
                    const float4 s4 = *reinterpret_cast<const float4 *>(p.sw + n);
                    store4(p.y, off, out, ((float)v[0] * sxm) * s4.x, ((float)v[1] * sxm) * s4.y,
                           ((float)v[2] * sxm) * s4.z, ((float)v[3] * sxm) * s4.w);
                }
            }
        }
    }
}

// ---- direct-to-LDS multi-stage pipeline (per-channel / raw int32) -------------------
//
// BN x BM output tile (BN weight rows, BM token rows), 128-byte K-tiles, STAGES LDS
// stages of (BN + BM) x 128 bytes. Tiles are copied L2 -> LDS with
// global_load_lds_dwordx4 (no VGPR staging): one instruction moves 1 KiB = 8 rows x 128
// bytes, lane i writing LDS bytes [16 i, 16 i + 16) of that block, so the chunk swizzle
// is applied on the global side (lane i fetches logical chunk (i % 8) ^ ((row >> 1) & 7)
// of its row). 128-byte row segments matter: measured on gfx950, DMA of 128-byte row
// segments streams at ~58 B/clk per CU, 64-byte segments at ~39.
// Each wave keeps the fragments of one 64-byte K-step in registers while the MFMAs of
// the other run:
//
//   loop kt:  DMA stage kt+STAGES-1 into the buffer freed by stage kt-1
//             read frags(kt, ks1);  MFMAs(ks0)
//             retire own LDS reads and own DMA of stage kt+1; barrier
//             read frags(kt+1, ks0); MFMAs(ks1); retire those reads
//
// With 3 stages the DMA of a stage has about 1.5 K-tiles of MFMA time to land.

template <int BN_, int BM_, int STAGES_, int WGN_, int WGM_>
struct MsShape {
    static constexpr int BN = BN_, BM = BM_, BK = 128, STAGES = STAGES_, WGN = WGN_, WGM = WGM_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int W_TILE = BN * BK, STAGE = (BM + BN) * BK;
    static constexpr int GROUPS = (BM + BN) / 8;          // 1 KiB row groups per stage
    static constexpr int GPW = (GROUPS + NW - 1) / NW;    // DMA instructions per wave (max)
    static constexpr int FULL_WAVES = GROUPS - (GPW - 1) * NW;  // waves that issue GPW, others GPW-1
    static_assert(BN % 8 == 0 && BM % 8 == 0 && WN % 16 == 0 && WM % 16 == 0, "tile shape");
    static_assert(STAGES * STAGE <= 163840, "LDS");
};

template <class S>
__device__ __forceinline__ void ms_issue(const int8_t *const (&src)[S::GPW], int koff, int8_t *stage_base,
                                         int wave) {
#pragma unroll
    for (int j = 0; j < S::GPW; ++j) {
        if (j < S::GPW - 1 || wave < S::FULL_WAVES)
            dma_16B(src[j] + koff, stage_base + (wave + j * S::NW) * 1024);
    }
}

// vmcnt wait for "all but the last `stages_after` stages of this wave's DMA".
template <class S>
__device__ __forceinline__ void ms_wait_dma(int stages_after, int wave) {
    constexpr int G = S::GPW, g = S::GPW - 1;
    const bool full = wave < S::FULL_WAVES;
    if (stages_after <= 0) {
        wait_vmcnt<0>();
    } else if (stages_after == 1) {
        if (full) wait_vmcnt<G>(); else wait_vmcnt<g>();
    } else {
        if (full) wait_vmcnt<(2 * G < 63 ? 2 * G : 63)>(); else wait_vmcnt<(2 * g < 63 ? 2 * g : 63)>();
    }
}

template <class S>
__device__ __forceinline__ void ms_frags(const int8_t *st, int ks, int wm, int wn, int frow, int fchunk,
                                         v4i (&a)[S::FN], v4i (&b)[S::FM]) {
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn)
        a[fn] = *reinterpret_cast<const v4i *>(st + swz<128>(wn * S::WN + fn * 16 + frow, ks * 4 + fchunk));
#pragma unroll
    for (int fm = 0; fm < S::FM; ++fm)
        b[fm] = *reinterpret_cast<const v4i *>(st + S::W_TILE +
                                               swz<128>(wm * S::WM + fm * 16 + frow, ks * 4 + fchunk));
}

// Byte stride of a 16-bit output row staged in LDS: 16 bytes of padding against bank
// conflicts between the 16 rows one MFMA fragment writes, when the pipeline buffers
// have room for it.
template <class S>
constexpr int ms_out_row_stride() {
    static_assert(S::BM * S::BN * 2 <= S::STAGES * S::STAGE, "staged output tile must fit the LDS buffers");
    return S::BM * (S::BN * 2 + 16) <= S::STAGES * S::STAGE ? S::BN * 2 + 16 : S::BN * 2;
}

template <class S>
__device__ __forceinline__ void ms_mma(v4i (&acc)[S::FN][S::FM], const v4i (&a)[S::FN], const v4i (&b)[S::FM]) {
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < S::FM; ++fm) acc[fn][fm] = mfma_i8(a[fn], b[fm], acc[fn][fm]);
}

// SPLIT: the workgroup runs one K-slice of its tile and stores the int32 sums of that slice
// to p.ws (slice-major, [M, N] each); the dequantization happens after all slices.
template <int BN, int BM, int STAGES, int WGN, int WGM, bool SPLIT>
// Declared for 512 threads even when launched with 4 waves: at that bound the compiler
// budgets 256 registers per wave and keeps the MFMA accumulators in arch VGPRs, each MFMA
// accumulating in place. With a 256-thread bound it moves them to AGPRs without tying
// source and destination, and copies every accumulator back at the loop edge.
__global__ __launch_bounds__(512) void gemm_ms_kernel(GemmProblem p, TileMap tmap) {
    using S = MsShape<BN, BM, STAGES, WGN, WGM>;
    constexpr int FM = S::FM, FN = S::FN, GPW = S::GPW;
    __shared__ __attribute__((aligned(1024))) int8_t smem[STAGES * S::STAGE];

    int tm, tn, ks = 0;
    if constexpr (SPLIT)
        map_unit(tmap, p.ksplit, tm, tn, ks);
    else
        map_tile(tmap, tm, tn);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WGN, wm = wave / WGN;
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    int kt0 = 0, KT = K / S::BK;
    if constexpr (SPLIT) slice_range(K / S::BK, p.ksplit, ks, kt0, KT);

    // Loader: wave w issues row groups g = w + j * NW of each stage (groups below BN / 8
    // are weight rows, the rest token rows); lane i covers row 8 g + i / 8 of the stage.
    const int8_t *src[GPW];
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int g = min(wave + j * S::NW, S::GROUPS - 1);
        const bool is_w = g < BN / 8;
        const int lrow = (is_w ? g : g - BN / 8) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((lrow >> 1) & 7);
        const int grow = is_w ? min(n0 + lrow, N - 1) : min(m0 + lrow, M - 1);
        src[j] = (is_w ? static_cast<const int8_t *>(p.wq) : p.xq) + ((int64_t)grow * K + kt0 * S::BK + 16 * c);
    }

    v4i acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int frow = lane & 15, fchunk = lane >> 4;
    // prologue: stages 0 .. STAGES-2 in flight, wait for stage 0
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < KT) ms_issue<S>(src, s * S::BK, smem + s * S::STAGE, wave);
    ms_wait_dma<S>(min(STAGES - 2, KT - 1), wave);
    lds_barrier();

    v4i a0[FN], b0[FM], a1[FN], b1[FM];
    ms_frags<S>(smem, 0, wm, wn, frow, fchunk, a0, b0);
    wait_lgkmcnt0();
    int cur = 0;  // buffer of stage kt
    for (int kt = 0; kt < KT; ++kt) {
        // the buffer of stage kt-1 was released by the barrier of the previous iteration
        const int fill = kt + STAGES - 1;
        if (fill < KT) {
            int fb = cur + STAGES - 1;
            fb -= fb >= STAGES ? STAGES : 0;
            ms_issue<S>(src, fill * S::BK, smem + fb * S::STAGE, wave);
        }
        const int8_t *st = smem + cur * S::STAGE;
        ms_frags<S>(st, 1, wm, wn, frow, fchunk, a1, b1);
        ms_mma<S>(acc, a0, b0);
        wait_lgkmcnt0();
        if (kt + 1 < KT) {
            // DMA issued after stage kt+1: stages kt+2 .. min(kt+STAGES-1, KT-1)
            ms_wait_dma<S>(min(STAGES - 2, KT - 2 - kt), wave);
            lds_barrier();
            int nb = cur + 1;
            nb -= nb >= STAGES ? STAGES : 0;
            ms_frags<S>(smem + nb * S::STAGE, 0, wm, wn, frow, fchunk, a0, b0);
            cur = nb;
        }
        ms_mma<S>(acc, a1, b1);
        wait_lgkmcnt0();
    }

    if constexpr (SPLIT) {
        int32_t *ws = static_cast<int32_t *>(p.ws) + (int64_t)ks * M * N;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + wm * S::WM + fm * 16 + frow;
            if (m >= M) continue;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = n0 + wn * S::WN + fn * 16 + 4 * fchunk;
                if (n >= N) continue;
                const v4i v = acc[fn][fm];
                *reinterpret_cast<int4 *>(ws + (int64_t)m * N + n) = make_int4(v[0], v[1], v[2], v[3]);
            }
        }
        return;
    }

    // ---- epilogue (per-channel dequant or raw int32) ----
    // All scale loads are issued before the first store: y may alias nothing the
    // compiler can see, so loads placed between stores would each be serialized
    // behind the previous store.
    const float *__restrict__ sxp = p.sx;
    const float *__restrict__ swp = p.sw;
    float sxm[FM];
    float4 s4[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sxm[fm] = sxp[min(m0 + wm * S::WM + fm * 16 + frow, M - 1)];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        s4[fn] = *reinterpret_cast<const float4 *>(swp + min(n0 + wn * S::WN + fn * 16 + 4 * fchunk, N - 4));
    const int out = p.out;
    if ((out == OUT_F16 || out == OUT_BF16) && p.y_rows16) {
        // 16-bit outputs go through LDS (the pipeline buffers are free once every wave has
        // passed the barrier below) so that global stores are whole 16-byte pieces of
        // output rows: lane-contiguous runs of a row instead of the MFMA layout's 8-byte
        // pieces of 16 different rows, which store at about 60% of the rate.
        constexpr int RS = ms_out_row_stride<S>();
        // staged and stored in two halves, rows [WM/2 h, WM/2 (h + 1)) of each wave row's WM:
        // the second half is converted while the first half's stores go out
        constexpr int CPR = S::BN / 8, HF = FM / 2, HR = S::WM / 2, ITS = S::BM / 2 * CPR / S::NT;
        static_assert(FM % 2 == 0 && S::BM / 2 * CPR % S::NT == 0, "staged halves");
        const int rows = min(S::BM, M - m0), cols = min(S::BN, N - n0);
        auto stage = [&](int fm) __attribute__((always_inline)) {
            const int lr = wm * S::WM + fm * 16 + frow;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const v4i v = acc[fn][fm];
                const float y0 = ((float)v[0] * sxm[fm]) * s4[fn].x, y1 = ((float)v[1] * sxm[fm]) * s4[fn].y;
                const float y2 = ((float)v[2] * sxm[fm]) * s4[fn].z, y3 = ((float)v[3] * sxm[fm]) * s4[fn].w;
                const uint2 w = out == OUT_F16 ? make_uint2(f16_bits(y0) | (f16_bits(y1) << 16), f16_bits(y2) | (f16_bits(y3) << 16))
                                               : make_uint2(bf16_rne(y0) | (bf16_rne(y1) << 16), bf16_rne(y2) | (bf16_rne(y3) << 16));
                *reinterpret_cast<uint2 *>(smem + lr * RS + 2 * (wn * S::WN + fn * 16 + 4 * fchunk)) = w;
            }
        };
        auto store = [&](int h, int it) __attribute__((always_inline)) {
            const int c = tid + it * S::NT;
            const int rr = c / CPR, cc = c - rr * CPR;
            const int r = (rr % HR) + (rr / HR) * S::WM + h * HR;
            if (r < rows && cc * 8 < cols) {
                const v4u v = *reinterpret_cast<const v4u *>(smem + r * RS + 16 * cc);
                // streaming store (see pp_store_staged)
                __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(static_cast<uint16_t *>(p.y) + ((int64_t)(m0 + r) * p.ldy + n0 + cc * 8)));
            }
        };
        lds_barrier();
#pragma unroll
        for (int fm = 0; fm < HF; ++fm) stage(fm);
        lds_barrier();
#pragma unroll
        for (int q = 0; q < HF; ++q) {
#pragma unroll
            for (int it = q * ITS / HF; it < (q + 1) * ITS / HF; ++it) store(0, it);
            stage(HF + q);
        }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < ITS; ++it) store(1, it);
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * S::WM + fm * 16 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + wn * S::WN + fn * 16 + 4 * fchunk;
            if (n >= N) continue;
            const int64_t off = (int64_t)m * p.ldy + n;
            const v4i v = acc[fn][fm];
            if (out == OUT_I32) {
                *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = make_int4(v[0], v[1], v[2], v[3]);
            } else {
                store4(p.y, off, out, ((float)v[0] * sxm[fm]) * s4[fn].x, ((float)v[1] * sxm[fm]) * s4[fn].y,
                       ((float)v[2] * sxm[fm]) * s4[fn].z, ((float)v[3] * sxm[fm]) * s4[fn].w);
            }
        }
    }
}

// ---- per-channel, two wave groups in alternation ("ping-pong") -----------------------
//
// BN x BM tile (weights x tokens), 64-value K-steps, STAGES LDS stages filled by
// global_load_lds, eight waves in two groups of four. Group g owns tokens
// [g BM/2, (g+1) BM/2) of the tile and wave q of a group owns weight rows [q BN/4,
// (q+1) BN/4), so each SIMD holds one wave of each group. Every K-step has two phases
// separated by workgroup barriers; group 1 starts one phase late (one extra barrier),
// so while one group issues its MFMAs the other reads its next fragments from LDS and
// issues its share of the DMA for a later stage. The matrix pipe of each SIMD then
// alternates between the two waves instead of idling while both wait on LDS at once,
// which is what a single barrier per K-tile with all waves in step leaves it doing.
//
// Stage j is read by group 0 in phase 2j and by group 1 in phase 2j+1. Each wave waits
// for its own DMA of stage j+1 at the end of its memory phase of K-step j, so both
// groups' parts of a stage have landed by the barrier before its first reader; the
// buffer of stage j-1 is refilled (with stage j+STAGES-1) in the memory phase of K-step
// j, which follows both groups' reads of it.
// BKS: K bytes per stage row. 64: a stage holds one K-step, 16 rows of 64 bytes per DMA
// piece. 128: a stage holds two K-steps, 8 rows of 128 bytes per piece (whole 128-byte row
// segments per DMA, which stream at a higher rate from L2), two stages.
// WK = W_INT4: int4 weights (per-channel scales or the raw int32 sums), 64 bytes per weight
// row per 128-value stage, 16 rows per DMA piece; the fragments are unpacked to 16 q in the
// memory phase and the sums shifted right by 4 (exact) before the epilogue.
template <int BN_, int BM_, int STAGES_, int BKS_ = 64, int WK_ = W_INT8>
struct PpShape {
    static constexpr int BN = BN_, BM = BM_, BK = 64, BKS = BKS_, STAGES = STAGES_, WK = WK_;
    static constexpr int KPS = BKS / BK;                 // K-steps per stage
    static constexpr int NW = 8, NT = 512;
    static constexpr int WN = BN / 4, WM = BM / 2;
    static constexpr int FN = WN / 16, FM = WM / 16;
    static constexpr int WB = WK == W_INT4 ? BKS / 2 : BKS;  // weight bytes per row per stage
    static constexpr int W_TILE = BN * WB, STAGE = BN * WB + BM * BKS;
    static constexpr int RPP = 1024 / BKS;               // token rows per 1 KiB DMA piece
    static constexpr int RPPW = 1024 / WB;               // weight rows per piece
    static constexpr int W_PIECES = BN / RPPW;
    static constexpr int PIECES = W_PIECES + BM / RPP;   // DMA pieces per stage
    static constexpr int PPW = (PIECES + NW - 1) / NW;   // pieces per wave (max)
    static constexpr int FULL_WAVES = PIECES - (PPW - 1) * NW;
    static constexpr int LDS = 163840;
    static constexpr int CPR = BN / 8;                   // 16-byte output chunks per staged row
    // The tile's scales (s_x of its BM tokens, then s_w of its BN channels), copied to LDS with
    // the first stage: past the stage buffers, and in the rows of the staged output that are
    // written last (rows 3/4 BM and up belong to the second half) or past the staged tile.
    static constexpr int SCO = STAGES * STAGE > BM * BN * 3 / 2 ? STAGES * STAGE : BM * BN * 3 / 2;
    static constexpr int SC_PIECES = (BM + BN) / 64;     // 4-byte DMA pieces of 64 scales
    static constexpr int HALF_ITS = BM / 2 * CPR / NT;   // store iterations per staged half
    static_assert(BN % 64 == 0 && BM % 32 == 0, "tile shape");
    static_assert(SCO + (BM + BN) * 4 <= LDS && SCO % 16 == 0, "scale region");
    static_assert(BM / 2 * CPR % NT == 0 && (BM / 16) % 2 == 0, "staged halves");
    static_assert(BKS == 64 ? STAGES >= 3 && STAGES <= 4 : BKS == 128 && STAGES == 2, "stages");
    static_assert(WK == W_INT8 || BKS == 128, "int4 weights take 128-value stages");
    static_assert(STAGES * STAGE <= LDS, "LDS");
    static_assert(BM * BN * 2 <= LDS, "staged output tile");
    static_assert(2 * PPW < 64, "vmcnt range");
};

template <class S>
__device__ __forceinline__ void pp_issue(const int8_t *const (&src)[S::PPW], int koff, int8_t *stage, int wave) {
#pragma unroll
    for (int j = 0; j < S::PPW; ++j)
        if (j < S::PPW - 1 || wave < S::FULL_WAVES) dma_16B(src[j] + koff, stage + (wave + j * S::NW) * 1024);
}

// Wait until at most `after` stages of this wave's DMA are still in flight.
template <class S>
__device__ __forceinline__ void pp_wait(int after, bool full) {
    constexpr int G = S::PPW, g = S::PPW - 1;
    if (after <= 0) {
        wait_vmcnt<0>();
    } else if (after == 1) {
        if (full) wait_vmcnt<G>(); else wait_vmcnt<g>();
    } else {
        if (full) wait_vmcnt<2 * G>(); else wait_vmcnt<2 * g>();
    }
}

// The K loop of one wave; Q = the wave's index in its group. A wave issues its DMA pieces
// for stage j + STAGES - 1 in its memory phase of K-step j, right after its fragment reads:
// the buffer refilled (that of stage j - 1) is free by then, since each group read it in an
// earlier phase, before a barrier, and the compute phase then holds MFMAs only. (Measured
// against issuing the pieces at fixed slots between the MFMAs of the compute phase: 94.3
// against 96.0 us at M = 4096, N = 10240, K = 2560; 155 against 157 us at M = 8192,
// N = 2560, K = 10240; 184.5 against 186.5 us at M = 8192, N = 10240, K = 2560.)
template <class S, int Q>
__device__ __forceinline__ void pp_loop(v4i (&acc)[S::FN][S::FM], const int8_t *const (&src)[S::PPW], int8_t *smem,
                                        int KT, int grp, int wave, bool full, int frow, int fchunk) {
    constexpr int FN = S::FN, FM = S::FM, PPW = S::PPW, STAGES = S::STAGES;
    v4i a[FN], b[FM];
    int cur = 0, fb = STAGES - 1;  // buffers of stage j and of stage j + STAGES - 1
    for (int j = 0; j < KT; ++j) {
        // memory phase: this K-step's fragments (this wave's part of stage j + 1 landed), then
        // this wave's DMA for stage j + STAGES - 1
        const int8_t *st = smem + cur * S::STAGE;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            a[fn] = *reinterpret_cast<const v4i *>(st + swz<64>(Q * S::WN + fn * 16 + frow, fchunk));
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            b[fm] = *reinterpret_cast<const v4i *>(st + S::W_TILE + swz<64>(grp * S::WM + fm * 16 + frow, fchunk));
        if (j + STAGES - 1 < KT) {
            const int koff = (j + STAGES - 1) * S::BK;
            int8_t *fdst = smem + fb * S::STAGE + wave * 1024;
#pragma unroll
            for (int piece = 0; piece < PPW; ++piece)
                if (piece < PPW - 1 || full) dma_16B(src[piece] + koff, fdst + piece * S::NW * 1024);
        }
        wait_lgkmcnt0();
        // stages issued after j + 1 by now: j + 2 .. j + STAGES - 1
        if (j + 1 < KT) pp_wait<S>(min(STAGES - 2, KT - 2 - j), full);
        lds_barrier();
        // compute phase: MFMAs only
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_i8(a[fn], b[fm], acc[fn][fm]);
        lds_barrier();
        cur = cur + 1 == STAGES ? 0 : cur + 1;
        fb = fb + 1 == STAGES ? 0 : fb + 1;
    }
}

// The K loop with two stages of 128-value K-tiles (BKS = 128): stage s (K-steps 2 s and
// 2 s + 1) sits in buffer s & 1. In its memory phase of K-step 2 s a wave reads its
// fragments of the first half of stage s and issues its DMA pieces for stage s + 1 into the
// other buffer, whose stage s - 1 both groups finished reading in earlier phases; at the end
// of its memory phase of K-step 2 s + 1 it waits for those pieces, so every part of stage
// s + 1 has landed by the barrier before its first reader.
template <class S, int Q>
__device__ __forceinline__ void pp_loop2(v4i (&acc)[S::FN][S::FM], const int8_t *const (&src)[S::PPW],
                                         const int (&kadv)[S::PPW], int8_t *smem, int KT, int grp, int wave, bool full,
                                         int frow, int fchunk) {
    constexpr int FN = S::FN, FM = S::FM, PPW = S::PPW;
    v4i a[FN], b[FM];
    for (int j = 0; j < KT; ++j) {
        const int stg = j >> 1, h = j & 1;
        const int8_t *st = smem + (stg & 1) * S::STAGE;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int r = Q * S::WN + fn * 16 + frow;
            if constexpr (S::WK == W_INT4)  // the 16-byte piece with this lane's 16 values
                a[fn] = *reinterpret_cast<const v4i *>(st + r * 64 + (((2 * h + (fchunk >> 1)) ^ ((r >> 2) & 3)) << 4));
            else
                a[fn] = *reinterpret_cast<const v4i *>(st + swz<128>(r, 4 * h + fchunk));
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            b[fm] = *reinterpret_cast<const v4i *>(st + S::W_TILE + swz<128>(grp * S::WM + fm * 16 + frow, 4 * h + fchunk));
        if (h == 0 && 2 * (stg + 1) < KT) {
            int8_t *fdst = smem + ((stg + 1) & 1) * S::STAGE + wave * 1024;
#pragma unroll
            for (int piece = 0; piece < PPW; ++piece)
                if (piece < PPW - 1 || full) dma_16B(src[piece] + (stg + 1) * kadv[piece], fdst + piece * S::NW * 1024);
        }
        wait_lgkmcnt0();
        if constexpr (S::WK == W_INT4) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint2 w = (fchunk & 1) ? make_uint2(a[fn][2], a[fn][3]) : make_uint2(a[fn][0], a[fn][1]);
                a[fn] = __builtin_bit_cast(v4i, unpack_nibbles_x16(w.x, w.y));
            }
        }
        if (h == 1 && j + 1 < KT) wait_vmcnt<0>();  // stage s + 1: this wave's pieces landed
        lds_barrier();
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_i8(a[fn], b[fm], acc[fn][fm]);
        lds_barrier();
    }
}

typedef float float2_t __attribute__((ext_vector_type(2)));

// f(integral_constant<int, i>) for i = I .. E-1, unrolled at compile time
template <int I, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < E) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, E>(f);
    }
}

// Source of DMA piece `piece` of stage `stage` (int8 weights and tokens, 128-byte stage
// rows): a 32-bit offset from the weight or token base, whichever the piece covers (both
// uniform), so no 64-bit address per piece stays live through the MFMAs.
template <class S>
__device__ __forceinline__ const int8_t *pp_piece_src(const int8_t *wb, const int8_t *xb, const uint32_t (&off)[S::PPW],
                                                      int piece, int stage, int wave) {
    const bool is_w = min(wave + piece * S::NW, S::PIECES - 1) < S::W_PIECES;
    return (is_w ? wb : xb) + (off[piece] + (uint32_t)stage * S::BKS);
}

// DMA pieces [LO, HI) of this wave for stage `stage` (buffer stage & 1).
template <class S, int LO, int HI>
__device__ __forceinline__ void pp_issue_range(const int8_t *wb, const int8_t *xb, const uint32_t (&off)[S::PPW],
                                               int8_t *smem, int stage, int wave, bool full) {
    int8_t *dst = smem + (stage & 1) * S::STAGE + wave * 1024;
#pragma unroll
    for (int piece = LO; piece < HI; ++piece)
        if (piece < S::PPW - 1 || full) dma_16B(pp_piece_src<S>(wb, xb, off, piece, stage, wave), dst + piece * S::NW * 1024);
}

// The K loop with two stages of 128-value K-tiles and each stage's DMA split between two
// memory phases of each group (pp_loop2 issues a wave's nine pieces of stage s + 1 in one
// memory phase, K-step 2 s, which then runs well past the other group's MFMAs while the
// memory phases of K-steps 2 s + 1 issue none). Stage s + 1 goes to the buffer of stage
// s - 1:
//   group 0: pieces [0, A) in its memory phase of K-step 2 s, [A, PPW) in that of 2 s + 1,
//            and it waits for them after its MFMAs of K-step 2 s + 1;
//   group 1 (one phase behind): pieces [0, B) in its memory phase of K-step 2 s - 1, right
//            after its own fragment reads of stage s - 1 have retired (group 0 read that
//            stage last in the phase before, so the buffer is free), [B, PPW) in its
//            memory phase of 2 s; it waits for them in its memory phase of 2 s + 1.
// Both waits precede the barrier in front of group 0's first read of stage s + 1 (its
// memory phase of K-step 2 s + 2). Group 1's pieces [0, B) of stage 1 go out in the phase
// by which it starts behind group 0.
template <class S, int Q, int A, int B>
__device__ __forceinline__ void pp_loop3(v4i (&acc)[S::FN][S::FM], const int8_t *wb, const int8_t *xb,
                                         const uint32_t (&off)[S::PPW], int8_t *smem, int KT, int grp, int wave,
                                         bool full, int frow, int fchunk) {
    static_assert(S::WK == W_INT8 && S::BKS == 128, "int8 weights, 128-value stages");
    constexpr int FN = S::FN, FM = S::FM, PPW = S::PPW;
    static_assert(0 < A && A <= PPW && 0 < B && B < PPW, "piece split");
    const int NS = KT >> 1;
    v4i a[FN], b[FM];
    for (int j = 0; j < KT; ++j) {
        const int stg = j >> 1, h = j & 1;
        const int8_t *st = smem + (stg & 1) * S::STAGE;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            a[fn] = *reinterpret_cast<const v4i *>(st + swz<128>(Q * S::WN + fn * 16 + frow, 4 * h + fchunk));
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            b[fm] = *reinterpret_cast<const v4i *>(st + S::W_TILE + swz<128>(grp * S::WM + fm * 16 + frow, 4 * h + fchunk));
        const bool next = stg + 1 < NS;
        if (grp == 0) {
            if (next) {
                if (h == 0) pp_issue_range<S, 0, A>(wb, xb, off, smem, stg + 1, wave, full);
                else if constexpr (A < PPW) pp_issue_range<S, A, PPW>(wb, xb, off, smem, stg + 1, wave, full);
            }
            wait_lgkmcnt0();
        } else if (h == 0) {
            if (next) pp_issue_range<S, B, PPW>(wb, xb, off, smem, stg + 1, wave, full);
            wait_lgkmcnt0();
        } else {
            wait_lgkmcnt0();  // this wave's reads of stage s retired: the buffer is free
            if (stg + 2 < NS) {
                pp_issue_range<S, 0, B>(wb, xb, off, smem, stg + 2, wave, full);
                if (next) wait_vmcnt<B>();  // its pieces of stage s + 1 landed (the B just issued may fly)
            } else if (next) {
                wait_vmcnt<0>();
            }
        }
        lds_barrier();
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_i8(a[fn], b[fm], acc[fn][fm]);
        if (grp == 0 && h == 1 && next) wait_vmcnt<0>();  // group 0's pieces of stage s + 1 landed
        lds_barrier();
    }
}

// Two outputs rounded to fp16 (or bf16) in one conversion, RNE, packed low-first. The fp32
// inputs are pinned in registers so that the compiler cannot merge the preceding multiply
// into a mixed-precision fma (one rounding of the exact product).
template <bool BF>
__device__ __forceinline__ uint32_t pack_2x16(float a, float b) {
    asm volatile("" : "+v"(a), "+v"(b));
    const float2_t v = {a, b};
    if constexpr (BF) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    } else {
        typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    }
}

// Epilogue of the 16-bit outputs: the tile is staged through LDS as [BM][BN] rows (16-byte
// chunk index XOR-ed with (row & 7): the MFMA layout's 8-byte writes, 16 rows per
// instruction, and the row-contiguous 16-byte reads both stay free of bank conflicts) and
// written as 16-byte pieces of output rows, in NP parts: rows [WM/NP h, WM/NP (h + 1)) of
// each group's WM (fragment rows fm in [FM/NP h, FM/NP (h + 1))). Each part is converted and
// staged while the previous part's stores go out, between them, so the conversion work and
// the store traffic overlap; with four parts instead of two the first stores start after a
// quarter of the conversions (M=4096 N=10240 K=2560 82.5 against 83.9 us, M=2048 N=10240
// K=2560 43.9 against 45.0, M=2048 N=24576 K=4096 on 256 x 256 tiles 150.8 against 153.1;
// identical outputs).
template <class S, bool BF, int NP = 2>
__device__ __forceinline__ void pp_store_staged(const v4i (&acc)[S::FN][S::FM], const float (&sxm)[S::FM],
                                                const float4 (&s4)[S::FN], int8_t *smem, const GemmProblem &p, int m0,
                                                int n0, int grp, int wq, int frow, int fchunk, int tid) {
    constexpr int FN = S::FN, FM = S::FM, RS = S::BN * 2, CPR = S::CPR;
    constexpr int PF = FM / NP, PR = S::WM / NP;           // fragment rows and rows per group in a part
    constexpr int PITS = S::BM / NP * CPR / S::NT;          // store iterations per part
    static_assert(FM % NP == 0 && S::BM / NP * CPR % S::NT == 0, "epilogue parts");
    int coff[FN];  // byte offset in a staged row of this lane's 8-byte piece (row & 7 == frow & 7)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int nl = wq * S::WN + fn * 16 + 4 * fchunk;
        coff[fn] = (((nl >> 3) ^ (frow & 7)) << 4) + ((nl & 4) << 1);
    }
    int8_t *rbase = smem + (grp * S::WM + frow) * RS;
    auto stage = [&](auto fmc) __attribute__((always_inline)) {
        constexpr int fm = decltype(fmc)::value;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const v4i v = acc[fn][fm];
            const float y0 = ((float)v[0] * sxm[fm]) * s4[fn].x, y1 = ((float)v[1] * sxm[fm]) * s4[fn].y;
            const float y2 = ((float)v[2] * sxm[fm]) * s4[fn].z, y3 = ((float)v[3] * sxm[fm]) * s4[fn].w;
            *reinterpret_cast<uint2 *>(rbase + fm * 16 * RS + coff[fn]) = make_uint2(pack_2x16<BF>(y0, y1), pack_2x16<BF>(y2, y3));
        }
    };
    const int rows = min(S::BM, p.M - m0), cols = min(S::BN, p.N - n0);
    uint16_t *y = static_cast<uint16_t *>(p.y);
    // store iteration `it` of part h: chunk c = tid + NT it of the part's BM / NP rows
    auto store = [&](int h, int it) __attribute__((always_inline)) {
        const int c = tid + it * S::NT;
        const int rr = c / CPR, cc = c - rr * CPR;
        const int r = (rr % PR) + (rr / PR) * S::WM + h * PR;
        if (r < rows && cc * 8 < cols) {
            const v4u v = *reinterpret_cast<const v4u *>(smem + r * RS + ((cc ^ (r & 7)) << 4));
            // streaming store: the tile's outputs are not read again here, and as ordinary
            // stores they take L2 lines from the operand panels the next K-tiles read
            // (M=8192 N=2560 K=10240: 137.8 against 139.6 us; M=4096 N=2560 K=10240 111.7
            // against 113.3; identical outputs)
            __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(y + ((int64_t)(m0 + r) * p.ldy + n0 + cc * 8)));
        }
    };
    static_for<0, PF>([&](auto q) { stage(q); });
    lds_barrier();
    static_for<1, NP>([&](auto pc) {
        constexpr int pi = decltype(pc)::value;
        static_for<0, PF>([&](auto q) {
            constexpr int qi = decltype(q)::value;
            static_for<qi * PITS / PF, (qi + 1) * PITS / PF>([&](auto it) { store(pi - 1, decltype(it)::value); });
            stage(std::integral_constant<int, pi * PF + qi>{});
        });
        lds_barrier();
    });
    static_for<0, PITS>([&](auto it) { store(NP - 1, decltype(it)::value); });
}

// SPREAD = 16 A + B selects pp_loop3 with that split of each stage's DMA pieces (int8
// weights, 128-value stages); 0 selects pp_loop2 (or pp_loop for 64-value stages).
template <int BN, int BM, int STAGES, int BKS = 64, int WK = W_INT8, int SPREAD = 0, int EPI = 2>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmProblem p, TileMap tmap) {
    using S = PpShape<BN, BM, STAGES, BKS, WK>;
    constexpr int FM = S::FM, FN = S::FN, PPW = S::PPW;
    __shared__ __attribute__((aligned(1024))) int8_t smem[S::LDS];

    int tm, tn;
    map_tile(tmap, tm, tn);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wq = wave & 3;
    const bool full = wave < S::FULL_WAVES;
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    // Loader: wave w issues pieces g = w + j * NW of each stage (pieces below W_PIECES are
    // weight rows, the rest token rows); lane i covers row RPP g + i / LPR of the stage (LPR =
    // 64 / RPP lanes per row) and loads its 16-byte chunk (i % LPR) ^ ((row >> 1) & (LPR - 1)),
    // which is where the fragment reads look for it (64-byte int4 weight rows: chunk
    // (i % 4) ^ ((row >> 2) & 3)). kadv: bytes a piece's source advances per stage.
    constexpr int RPP = S::RPP, LPR = 64 / S::RPP, LPRW = 64 / S::RPPW;
    const int8_t *src[PPW];
    int kadv[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int g = min(wave + j * S::NW, S::PIECES - 1);
        const bool is_w = g < S::W_PIECES;
        if (is_w) {
            const int lrow = g * S::RPPW + lane / LPRW;
            const int c = WK == W_INT4 ? (lane % LPRW) ^ ((lrow >> 2) & 3) : (lane % LPRW) ^ ((lrow >> 1) & (LPRW - 1));
            const int64_t rb = WK == W_INT4 ? K / 2 : K;  // bytes per weight row
            src[j] = static_cast<const int8_t *>(p.wq) + ((int64_t)min(n0 + lrow, N - 1) * rb + 16 * c);
            kadv[j] = S::WB;
        } else {
            const int lrow = (g - S::W_PIECES) * RPP + lane / LPR;
            const int c = (lane % LPR) ^ ((lrow >> 1) & (LPR - 1));
            src[j] = p.xq + ((int64_t)min(m0 + lrow, M - 1) * K + 16 * c);
            kadv[j] = S::BKS;
        }
    }

    // the spread-DMA loop takes the same sources as 32-bit offsets from the two bases (the
    // launcher checks that both operands span less than 4 GiB)
    const int8_t *const wb = static_cast<const int8_t *>(p.wq), *const xb = p.xq;
    uint32_t off[PPW];
    if constexpr (SPREAD > 0) {
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
            const bool is_w = min(wave + j * S::NW, S::PIECES - 1) < S::W_PIECES;
            off[j] = (uint32_t)(src[j] - (is_w ? wb : xb));
        }
    }

    v4i acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int frow = lane & 15, fchunk = lane >> 4;
    const int KT = K / S::BK;
    // the tile's scales go out first, so every wait for the first stage retires them
    for (int i = wave; i < S::SC_PIECES; i += S::NW) {
        const float *ssrc = i < BM / 64 ? p.sx + min(m0 + 64 * i + lane, M - 1)
                                        : p.sw + min(n0 + 64 * (i - BM / 64) + lane, N - 1);
        dma_4B(ssrc, smem + S::SCO + 256 * i);
    }
    if constexpr (S::BKS == 64) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < KT) pp_issue<S>(src, s * S::BK, smem + s * S::STAGE, wave);
        pp_wait<S>(min(STAGES - 2, KT - 1), full);
    } else {
        pp_issue<S>(src, 0, smem, wave);  // stage 0; stage 1 goes out in the first K-step
        wait_vmcnt<0>();
    }
    lds_barrier();
    if (grp == 1) {
        // group 1 runs one phase behind group 0; with the spread DMA it issues its first
        // third of stage 1 in that phase
        if constexpr (SPREAD > 0)
            if (KT >= 4) pp_issue_range<S, 0, SPREAD % 16>(wb, xb, off, smem, 1, wave, full);
        lds_barrier();
    }

    if constexpr (S::BKS == 64) {
        switch (wq) {
            case 0: pp_loop<S, 0>(acc, src, smem, KT, grp, wave, full, frow, fchunk); break;
            case 1: pp_loop<S, 1>(acc, src, smem, KT, grp, wave, full, frow, fchunk); break;
            case 2: pp_loop<S, 2>(acc, src, smem, KT, grp, wave, full, frow, fchunk); break;
            default: pp_loop<S, 3>(acc, src, smem, KT, grp, wave, full, frow, fchunk); break;
        }
    } else if constexpr (SPREAD > 0) {
        switch (wq) {
            case 0: pp_loop3<S, 0, SPREAD / 16, SPREAD % 16>(acc, wb, xb, off, smem, KT, grp, wave, full, frow, fchunk); break;
            case 1: pp_loop3<S, 1, SPREAD / 16, SPREAD % 16>(acc, wb, xb, off, smem, KT, grp, wave, full, frow, fchunk); break;
            case 2: pp_loop3<S, 2, SPREAD / 16, SPREAD % 16>(acc, wb, xb, off, smem, KT, grp, wave, full, frow, fchunk); break;
            default: pp_loop3<S, 3, SPREAD / 16, SPREAD % 16>(acc, wb, xb, off, smem, KT, grp, wave, full, frow, fchunk); break;
        }
    } else {
        switch (wq) {
            case 0: pp_loop2<S, 0>(acc, src, kadv, smem, KT, grp, wave, full, frow, fchunk); break;
            case 1: pp_loop2<S, 1>(acc, src, kadv, smem, KT, grp, wave, full, frow, fchunk); break;
            case 2: pp_loop2<S, 2>(acc, src, kadv, smem, KT, grp, wave, full, frow, fchunk); break;
            default: pp_loop2<S, 3>(acc, src, kadv, smem, KT, grp, wave, full, frow, fchunk); break;
        }
    }
    if (grp == 0) lds_barrier();  // pairs with group 1's last compute barrier: LDS is free
    if constexpr (WK == W_INT4) {
        // int4: the sums of 16 q, shifted back exactly (K <= kInt4X16MaxK)
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = acc[i][j] >> 4;
    }

    // ---- epilogue (per-channel dequant or raw int32) ----
    // scales from the tile's LDS copy: entry j of s_w is s_w[min(n0 + j, N - 1)], so the
    // channels of a partial tile that are stored read their own scales
    const float *scl = reinterpret_cast<const float *>(smem + S::SCO);
    float sxm[FM];
    float4 s4[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sxm[fm] = scl[grp * S::WM + fm * 16 + frow];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) s4[fn] = *reinterpret_cast<const float4 *>(scl + BM + wq * S::WN + fn * 16 + 4 * fchunk);
    const int out = p.out;
    if ((out == OUT_F16 || out == OUT_BF16) && p.y_rows16) {
        if (out == OUT_F16)
            pp_store_staged<S, false, EPI>(acc, sxm, s4, smem, p, m0, n0, grp, wq, frow, fchunk, tid);
        else
            pp_store_staged<S, true, EPI>(acc, sxm, s4, smem, p, m0, n0, grp, wq, frow, fchunk, tid);
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + grp * S::WM + fm * 16 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + wq * S::WN + fn * 16 + 4 * fchunk;
            if (n >= N) continue;
            const int64_t off = (int64_t)m * p.ldy + n;
            const v4i v = acc[fn][fm];
            if (out == OUT_I32) {
                *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = make_int4(v[0], v[1], v[2], v[3]);
            } else {
                store4(p.y, off, out, ((float)v[0] * sxm[fm]) * s4[fn].x, ((float)v[1] * sxm[fm]) * s4[fn].y,
                       ((float)v[2] * sxm[fm]) * s4[fn].z, ((float)v[3] * sxm[fm]) * s4[fn].w);
            }
        }
    }
}

// ---- per-group and W4A8 on the direct-to-LDS pipeline ---------------------------------
//
// The structure of gemm_ms_kernel (BN x BM tile, 128-value K-tiles, STAGES LDS stages filled
// by global_load_lds, one barrier per K-tile) with the per-group dequantization of the
// pages' segmented form: per group g, acc_g (int32, started by an MFMA on a zero
// accumulator) is folded into an fp32 accumulator, t = fma(fp32(acc_g), s_w[n, g], t), g
// ascending; at the end y = t * s_x[m]. Each stage also carries the K-tile's group scales of
// the tile's BN output channels ([group][n] floats, 4-byte DMA gathers from s_w [N, G]); a
// wave reads them into registers before the stage's barrier, together with the next
// K-step's fragments, so the buffer can be refilled as soon as every wave passed it.
//
// int4 weights (WK = W_INT4) are 64 bytes per row per K-tile; a DMA instruction moves 16
// rows x 64 bytes and the 16-byte pieces of row r sit at position piece ^ ((r >> 2) & 3),
// which keeps the 8-byte fragment reads conflict-free; fragments are unpacked after the
// LDS read to the int8 values 16 q (see unpack_nibbles_x16), so each group's int32 sum is
// 16 acc_g and the fold keeps 16 t: fma(fp32(16 a), s, 16 t) = 16 fma(fp32(a), s, t)
// exactly while no value is subnormal (a power-of-two scaling commutes with rounding in
// the normal range; every product of a nonzero sum and a scale >= 2^-100 is normal).
// The epilogue multiplies by 2^-4 (exact) before s_x.
//
// GS = 0: per-channel weight scales (int4 weights of one scale per output channel, Cider
// README "量化": per-column INT4; or the raw int32 sums of int4 weights): no fold, the int32
// sums run over all of K (16 x the sums for int4, exactly while K <= kInt4X16MaxK, which the
// launcher checks), shifted right by 4 (exact) and dequantized as the per-channel kernels do,
// y = (fp32(acc) * s_x[m]) * s_w[n].
template <int BN_, int BM_, int STAGES_, int WGN_, int WGM_, int GS_, int WK_>
struct MgShape {
    static constexpr int BN = BN_, BM = BM_, BK = 128, STAGES = STAGES_, WGN = WGN_, WGM = WGM_, GS = GS_, WK = WK_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int WB = WK == W_INT4 ? 64 : 128;        // weight bytes per row per K-tile
    static constexpr int W_TILE = BN * WB, X_TILE = BM * BK;
    static constexpr bool PC = GS == 0;                         // per-channel scales: no fold
    static constexpr int GPK = PC ? 0 : BK / GS;                // groups per K-tile (1 or 2)
    static constexpr int SCALES = GPK * BN * 4;
    static constexpr int STAGE = W_TILE + X_TILE + SCALES;
    static constexpr int WG = W_TILE / 1024, XG = X_TILE / 1024;  // 1 KiB DMA pieces per stage
    static constexpr int NG = WG + XG;
    static constexpr int NSD = GPK * BN / 64;                   // 4-byte scale DMAs per stage (none for PC)
    static constexpr int GPW = (NG + NW - 1) / NW;              // tile DMAs per wave (max)
    static_assert(GS == 0 || GS == 64 || GS == 128, "group size");
    static_assert(BN % 64 == 0 && BM % 8 == 0 && WN % 16 == 0 && WM % 16 == 0, "tile shape");
    static_assert(W_TILE % 1024 == 0 && NSD <= NW, "loader shape");
    static_assert(STAGES * STAGE <= 163840, "LDS");
};

// s_waitcnt vmcnt(n) for a uniform n known only at run time (n clamped to 40; a smaller
// count only waits longer).
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
    switch (n) {
#define W8A8_VM_CASE(k) case k: wait_vmcnt<k>(); break;
        W8A8_VM_CASE(0) W8A8_VM_CASE(1) W8A8_VM_CASE(2) W8A8_VM_CASE(3) W8A8_VM_CASE(4) W8A8_VM_CASE(5)
        W8A8_VM_CASE(6) W8A8_VM_CASE(7) W8A8_VM_CASE(8) W8A8_VM_CASE(9) W8A8_VM_CASE(10) W8A8_VM_CASE(11)
        W8A8_VM_CASE(12) W8A8_VM_CASE(13) W8A8_VM_CASE(14) W8A8_VM_CASE(15) W8A8_VM_CASE(16) W8A8_VM_CASE(17)
        W8A8_VM_CASE(18) W8A8_VM_CASE(19) W8A8_VM_CASE(20) W8A8_VM_CASE(21) W8A8_VM_CASE(22) W8A8_VM_CASE(23)
        W8A8_VM_CASE(24) W8A8_VM_CASE(25) W8A8_VM_CASE(26) W8A8_VM_CASE(27) W8A8_VM_CASE(28) W8A8_VM_CASE(29)
        W8A8_VM_CASE(30) W8A8_VM_CASE(31) W8A8_VM_CASE(32) W8A8_VM_CASE(33) W8A8_VM_CASE(34) W8A8_VM_CASE(35)
        W8A8_VM_CASE(36) W8A8_VM_CASE(37) W8A8_VM_CASE(38) W8A8_VM_CASE(39)
#undef W8A8_VM_CASE
        default: wait_vmcnt<40>(); break;
    }
}

// DMA of K-tile kt of the tile (m0, n0) into one stage. Wave w issues pieces g = w + j NW
// (weight pieces first, then token pieces) and, if w < NSD, scale gather w.
template <class S>
__device__ __forceinline__ void mg_issue(const GemmProblem &p, int m0, int n0, int kt, int8_t *st, int wave,
                                         int lane) {
    const int G = S::PC ? 1 : p.K / (S::PC ? 1 : S::GS);
#pragma unroll
    for (int j = 0; j < S::GPW; ++j) {
        const int g = wave + j * S::NW;
        if (g < S::NG) {
            if (g < S::WG) {
                // weight piece: WB = 128 -> 8 rows x 128 B; WB = 64 -> 16 rows x 64 B
                constexpr int LPR = S::WB / 16;  // lanes per row
                const int lrow = g * (64 / LPR) + lane / LPR, pos = lane % LPR;
                const int c = S::WB == 128 ? pos ^ ((lrow >> 1) & 7) : pos ^ ((lrow >> 2) & 3);
                const int grow = min(n0 + lrow, p.N - 1);
                const int8_t *w = static_cast<const int8_t *>(p.wq) + (int64_t)grow * (S::WK == W_INT4 ? p.K / 2 : p.K);
                dma_16B(w + kt * S::WB + 16 * c, st + g * 1024);
            } else {
                const int xg = g - S::WG;
                const int lrow = xg * 8 + (lane >> 3);
                const int c = (lane & 7) ^ ((lrow >> 1) & 7);
                const int grow = min(m0 + lrow, p.M - 1);
                dma_16B(p.xq + (int64_t)grow * p.K + kt * S::BK + 16 * c, st + S::W_TILE + xg * 1024);
            }
        }
    }
    if (!S::PC && wave < S::NSD) {
        // scales [gi][n] of this K-tile: gather gi = wave / (BN / 64), n block wave % (BN / 64)
        const int gi = wave / (S::BN / 64), nb = wave % (S::BN / 64);
        const int n = min(n0 + nb * 64 + lane, p.N - 1);
        dma_4B(p.sw + (int64_t)n * G + kt * S::GPK + gi, st + S::W_TILE + S::X_TILE + (gi * S::BN + nb * 64) * 4);
    }
}

template <class S>
__device__ __forceinline__ int mg_ops_per_stage(int wave) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < S::GPW; ++j) n += (wave + j * S::NW < S::NG) ? 1 : 0;
    return n + (!S::PC && wave < S::NSD ? 1 : 0);
}

// Weight fragments as read from LDS: int8 codes (v4i), or for int4 the lane's 16 packed
// nibbles (uint2), unpacked by mg_unpack once the read has landed.
template <class S>
using MgRawA = typename std::conditional<S::WK == W_INT4, uint2, v4i>::type;

template <class S>
__device__ __forceinline__ void mg_frags(const int8_t *st, int ks, int wm, int wn, int frow, int fchunk,
                                         MgRawA<S> (&a)[S::FN], v4i (&b)[S::FM]) {
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn) {
        const int r = wn * S::WN + fn * 16 + frow;
        if constexpr (S::WK == W_INT4) {
            const int byte = ks * 32 + fchunk * 8;  // 16 int4 values of this lane
            const v4i q = *reinterpret_cast<const v4i *>(st + r * 64 + (((byte >> 4) ^ ((r >> 2) & 3)) << 4));
            a[fn] = (byte & 8) ? make_uint2(q[2], q[3]) : make_uint2(q[0], q[1]);
        } else {
            a[fn] = *reinterpret_cast<const v4i *>(st + swz<128>(r, ks * 4 + fchunk));
        }
    }
#pragma unroll
    for (int fm = 0; fm < S::FM; ++fm)
        b[fm] = *reinterpret_cast<const v4i *>(st + S::W_TILE + swz<128>(wm * S::WM + fm * 16 + frow, ks * 4 + fchunk));
}

template <class S>
__device__ __forceinline__ void mg_unpack(const MgRawA<S> (&raw)[S::FN], v4i (&a)[S::FN]) {
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn) {
        if constexpr (S::WK == W_INT4)
            a[fn] = __builtin_bit_cast(v4i, unpack_nibbles_x16(raw[fn].x, raw[fn].y));
        else
            a[fn] = raw[fn];
    }
}

// MFMAs of one K-step; FIRST: the step opens a group (accumulate from zero).
template <class S, bool FIRST>
__device__ __forceinline__ void mg_mma(v4i (&acc)[S::FN][S::FM], const v4i (&a)[S::FN], const v4i (&b)[S::FM]) {
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < S::FM; ++fm)
            acc[fn][fm] = mfma_i8(a[fn], b[fm], FIRST ? v4i{0, 0, 0, 0} : acc[fn][fm]);
}

// t = fma(fp32(acc_g), s_w[n, g], t) for the group that just closed.
template <class S>
__device__ __forceinline__ void mg_fold(const v4i (&acc)[S::FN][S::FM], const float4 (&sw)[S::FN],
                                        float4 (&t)[S::FN][S::FM]) {
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < S::FM; ++fm) {
            t[fn][fm].x = __builtin_fmaf((float)acc[fn][fm][0], sw[fn].x, t[fn][fm].x);
            t[fn][fm].y = __builtin_fmaf((float)acc[fn][fm][1], sw[fn].y, t[fn][fm].y);
            t[fn][fm].z = __builtin_fmaf((float)acc[fn][fm][2], sw[fn].z, t[fn][fm].z);
            t[fn][fm].w = __builtin_fmaf((float)acc[fn][fm][3], sw[fn].w, t[fn][fm].w);
        }
}

// The fold of the group held in acc, interleaved with the MFMAs that open the next group:
// per fragment, fold it (its MFMA was issued a full K-step earlier), then issue the MFMA
// that overwrites it. A wave's VALU work then issues while its own MFMAs run.
template <class S>
__device__ __forceinline__ void mg_fold_mma(v4i (&acc)[S::FN][S::FM], const float4 (&sw)[S::FN],
                                            float4 (&t)[S::FN][S::FM], const v4i (&a)[S::FN],
                                            const v4i (&b)[S::FM]) {
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < S::FM; ++fm) {
            t[fn][fm].x = __builtin_fmaf((float)acc[fn][fm][0], sw[fn].x, t[fn][fm].x);
            t[fn][fm].y = __builtin_fmaf((float)acc[fn][fm][1], sw[fn].y, t[fn][fm].y);
            t[fn][fm].z = __builtin_fmaf((float)acc[fn][fm][2], sw[fn].z, t[fn][fm].z);
            t[fn][fm].w = __builtin_fmaf((float)acc[fn][fm][3], sw[fn].w, t[fn][fm].w);
            // the fold stays here (not sunk behind the MFMAs, which would keep both
            // accumulator sets live)
            asm volatile("" : "+v"(t[fn][fm].x), "+v"(t[fn][fm].y), "+v"(t[fn][fm].z), "+v"(t[fn][fm].w));
            acc[fn][fm] = mfma_i8(a[fn], b[fm], v4i{0, 0, 0, 0});
            __builtin_amdgcn_sched_barrier(0);
        }
}

// The group scales of a stage, FN float4 64 bytes apart, read in one asm block that also
// retires them. The stage landed before the barrier that opened it; read as ordinary loads,
// the compiler cannot tell them from the LDS targets of the DMA still in flight and waits
// for all of that DMA first (vmcnt(0) every K-tile, which empties the stage ring).
template <class S>
__device__ __forceinline__ void mg_scales(const int8_t *st, int gi, int wn, int fchunk, float4 (&sw)[S::FN]) {
    typedef float v4f_t __attribute__((ext_vector_type(4)));
    const float *sc = reinterpret_cast<const float *>(st + S::W_TILE + S::X_TILE) + gi * S::BN + wn * S::WN + 4 * fchunk;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float *)sc;
    static_assert(S::FN == 2 || S::FN == 4, "scale reads per wave");
    v4f_t v[4];
    if constexpr (S::FN == 4) {
        asm volatile(
            "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:64\n\t"
            "ds_read_b128 %2, %4 offset:128\n\tds_read_b128 %3, %4 offset:192\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
            : "v"(a)
            : "memory");
    } else {
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:64\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1])
                     : "v"(a)
                     : "memory");
    }
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn) sw[fn] = make_float4(v[fn][0], v[fn][1], v[fn][2], v[fn][3]);
}

// Per-channel epilogue of the GS = 0 form: the int32 sums (16 x the sums for int4 weights,
// shifted back exactly) dequantized as y = (fp32(acc) * s_x[m]) * s_w[n], or stored raw for
// I32 output; SPLIT stores the slice's int32 sums to p.ws for splitk_finish_kernel.
template <class S, bool SPLIT>
__device__ __forceinline__ void mg_pc_epilogue(const GemmProblem &p, v4i (&acc)[S::FN][S::FM], int8_t *smem, int m0,
                                               int n0, int wm, int wn, int frow, int fchunk, int tid, int ks) {
    constexpr int FM = S::FM, FN = S::FN;
    const int M = p.M, N = p.N;
    if constexpr (S::WK == W_INT4) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = acc[fn][fm] >> 4;
    }
    if constexpr (SPLIT) {
        int32_t *ws = static_cast<int32_t *>(p.ws) + (int64_t)ks * M * N;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + wm * S::WM + fm * 16 + frow;
            if (m >= M) continue;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = n0 + wn * S::WN + fn * 16 + 4 * fchunk;
                if (n >= N) continue;
                const v4i v = acc[fn][fm];
                *reinterpret_cast<int4 *>(ws + (int64_t)m * N + n) = make_int4(v[0], v[1], v[2], v[3]);
            }
        }
        return;
    }
    const float *__restrict__ sxp = p.sx;
    const float *__restrict__ swp = p.sw;
    float sxm[FM];
    float4 s4[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sxm[fm] = sxp[min(m0 + wm * S::WM + fm * 16 + frow, M - 1)];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        s4[fn] = *reinterpret_cast<const float4 *>(swp + min(n0 + wn * S::WN + fn * 16 + 4 * fchunk, N - 4));
    const int out = p.out;
    if ((out == OUT_F16 || out == OUT_BF16) && p.y_rows16) {
        constexpr int RS = S::BM * (S::BN * 2 + 16) <= S::STAGES * S::STAGE ? S::BN * 2 + 16 : S::BN * 2;
        static_assert(S::BM * S::BN * 2 <= S::STAGES * S::STAGE, "staged output tile must fit the LDS buffers");
        lds_barrier();
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int lr = wm * S::WM + fm * 16 + frow;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const v4i v = acc[fn][fm];
                const float y0 = ((float)v[0] * sxm[fm]) * s4[fn].x, y1 = ((float)v[1] * sxm[fm]) * s4[fn].y;
                const float y2 = ((float)v[2] * sxm[fm]) * s4[fn].z, y3 = ((float)v[3] * sxm[fm]) * s4[fn].w;
                const uint2 w = out == OUT_F16 ? make_uint2(f16_bits(y0) | (f16_bits(y1) << 16), f16_bits(y2) | (f16_bits(y3) << 16))
                                               : make_uint2(bf16_rne(y0) | (bf16_rne(y1) << 16), bf16_rne(y2) | (bf16_rne(y3) << 16));
                *reinterpret_cast<uint2 *>(smem + lr * RS + 2 * (wn * S::WN + fn * 16 + 4 * fchunk)) = w;
            }
        }
        lds_barrier();
        constexpr int CPR = S::BN / 8;
        const int rows = min(S::BM, M - m0), cols = min(S::BN, N - n0);
#pragma unroll 4
        for (int c = tid; c < S::BM * CPR; c += S::NT) {
            const int r = c / CPR, cc = c - r * CPR;
            if (r < rows && cc * 8 < cols) {
                const v4u v = *reinterpret_cast<const v4u *>(smem + r * RS + 16 * cc);
                // streaming store (see pp_store_staged)
                __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(static_cast<uint16_t *>(p.y) + ((int64_t)(m0 + r) * p.ldy + n0 + cc * 8)));
            }
        }
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * S::WM + fm * 16 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + wn * S::WN + fn * 16 + 4 * fchunk;
            if (n >= N) continue;
            const int64_t off = (int64_t)m * p.ldy + n;
            const v4i v = acc[fn][fm];
            if (out == OUT_I32) {
                *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = make_int4(v[0], v[1], v[2], v[3]);
            } else {
                store4(p.y, off, out, ((float)v[0] * sxm[fm]) * s4[fn].x, ((float)v[1] * sxm[fm]) * s4[fn].y,
                       ((float)v[2] * sxm[fm]) * s4[fn].z, ((float)v[3] * sxm[fm]) * s4[fn].w);
            }
        }
    }
}

// SPLIT: one K-slice per workgroup; the slice's fold t (times 2^-4 for int4) goes to p.ws as
// fp32, and the slices are added and scaled by s_x afterwards.
template <int BN, int BM, int STAGES, int WGN, int WGM, int GS, int WK, bool SPLIT>
__global__ __launch_bounds__(512) void gemm_mg_kernel(GemmProblem p, TileMap tmap) {  // see gemm_ms_kernel
    using S = MgShape<BN, BM, STAGES, WGN, WGM, GS, WK>;
    constexpr int FM = S::FM, FN = S::FN;
    __shared__ __attribute__((aligned(1024))) int8_t smem[STAGES * S::STAGE];

    int tm, tn, ks = 0;
    if constexpr (SPLIT)
        map_unit(tmap, p.ksplit, tm, tn, ks);
    else
        map_tile(tmap, tm, tn);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WGN, wm = wave / WGN;
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N;
    const int frow = lane & 15, fchunk = lane >> 4;
    int kt0 = 0, KT = p.K / S::BK;
    if constexpr (SPLIT) slice_range(p.K / S::BK, p.ksplit, ks, kt0, KT);
    const int OPS = mg_ops_per_stage<S>(wave);

    v4i acc[FN][FM];
    float4 t[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            acc[i][j] = v4i{0, 0, 0, 0};
            t[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }

    // prologue: stages 0 .. STAGES-2 in flight, wait for stage 0
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < KT) mg_issue<S>(p, m0, n0, kt0 + s, smem + s * S::STAGE, wave, lane);
    wait_vmcnt_rt(OPS * min(STAGES - 2, KT - 1));
    lds_barrier();

    v4i a0[FN], b0[FM], a1[FN], b1[FM];
    MgRawA<S> r0[FN], r1[FN];  // weight fragments as read (int4: packed until unpacked)
    // scales of the group acc holds (zero before the first group, whose fold adds +0 to t = +0)
    float4 sw0[FN], sw1[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) sw0[i] = sw1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    int cur = 0;
    // One group per K-tile with eight waves: the waves of the second half (one on each SIMD)
    // run each K-tile as [fold the closed group and open the next with K-step 0][K-step 1],
    // the first half as [K-step 1 of the previous K-tile][fold and open]. Between two
    // barriers each SIMD then has one wave folding while the other runs MFMAs only, where
    // with all waves in step both fold at once (VALU-bound) and then both wait on MFMAs.
    // Both halves read all of a stage before the barrier that ends it.
    constexpr bool LAG = !S::PC && S::GPK == 1 && S::NW == 8;
    if (LAG && wave >= S::NW / 2) {
        for (int kt = 0; kt < KT; ++kt) {
            const int fill = kt + STAGES - 1;
            if (fill < KT) {
                int fb = cur + STAGES - 1;
                fb -= fb >= STAGES ? STAGES : 0;
                mg_issue<S>(p, m0, n0, kt0 + fill, smem + fb * S::STAGE, wave, lane);
            }
            const int8_t *st = smem + cur * S::STAGE;
            mg_frags<S>(st, 0, wm, wn, frow, fchunk, r0, b0);
            mg_unpack<S>(r0, a0);
            mg_fold_mma<S>(acc, sw0, t, a0, b0);  // group kt-1 folds, group kt opens
            mg_frags<S>(st, 1, wm, wn, frow, fchunk, r1, b1);
            mg_scales<S>(st, 0, wn, fchunk, sw0);
            mg_unpack<S>(r1, a1);
            mg_mma<S, false>(acc, a1, b1);  // K-step 1 closes group kt
            if (kt + 1 < KT) {
                wait_vmcnt_rt(OPS * min(STAGES - 2, KT - 2 - kt));
                lds_barrier();
                cur = cur + 1 == STAGES ? 0 : cur + 1;
            }
        }
    } else {
    mg_frags<S>(smem, 0, wm, wn, frow, fchunk, r0, b0);
    wait_lgkmcnt0();
    mg_unpack<S>(r0, a0);
    for (int kt = 0; kt < KT; ++kt) {
        const int fill = kt + STAGES - 1;
        if (fill < KT) {
            int fb = cur + STAGES - 1;
            fb -= fb >= STAGES ? STAGES : 0;
            mg_issue<S>(p, m0, n0, kt0 + fill, smem + fb * S::STAGE, wave, lane);
        }
        const int8_t *st = smem + cur * S::STAGE;
        // everything this wave still needs from stage kt is read before its barrier
        mg_frags<S>(st, 1, wm, wn, frow, fchunk, r1, b1);
        if constexpr (S::PC) {
            mg_mma<S, false>(acc, a0, b0);
        } else {
            // K-step 0 opens group kt (gs 128) or 2 kt (gs 64) while the previous group is folded
            mg_fold_mma<S>(acc, S::GPK == 2 ? sw1 : sw0, t, a0, b0);
            mg_scales<S>(st, 0, wn, fchunk, sw0);
            if constexpr (S::GPK == 2) mg_scales<S>(st, 1, wn, fchunk, sw1);
        }
        wait_lgkmcnt0();
        mg_unpack<S>(r1, a1);
        if (kt + 1 < KT) {
            wait_vmcnt_rt(OPS * min(STAGES - 2, KT - 2 - kt));
            lds_barrier();
            int nb = cur + 1;
            nb -= nb >= STAGES ? STAGES : 0;
            // read now, unpacked after the MFMAs below are issued
            mg_frags<S>(smem + nb * S::STAGE, 0, wm, wn, frow, fchunk, r0, b0);
            cur = nb;
        }
        if constexpr (S::GPK == 2) {
            mg_fold_mma<S>(acc, sw0, t, a1, b1);  // K-step 1 is group 2 kt + 1; group 2 kt folds
        } else {
            mg_mma<S, false>(acc, a1, b1);  // K-step 1 closes group kt
        }
        wait_lgkmcnt0();
        mg_unpack<S>(r0, a0);
    }
    }
    if constexpr (S::PC) {
        mg_pc_epilogue<S, SPLIT>(p, acc, smem, m0, n0, wm, wn, frow, fchunk, tid, ks);
        return;
    }
    mg_fold<S>(acc, S::GPK == 2 ? sw1 : sw0, t);  // the last group

    // ---- epilogue: y = t * s_x[m] ----
    // int4: t holds 16 x the sum (the unpacked codes are 16 q); the scaling by 2^-4 is exact
    constexpr float TS = S::WK == W_INT4 ? 0.0625f : 1.0f;
    if constexpr (SPLIT) {
        float *ws = static_cast<float *>(p.ws) + (int64_t)ks * M * N;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + wm * S::WM + fm * 16 + frow;
            if (m >= M) continue;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = n0 + wn * S::WN + fn * 16 + 4 * fchunk;
                if (n >= N) continue;
                const float4 v = t[fn][fm];
                *reinterpret_cast<float4 *>(ws + (int64_t)m * N + n) = make_float4(v.x * TS, v.y * TS, v.z * TS, v.w * TS);
            }
        }
        return;
    }
    const float *__restrict__ sxp = p.sx;
    float sxm[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sxm[fm] = sxp[min(m0 + wm * S::WM + fm * 16 + frow, M - 1)];
    const int out = p.out;
    if ((out == OUT_F16 || out == OUT_BF16) && p.y_rows16) {
        constexpr int RS = S::BM * (S::BN * 2 + 16) <= S::STAGES * S::STAGE ? S::BN * 2 + 16 : S::BN * 2;
        static_assert(S::BM * S::BN * 2 <= S::STAGES * S::STAGE, "staged output tile must fit the LDS buffers");
        // staged and stored in two halves, rows [WM/2 h, WM/2 (h + 1)) of each wave row's WM:
        // the second half is converted while the first half's stores go out
        constexpr int CPR = S::BN / 8, HF = FM / 2, HR = S::WM / 2, ITS = S::BM / 2 * CPR / S::NT;
        static_assert(FM % 2 == 0 && S::BM / 2 * CPR % S::NT == 0, "staged halves");
        const int rows = min(S::BM, M - m0), cols = min(S::BN, N - n0);
        auto stage = [&](int fm) __attribute__((always_inline)) {
            const int lr = wm * S::WM + fm * 16 + frow;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const float4 v = t[fn][fm];
                const float y0 = (v.x * TS) * sxm[fm], y1 = (v.y * TS) * sxm[fm];
                const float y2 = (v.z * TS) * sxm[fm], y3 = (v.w * TS) * sxm[fm];
                const uint2 w = out == OUT_F16 ? make_uint2(f16_bits(y0) | (f16_bits(y1) << 16), f16_bits(y2) | (f16_bits(y3) << 16))
                                               : make_uint2(bf16_rne(y0) | (bf16_rne(y1) << 16), bf16_rne(y2) | (bf16_rne(y3) << 16));
                *reinterpret_cast<uint2 *>(smem + lr * RS + 2 * (wn * S::WN + fn * 16 + 4 * fchunk)) = w;
            }
        };
        auto store = [&](int h, int it) __attribute__((always_inline)) {
            const int c = tid + it * S::NT;
            const int rr = c / CPR, cc = c - rr * CPR;
            const int r = (rr % HR) + (rr / HR) * S::WM + h * HR;
            if (r < rows && cc * 8 < cols) {
                const v4u v = *reinterpret_cast<const v4u *>(smem + r * RS + 16 * cc);
                // streaming store (see pp_store_staged)
                __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(static_cast<uint16_t *>(p.y) + ((int64_t)(m0 + r) * p.ldy + n0 + cc * 8)));
            }
        };
        lds_barrier();
#pragma unroll
        for (int fm = 0; fm < HF; ++fm) stage(fm);
        lds_barrier();
#pragma unroll
        for (int q = 0; q < HF; ++q) {
#pragma unroll
            for (int it = q * ITS / HF; it < (q + 1) * ITS / HF; ++it) store(0, it);
            stage(HF + q);
        }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < ITS; ++it) store(1, it);
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * S::WM + fm * 16 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + wn * S::WN + fn * 16 + 4 * fchunk;
            if (n >= N) continue;
            const float4 v = t[fn][fm];
            store4(p.y, (int64_t)m * p.ldy + n, out, (v.x * TS) * sxm[fm], (v.y * TS) * sxm[fm],
                   (v.z * TS) * sxm[fm], (v.w * TS) * sxm[fm]);
        }
    }
}

// ---- weights through LDS, activations direct to registers ----------------------------
//
// Measured on gfx950: LDS serves about 128 B/clk per CU for ds_read_b128 and DMA writes
// combined. A tile that stages both operands in LDS spends most of that on operand
// re-reads, so here only the weight tile goes through LDS; activation fragments are
// loaded straight from L2 into VGPRs, where the MFMA B operand wants them.
//
// Tile: 256 weight rows (n) x 256 tokens (m), 128-byte K-tiles, 4 * WGN waves; wave
// (wn, wm) covers n in [wn * 256 / WGN, ...) and tokens [64 wm, 64 wm + 64). With WGN = 2
// (8 waves, two per SIMD) a wave holds 8 x 4 MFMA 16x16x64 accumulators (128 VGPRs).
// Weight K-tiles stream through a 4-deep LDS ring (32 KiB each) by global_load_lds.
// A K-tile is 2 * FN weight fragments per wave (FN n-blocks x 2 K-steps); every
// fragment feeds 4 MFMAs and is read from LDS WIN fragments ahead of its use. Per K-tile t:
//
//   top:  load x fragments of K-tile t+1 (VGPR double buffer)
//   fragments of K-step 0 and 1, each: 4 MFMAs, read fragment f + WIN
//   mid (after the last read of stage t was issued):
//         wait own weight DMA of stage t+1; barrier; DMA weight stage t+3 into the
//         buffer of stage t-1 (free: every wave passed this barrier after finishing it)
//   the reads that run past the K-tile fetch stage t+1
//   end:  wait x of K-tile t+1
//
// VMEM issue order is x(t+1) at the top, weights(t+3) at mid; global loads return in
// order, so the vmcnt limits below count exactly the loads issued after the one needed.
// LDS traffic per K-tile: 32 KiB DMA + 128 KiB fragment reads over 2048 MFMA cycles/SIMD.
template <int WGN_>
struct XdShape {
    static constexpr int WGN = WGN_;
    static constexpr int BN = 256, BM = 256, BK = 128, STAGES = 4, NW = 4 * WGN;
    static constexpr int WM = 64, FM = 4, WN = BN / WGN, FN = WN / 16, NFRAG = 2 * FN, WIN = 4;
    static constexpr int STAGE = BN * BK;      // 32 KiB of weights
    static constexpr int GPW = (BN / 8) / NW;  // weight DMA instructions per wave per stage
    static constexpr int XL = FM * 2;          // x load instructions per wave per K-tile (8)
    static constexpr int MID = NFRAG - 1 - WIN;  // last fragment index whose prefetch is in stage t
};

template <class S>
__device__ __forceinline__ const v4i *xd_frag_ptr(const int8_t *st, int f, int wn, int frow, int fchunk) {
    // fragment f: n-block f % FN of this wave, K-step f / FN
    return reinterpret_cast<const v4i *>(
        st + swz<128>(wn * S::WN + (f % S::FN) * 16 + frow, (f / S::FN) * 4 + fchunk));
}

template <class S>
__device__ __forceinline__ void xd_load_x(const int8_t *const (&xrow)[S::FM], int k0, int fchunk,
                                          v4i (&x)[S::FM][2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int fm = 0; fm < S::FM; ++fm)
            x[fm][ks] = *reinterpret_cast<const v4i *>(xrow[fm] + k0 + ks * 64 + fchunk * 16);
}

template <class S>
__device__ __forceinline__ void xd_issue_w(const int8_t *const (&wsrc)[S::GPW], int k0, int8_t *dst, int wave) {
#pragma unroll
    for (int j = 0; j < S::GPW; ++j) dma_16B(wsrc[j] + k0, dst + (wave + j * S::NW) * 1024);
}

// One K-tile of the main loop (X = x fragments of this K-tile, XN = buffer for the next).
// STEADY: t + 3 < KT is known, so the body has no data-dependent branches.
template <class S, bool STEADY>
__device__ __forceinline__ void xd_ktile(int t, int KT, int8_t *smem, const int8_t *const (&wsrc)[S::GPW],
                                         const int8_t *const (&xrow)[S::FM], int wave, int wn, int frow,
                                         int fchunk, v4i (&win)[S::WIN], v4i (&acc)[S::FN][S::FM],
                                         const v4i (&X)[S::FM][2], v4i (&XN)[S::FM][2]) {
    if (STEADY || t + 1 < KT) xd_load_x<S>(xrow, (t + 1) * S::BK, fchunk, XN);
    const int8_t *st = smem + (t & 3) * S::STAGE;
    const int8_t *st_next = smem + ((t + 1) & 3) * S::STAGE;
#pragma unroll
    for (int f = 0; f < S::NFRAG; ++f) {
        const v4i a = win[f % S::WIN];
        const int fr = f + S::WIN;  // fragment to prefetch into this window slot
        if (fr < S::NFRAG)
            win[f % S::WIN] = *xd_frag_ptr<S>(st, fr, wn, frow, fchunk);
        else if (STEADY || t + 1 < KT)
            win[f % S::WIN] = *xd_frag_ptr<S>(st_next, fr - S::NFRAG, wn, frow, fchunk);
        const int ks = f / S::FN, fn = f % S::FN;
#pragma unroll
        for (int fm = 0; fm < S::FM; ++fm) acc[fn][fm] = mfma_i8(a, X[fm][ks], acc[fn][fm]);
        if (f == S::MID) {
            // every read issued so far is of stage t; the next one is of stage t+1
            if (STEADY) {
                // loads issued after weight stage t+1: x(t), w(t+2), x(t+1)
                wait_vmcnt<S::GPW + 2 * S::XL>();
                lds_barrier();
                xd_issue_w<S>(wsrc, (t + 3) * S::BK, smem + ((t + 3) & 3) * S::STAGE, wave);
            } else {
                if (t + 1 < KT) {
                    if (t + 2 < KT) wait_vmcnt<S::GPW + 2 * S::XL>();
                    else wait_vmcnt<2 * S::XL>();
                    lds_barrier();
                }
                if (t + 3 < KT) xd_issue_w<S>(wsrc, (t + 3) * S::BK, smem + ((t + 3) & 3) * S::STAGE, wave);
            }
        }
    }
    // x(t+1) must be complete before the next K-tile; only weights(t+3) may still fly
    if (STEADY || t + 3 < KT) wait_vmcnt<S::GPW>();
    else wait_vmcnt<0>();
}

template <int WGN>
__global__ __launch_bounds__(256 * WGN) void gemm_xd_kernel(GemmProblem p, TileMap tmap) {
    using S = XdShape<WGN>;
    constexpr int FM = S::FM, FN = S::FN, GPW = S::GPW;
    __shared__ __attribute__((aligned(1024))) int8_t smem[S::STAGES * S::STAGE];

    int tm, tn;
    map_tile(tmap, tm, tn);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WGN, wm = wave / WGN;
    const int m0 = tm * S::BM, n0 = tn * S::BN;
    const int M = p.M, N = p.N, K = p.K;
    const int frow = lane & 15, fchunk = lane >> 4;

    // weight DMA: wave w issues row groups g = w + NW j (8 rows x 128 B each) of every stage
    const int8_t *wsrc[GPW];
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int lrow = (wave + j * S::NW) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((lrow >> 1) & 7);
        wsrc[j] = static_cast<const int8_t *>(p.wq) + ((int64_t)min(n0 + lrow, N - 1) * K + 16 * c);
    }
    // activation rows of this wave's fragments
    const int8_t *xrow[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
        xrow[fm] = p.xq + (int64_t)min(m0 + wm * S::WM + fm * 16 + frow, M - 1) * K;

    v4i acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int KT = K / S::BK;
    // prologue: x(0), weight stages 0..2; everything waited
    v4i xa[FM][2], xb[FM][2];
    xd_load_x<S>(xrow, 0, fchunk, xa);
#pragma unroll
    for (int s = 0; s < S::STAGES - 1; ++s)
        if (s < KT) xd_issue_w<S>(wsrc, s * S::BK, smem + s * S::STAGE, wave);
    wait_vmcnt<0>();
    lds_barrier();
    v4i win[S::WIN];
#pragma unroll
    for (int i = 0; i < S::WIN; ++i) win[i] = *xd_frag_ptr<S>(smem, i, wn, frow, fchunk);

    // steady state, two K-tiles per trip so the x buffers alternate statically
    int t = 0;
    for (; t + 4 < KT; t += 2) {
        xd_ktile<S, true>(t, KT, smem, wsrc, xrow, wave, wn, frow, fchunk, win, acc, xa, xb);
        xd_ktile<S, true>(t + 1, KT, smem, wsrc, xrow, wave, wn, frow, fchunk, win, acc, xb, xa);
    }
    // last K-tiles (at most 4)
    for (; t < KT; t += 2) {
        xd_ktile<S, false>(t, KT, smem, wsrc, xrow, wave, wn, frow, fchunk, win, acc, xa, xb);
        if (t + 1 < KT) xd_ktile<S, false>(t + 1, KT, smem, wsrc, xrow, wave, wn, frow, fchunk, win, acc, xb, xa);
    }

    // ---- epilogue (per-channel dequant or raw int32) ----
    const float *__restrict__ sxp = p.sx;
    const float *__restrict__ swp = p.sw;
    float sxm[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sxm[fm] = sxp[min(m0 + wm * S::WM + fm * 16 + frow, M - 1)];
    const int out = p.out;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + wn * S::WN + fn * 16 + 4 * fchunk;
        const float4 s4 = *reinterpret_cast<const float4 *>(swp + min(n, N - 4));
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + wm * S::WM + fm * 16 + frow;
            if (m >= M || n >= N) continue;
            const int64_t off = (int64_t)m * p.ldy + n;
            const v4i v = acc[fn][fm];
            if (out == OUT_I32) {
                *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = make_int4(v[0], v[1], v[2], v[3]);
            } else {
                store4(p.y, off, out, ((float)v[0] * sxm[fm]) * s4.x, ((float)v[1] * sxm[fm]) * s4.y,
                       ((float)v[2] * sxm[fm]) * s4.z, ((float)v[3] * sxm[fm]) * s4.w);
            }
        }
    }
}

template <int WGN>
hipError_t launch_xd(const GemmProblem &p, int group_m, hipStream_t stream) {
    TileMap t;
    t.tiles_m = (p.M + 255) / 256;
    t.tiles_n = (p.N + 255) / 256;
    t.group_m = group_m;
    dim3 grid(t.tiles_m * t.tiles_n), block(256 * WGN);
    hipLaunchKernelGGL(gemm_xd_kernel<WGN>, grid, block, 0, stream, p, t);
    return hipGetLastError();
}


// ---- small-M path: weight-streaming GEMV on matrix cores ------------------------------
//
// For M <= 16 the layer is bound by streaming the weights once from HBM. A workgroup owns
// 16 output rows; its S waves (S = blockDim / 64, at most 8) split K into S contiguous
// segments (whole groups for the per-group path) of at most CH K-steps, so that each
// wave issues every weight load of its segment before its first MFMA: one HBM round
// trip, with all waves of the grid resident at once. Each lane loads its MFMA fragments
// straight from global memory (16 bytes of a weight row, 8 for int4; the token fragment
// from the small x_q), so no LDS is needed on the way in. Tokens m >= M read row M-1 and
// their results are discarded. The S partial tiles are summed through LDS in segment
// order by wave 0 (int32 for per-channel: exact; fp32 for per-group), which also applies
// the dequant and stores.
constexpr int GEMV_MAX_WAVES = 8;

template <int GS, int WK, int CH>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv_kernel(GemmProblem p, int seg_steps) {
    constexpr bool GROUPED = GS > 0;
    constexpr int SPG = GROUPED ? GS / 64 : 1;  // K-steps per group
    constexpr int GPB = GROUPED ? CH / SPG : 1;  // groups per batch
    static_assert(!GROUPED || CH % SPG == 0, "a batch holds whole groups");
    __shared__ __attribute__((aligned(16))) float redf[GROUPED ? GEMV_MAX_WAVES : 1][64][4];
    __shared__ __attribute__((aligned(16))) int redi[GROUPED ? 1 : GEMV_MAX_WAVES][64][4];

    const int S = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int frow = lane & 15, fchunk = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int M = p.M, N = p.N, K = p.K;
    const int G = GROUPED ? K / GS : 1;
    const int KS = K / 64;
    const int ks0 = wave * seg_steps, ks1 = min(KS, ks0 + seg_steps);

    const int8_t *xrow = p.xq + (int64_t)min(frow, M - 1) * K;
    const int nrow = min(n0 + frow, N - 1);
    const int8_t *wrow8 = static_cast<const int8_t *>(p.wq) + (int64_t)nrow * K;
    const uint8_t *wrow4 = static_cast<const uint8_t *>(p.wq) + (int64_t)nrow * (K / 2);

    v4i acc = {0, 0, 0, 0};
    float facc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int kb = ks0; kb < ks1; kb += CH) {
        // every load of the batch first (weights, then tokens, then group scales)
        v4i a8[CH];
        v2u a4[CH];
        v4i b[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ks = min(kb + c, ks1 - 1);
            if constexpr (WK == W_INT4)
                a4[c] = __builtin_nontemporal_load(reinterpret_cast<const v2u *>(wrow4 + ks * 32 + fchunk * 8));
            else
                a8[c] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wrow8 + ks * 64 + fchunk * 16));
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ks = min(kb + c, ks1 - 1);
            b[c] = *reinterpret_cast<const v4i *>(xrow + ks * 64 + fchunk * 16);
        }
        float sw[GROUPED ? GPB : 1][4];
        if constexpr (GROUPED) {
#pragma unroll
            for (int j = 0; j < GPB; ++j) {
                const int g = min(kb / SPG + j, G - 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) sw[j][e] = p.sw[(int64_t)min(n0 + 4 * fchunk + e, N - 1) * G + g];
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (kb + c >= ks1) continue;  // uniform; no early exit, so the loop unrolls fully
            v4i a;
            if constexpr (WK == W_INT4)
                a = __builtin_bit_cast(v4i, unpack_nibbles(a4[c].x, a4[c].y));
            else
                a = a8[c];
            if constexpr (GROUPED) {
                acc = mfma_i8(a, b[c], (c % SPG) == 0 ? v4i{0, 0, 0, 0} : acc);
                if ((c % SPG) == SPG - 1) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) facc[e] = __builtin_fmaf((float)acc[e], sw[c / SPG][e], facc[e]);
                }
            } else {
                acc = mfma_i8(a, b[c], acc);
            }
        }
    }
    // partials -> LDS, summed in segment order by wave 0 (int32 for per-channel: exact)
    if constexpr (GROUPED) {
        *reinterpret_cast<float4 *>(&redf[wave][lane][0]) = make_float4(facc[0], facc[1], facc[2], facc[3]);
    } else {
        *reinterpret_cast<int4 *>(&redi[wave][lane][0]) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
    if (wave != 0) return;
    const int m = frow;
    const int n = n0 + 4 * fchunk;
    if (m >= M || n >= N) return;
    const int64_t off = (int64_t)m * p.ldy + n;
    if constexpr (GROUPED) {
        float4 t = *reinterpret_cast<const float4 *>(&redf[0][lane][0]);
#pragma unroll
        for (int w = 1; w < S; ++w) {
            const float4 u = *reinterpret_cast<const float4 *>(&redf[w][lane][0]);
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        const float sxm = p.sx[m];
        store4(p.y, off, p.out, t.x * sxm, t.y * sxm, t.z * sxm, t.w * sxm);
    } else {
        int4 t = *reinterpret_cast<const int4 *>(&redi[0][lane][0]);
#pragma unroll
        for (int w = 1; w < S; ++w) {
            const int4 u = *reinterpret_cast<const int4 *>(&redi[w][lane][0]);
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        if (p.out == OUT_I32) {
            *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = t;
            return;
        }
        const float sxm = p.sx[m];
        const float4 s4 = *reinterpret_cast<const float4 *>(p.sw + n);
        store4(p.y, off, p.out, ((float)t.x * sxm) * s4.x, ((float)t.y * sxm) * s4.y, ((float)t.z * sxm) * s4.z,
               ((float)t.w * sxm) * s4.w);
    }
}

template <int GS, int WK>
hipError_t launch_gemv(const GemmProblem &p, hipStream_t stream) {
    const int KS = p.K / 64;
    const int blocks = (p.N + 15) / 16;
    const int unit = GS > 0 ? GS / 64 : 1;  // K-steps per group
    // Waves per workgroup: segments of at most 16 K-steps (whole groups), and at least
    // about 2048 waves in the grid while segments stay at 4 K-steps or more.
    int S = (KS + 15) / 16;
    while (S < GEMV_MAX_WAVES && (int64_t)blocks * S < 2048 && (KS + S) / (S + 1) >= 4) ++S;
    S = min(S, GEMV_MAX_WAVES);
    int seg = (KS + S - 1) / S;
    seg = (seg + unit - 1) / unit * unit;
    S = (KS + seg - 1) / seg;
    dim3 grid(blocks), block(64 * S);
    if (seg <= 8)
        hipLaunchKernelGGL((gemv_kernel<GS, WK, 8>), grid, block, 0, stream, p, seg);
    else
        hipLaunchKernelGGL((gemv_kernel<GS, WK, 16>), grid, block, 0, stream, p, seg);
    return hipGetLastError();
}

// ---- small-M path with the weights staged through LDS --------------------------------
//
// Measured on MI355X: global loads in the MFMA operand layout (64 lanes taking 64 bytes
// from each of 16 rows) stream from HBM at about 3.2 TB/s, while loads that take 128
// contiguous bytes or more of each row run at the rate of a plain linear read (~4.1 TB/s
// for a 26 MB matrix in one launch). So the weights go to LDS with global_load_lds in
// pieces of 8 rows x 128 bytes and the fragments are read from there.
//
// A workgroup owns 16 output rows; its S waves split the row's 128-byte chunks into S
// contiguous segments (whole groups for per-group scales). Each wave streams its segment
// through a private ring of up to RING chunk slots (16 rows x 128 bytes, 2 KiB each), so
// no data is shared between waves and no barrier is needed before the final reduction.
// Within a slot, row r's 16-byte piece c sits at position c ^ ((r >> 1) & 7) (the swizzle
// is applied to the DMA source addresses), which keeps the fragment reads free of bank
// conflicts. With XL (when it fits in LDS) the wave's segment of the x_q rows is copied to LDS once,
// up front, and the token fragments are read from there; otherwise (x_q is small and
// stays in L2) they are loaded with each chunk's DMA. Loads that return little data still
// hold a place in the CU's memory queue and retire in order behind the weight stream, so
// at M = 1 half of the queue would carry 16 bytes of useful data per instruction. The
// per-group scales of the wave's segment are put in an LDS table first.
template <int GS, int WK, bool XL>
struct GvShape {
    static constexpr bool GROUPED = GS > 0;
    static constexpr int KPC = WK == W_INT4 ? 256 : 128;  // k values per 128-byte chunk
    static constexpr int SPC = KPC / 64;                  // K-steps per chunk
    static constexpr int RING = WK == W_INT4 ? 4 : 8;     // slots per wave
    static constexpr int OPS = XL ? 2 : 2 + SPC;          // vector-memory ops per chunk
    static constexpr int SPG = GROUPED ? GS / 64 : 1;     // K-steps per group
    static constexpr int GPC = GROUPED ? (SPC >= SPG ? SPC / SPG : 1) : 1;  // groups per chunk
    static constexpr int CPG = GROUPED ? (SPG > SPC ? SPG / SPC : 1) : 1;   // chunks per group
};

template <class S, int N>
__device__ __forceinline__ void gv_wait_tail(int after) {
    // vmcnt wait allowing `after` chunks (S::OPS ops each) issued after the one needed
    if constexpr (N > 0) {
        if (after >= N) {
            wait_vmcnt<S::OPS * N>();
            return;
        }
        gv_wait_tail<S, N - 1>(after);
    } else {
        wait_vmcnt<0>();
    }
}

template <int GS, int WK, bool XL, int FQ>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv_dma_kernel(GemmProblem p, int seg_chunks, int slots,
                                                                        int table_groups) {
    using S = GvShape<GS, WK, XL>;
    // FQ: 0 = x_q given; 1 / 2 = quantize fp16 / bf16 rows of p.x here (needs XL)
    static_assert(FQ == 0 || XL, "in-kernel quantization writes the codes to the LDS token region");
    constexpr bool BF16X = FQ == 2;
    constexpr int RING = S::RING, SPC = S::SPC;
    extern __shared__ __attribute__((aligned(1024))) int8_t gv_lds[];

    const int NW = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int frow = lane & 15, fchunk = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int M = p.M, N = p.N, K = p.K;
    const int G = S::GROUPED ? K / GS : 1;
    const int NCH = K / S::KPC;
    const int c0 = wave * seg_chunks, nch = max(min(NCH, c0 + seg_chunks) - c0, 0);
    const int RB = WK == W_INT4 ? K / 2 : K;  // bytes per weight row

    int8_t *my_ring = gv_lds + wave * slots * 2048;
    float *table = reinterpret_cast<float *>(gv_lds + NW * slots * 2048) + wave * table_groups * 16;
    // XL region of this wave: room for M rows of seg_chunks * KPC bytes (rounded up to 1 KiB)
    const int xl_bytes = (M * seg_chunks * S::KPC + 1023) & ~1023;
    int8_t *xl = gv_lds + NW * slots * 2048 + NW * table_groups * 64 + wave * xl_bytes;
    // FQ: this wave's fp16 / bf16 x segment (twice the code bytes), then row maxima [NW][16]
    const int xh_bytes = FQ ? (2 * M * seg_chunks * S::KPC + 1023) & ~1023 : 0;
    int8_t *xh = gv_lds + NW * slots * 2048 + NW * table_groups * 64 + NW * xl_bytes + wave * xh_bytes;
    uint32_t *pmax = reinterpret_cast<uint32_t *>(gv_lds + NW * slots * 2048 + NW * table_groups * 64 +
                                                  NW * xl_bytes + NW * xh_bytes);

    // the epilogue's scales, fetched first so that they arrive with the weight stream
    // (retired by the first chunk wait: they precede every DMA)
    const int em = min(frow, M - 1), en = min(n0 + 4 * fchunk, N - 4);
    float e_sx = 0.f;
    float4 e_sw = make_float4(0.f, 0.f, 0.f, 0.f);
    if (wave == 0) {
        if constexpr (FQ == 0) e_sx = p.sx[em];
        if constexpr (!S::GROUPED) e_sw = *reinterpret_cast<const float4 *>(p.sw + en);
    }

    // per-group scales of this wave's segment: table[(g - g0) * 16 + r] = s_w[n0 + r, g],
    // copied with 4-byte DMA (64 entries per instruction; table_groups is a multiple of 4)
    // so that no register waits on them: the first chunk wait retires them
    const int g0 = S::GROUPED ? (c0 * SPC) / S::SPG : 0;
    if constexpr (S::GROUPED) {
        const int ng = min(G - g0, table_groups);
        for (int b = 0; b * 64 < ng * 16; ++b) {
            const int e = b * 64 + lane;
            const int gg = min(e >> 4, ng - 1), r = e & 15;
            dma_4B(p.sw + (int64_t)min(n0 + r, N - 1) * G + g0 + gg, table + b * 64);
        }
    }

    // DMA roles: lane i of a piece covers row (half * 8 + i / 8), slot position i % 8,
    // which holds the row's logical 16-byte piece (i % 8) ^ ((row >> 1) & 7)
    const int dr = lane >> 3, dpos = lane & 7;
    const uint8_t *W = static_cast<const uint8_t *>(p.wq);
    const uint8_t *src_lo = W + (int64_t)min(n0 + dr, N - 1) * RB + 16 * (dpos ^ ((dr >> 1) & 7));
    const uint8_t *src_hi = W + (int64_t)min(n0 + 8 + dr, N - 1) * RB + 16 * (dpos ^ (((8 + dr) >> 1) & 7));
    const int8_t *xrow = p.xq + (int64_t)min(frow, M - 1) * K;

    v4i xf[RING][SPC];  // token fragments of the chunks in flight, by slot

    // XL: rows 0..M-1 of x_q, bytes [c0 KPC, (c0 + nch) KPC) (this wave's chunks only, so
    // never past the row end), stored flat with row stride xlr; 1 KiB per DMA, lane i
    // taking flat byte 1024 b + 16 i (clamped to the last row's end)
    const int xlr = nch * S::KPC;
    if constexpr (FQ != 0) {
        // the same rows of x (2 bytes per element), flat with row stride 2 xlr
        const int total = 2 * M * xlr;
        for (int b = 0; b * 1024 < total; ++b) {
            const int flat = min(b * 1024 + 16 * lane, total - 16);
            const int r = flat / (2 * xlr), col = flat - r * (2 * xlr);
            dma_16B(static_cast<const int8_t *>(p.x) + 2 * ((int64_t)r * p.ldx + c0 * S::KPC) + col, xh + b * 1024);
        }
    } else if constexpr (XL) {
        const int total = M * xlr;
        for (int b = 0; b * 1024 < total; ++b) {
            const int flat = min(b * 1024 + 16 * lane, total - 16);
            const int r = flat / xlr, col = flat - r * xlr;
            dma_16B(p.xq + (int64_t)r * K + c0 * S::KPC + col, xl + b * 1024);
        }
    }
    const int8_t *xl_row = xl + min(frow, M - 1) * xlr;

    v4i acc = {0, 0, 0, 0};
    float facc[4] = {0.f, 0.f, 0.f, 0.f};
    // One chunk's MFMAs from ring slot `slot` (token fragments from xl_row, or xf[s]).
    auto chunk_mma = [&](int j, const int8_t *slot, const v4i *xfs) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < SPC; ++t) {
            v4i a;
            if constexpr (WK == W_INT4) {
                // K-step t: bytes 32 t + 8 fchunk of the row's 128
                // (read as the whole 16-byte piece: with 8-byte LDS reads here the compiler
                // waits for every weight DMA in flight before each read)
                const int byte = t * 32 + fchunk * 8;
                const v4i q = *reinterpret_cast<const v4i *>(slot + frow * 128 + (((byte >> 4) ^ ((frow >> 1) & 7)) << 4));
                const uint2 w = (byte & 8) ? make_uint2(q[2], q[3]) : make_uint2(q[0], q[1]);
                // 16 q: grouped, facc holds 16 t; per channel and the raw int32 sums, the
                // sums of 16 q are shifted back at the end (K <= kInt4X16MaxK)
                a = __builtin_bit_cast(v4i, unpack_nibbles_x16(w.x, w.y));
            } else {
                a = *reinterpret_cast<const v4i *>(slot + frow * 128 + (((t * 4 + fchunk) ^ ((frow >> 1) & 7)) << 4));
            }
            const v4i bx = XL ? *reinterpret_cast<const v4i *>(xl_row + j * S::KPC + t * 64 + fchunk * 16) : xfs[t];
            if constexpr (S::GROUPED) {
                const int ks = (c0 + j) * SPC + t;  // global K-step
                acc = mfma_i8(a, bx, (ks % S::SPG) == 0 ? v4i{0, 0, 0, 0} : acc);
                if ((ks % S::SPG) == S::SPG - 1) {
                    // (the table's DMA was retired by the first chunk wait)
                    const float4 sw = lds_read_f4_now(table + (ks / S::SPG - g0) * 16 + 4 * fchunk);
                    facc[0] = __builtin_fmaf((float)acc[0], sw.x, facc[0]);
                    facc[1] = __builtin_fmaf((float)acc[1], sw.y, facc[1]);
                    facc[2] = __builtin_fmaf((float)acc[2], sw.z, facc[2]);
                    facc[3] = __builtin_fmaf((float)acc[3], sw.w, facc[3]);
                }
            } else {
                acc = mfma_i8(a, bx, acc);
            }
        }
    };
    if constexpr (XL) {
        // ring of `slots` slots (any depth <= RING), chunk j in slot j % slots
        const int R = min(slots, nch);
        // With in-kernel quantization only the first chunks go out before it: a wave blocks
        // while issuing into a full memory queue, and the quantization should run while the
        // first weights are in flight, not after the whole prologue has been issued.
        const int R0 = FQ != 0 ? min(R, 2) : R;
        for (int j = 0; j < R0; ++j) {
            dma_16B(src_lo + (c0 + j) * 128, my_ring + j * 2048);
            dma_16B(src_hi + (c0 + j) * 128, my_ring + j * 2048 + 1024);
        }
        if constexpr (FQ != 0) {
            // In-kernel activation quantization, with the arithmetic of the quantize kernel.
            // The x copy and the scale table precede the R0 chunk DMAs (2 ops each).
            gv_wait_tail<S, 2>(R0);
            const int nc8 = xlr / 8;  // 16-byte pieces (8 elements) of a row segment
            for (int m = 0; m < M; ++m) {
                act::u16x2 mm = {0, 0};
                for (int c = lane; c < nc8; c += 64)
                    mm = act::absmax8(*reinterpret_cast<const uint4 *>(xh + m * 2 * xlr + 16 * c), mm);
                const uint32_t a = act::wave_max_u32(mm.x > mm.y ? mm.x : mm.y);
                if (lane == 0) pmax[wave * 16 + m] = a;
            }
            __syncthreads();
            const bool out0 = blockIdx.x == 0;
            for (int m = 0; m < M; ++m) {
                uint32_t a = 0;
                for (int w = 0; w < NW; ++w) a = max(a, pmax[w * 16 + m]);
                const float sc = act::row_scale<BF16X>(a);
                if (em == m) e_sx = sc;
                if (out0 && wave == 0 && lane == 0) p.sx_out[m] = sc;
                const int8_t *hrow = xh + m * 2 * xlr;
                int8_t *crow = xl + m * xlr;
                int8_t *grow = p.xq_out + (int64_t)m * K + c0 * S::KPC;
                if (sc == 0.0f) {
                    for (int c = lane; c < nc8; c += 64) {
                        *reinterpret_cast<uint2 *>(crow + 8 * c) = make_uint2(0, 0);
                        if (out0) *reinterpret_cast<uint2 *>(grow + 8 * c) = make_uint2(0, 0);
                    }
                } else if (sc >= act::kMinFastScale) {
                    const float rc = 1.0f / sc;
                    for (int c = lane; c < nc8; c += 64) {
                        const uint2 q = act::quant8<BF16X, true>(*reinterpret_cast<const uint4 *>(hrow + 16 * c), sc, rc);
                        *reinterpret_cast<uint2 *>(crow + 8 * c) = q;
                        if (out0) *reinterpret_cast<uint2 *>(grow + 8 * c) = q;
                    }
                } else {
                    for (int c = lane; c < nc8; c += 64) {
                        const uint2 q = act::quant8<BF16X, false>(*reinterpret_cast<const uint4 *>(hrow + 16 * c), sc, 0.f);
                        *reinterpret_cast<uint2 *>(crow + 8 * c) = q;
                        if (out0) *reinterpret_cast<uint2 *>(grow + 8 * c) = q;
                    }
                }
            }
            for (int j = R0; j < R; ++j) {
                dma_16B(src_lo + (c0 + j) * 128, my_ring + j * 2048);
                dma_16B(src_hi + (c0 + j) * 128, my_ring + j * 2048 + 1024);
            }
        }
        int sl = 0;
        for (int j = 0; j < nch; ++j) {
            // chunks issued so far: min(nch, j + R); those after chunk j may be in flight
            gv_wait_tail<S, RING - 1>(min(nch, j + R) - j - 1);
            chunk_mma(j, my_ring + sl * 2048, nullptr);
            if (j + R < nch) {
                wait_lgkmcnt0();  // the slot's fragment reads are done before it is refilled
                dma_16B(src_lo + (c0 + j + R) * 128, my_ring + sl * 2048);
                dma_16B(src_hi + (c0 + j + R) * 128, my_ring + sl * 2048 + 1024);
            }
            sl = sl + 1 == R ? 0 : sl + 1;
        }
    } else {
        // ring of RING slots (the launcher gives min(RING, seg_chunks)), chunk j in slot
        // j % RING; the token fragments of a slot live in registers, so slots are constants
#pragma unroll
        for (int s = 0; s < RING; ++s)
            if (s < nch) {
                const int ck = c0 + s;
                dma_16B(src_lo + ck * 128, my_ring + s * 2048);
                dma_16B(src_hi + ck * 128, my_ring + s * 2048 + 1024);
#pragma unroll
                for (int t = 0; t < SPC; ++t)
                    xf[s][t] = *reinterpret_cast<const v4i *>(xrow + ck * S::KPC + t * 64 + fchunk * 16);
            }
        for (int j0 = 0; j0 < nch; j0 += RING) {
#pragma unroll
            for (int s = 0; s < RING; ++s) {
                const int j = j0 + s;
                if (j < nch) {
                    gv_wait_tail<S, RING - 1>(min(nch, j + RING) - j - 1);
                    chunk_mma(j, my_ring + s * 2048, xf[s]);
                    if (j + RING < nch) {
                        wait_lgkmcnt0();
                        const int ck = c0 + j + RING;
                        dma_16B(src_lo + ck * 128, my_ring + s * 2048);
                        dma_16B(src_hi + ck * 128, my_ring + s * 2048 + 1024);
#pragma unroll
                        for (int t = 0; t < SPC; ++t)
                            xf[s][t] = *reinterpret_cast<const v4i *>(xrow + ck * S::KPC + t * 64 + fchunk * 16);
                    }
                }
            }
        }
    }

    // partials -> LDS (the ring space, once every wave is done with it), summed in
    // segment order by wave 0 (int32 for per-channel: exact)
    __syncthreads();
    if constexpr (S::GROUPED) {
        float4 *red = reinterpret_cast<float4 *>(gv_lds);
        red[wave * 64 + lane] = make_float4(facc[0], facc[1], facc[2], facc[3]);
    } else {
        int4 *red = reinterpret_cast<int4 *>(gv_lds);
        red[wave * 64 + lane] = make_int4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
    if (wave != 0) return;
    const int m = frow;
    const int n = n0 + 4 * fchunk;
    if (m >= M || n >= N) return;
    const int64_t off = (int64_t)m * p.ldy + n;
    if constexpr (S::GROUPED) {
        const float4 *red = reinterpret_cast<const float4 *>(gv_lds);
        float4 t = red[lane];
        for (int w = 1; w < NW; ++w) {
            const float4 u = red[w * 64 + lane];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        // int4: the partials are 16 x the sums (codes unpacked as 16 q); 2^-4 is exact
        constexpr float TS = WK == W_INT4 ? 0.0625f : 1.0f;
        store4(p.y, off, p.out, (t.x * TS) * e_sx, (t.y * TS) * e_sx, (t.z * TS) * e_sx, (t.w * TS) * e_sx);
    } else {
        const int4 *red = reinterpret_cast<const int4 *>(gv_lds);
        int4 t = red[lane];
        for (int w = 1; w < NW; ++w) {
            const int4 u = red[w * 64 + lane];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        if constexpr (WK == W_INT4) t = make_int4(t.x >> 4, t.y >> 4, t.z >> 4, t.w >> 4);  // exact
        if (p.out == OUT_I32) {
            *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = t;
            return;
        }
        store4(p.y, off, p.out, ((float)t.x * e_sx) * e_sw.x, ((float)t.y * e_sx) * e_sw.y,
               ((float)t.z * e_sx) * e_sw.z, ((float)t.w * e_sx) * e_sw.w);
    }
}

// Launch of the LDS-staged GEMV; returns hipErrorNotSupported (without launching) when the
// shape does not fit it, and the caller then uses the direct-load GEMV.
template <int GS, int WK, bool XL, int FQ = 0>
hipError_t launch_gemv_dma_x(const GemmProblem &p, hipStream_t stream) {
    using S = GvShape<GS, WK, XL>;
    const int RB = WK == W_INT4 ? p.K / 2 : p.K;
    if (RB % 128 != 0 || p.M > 16) return hipErrorNotSupported;
    // int4 per channel / raw sums: int32 sums of 16 q (longer K: the register-staged GEMV,
    // or quantize + GEMM for the fused call)
    if (WK == W_INT4 && GS == 0 && p.K > kInt4X16MaxK) return hipErrorNotSupported;
    // in-kernel quantization copies x rows with 16-byte DMA: rows must start 16-byte aligned
    if (FQ && ((reinterpret_cast<uintptr_t>(p.x) & 15) != 0 || (p.ldx * 2) % 16 != 0)) return hipErrorNotSupported;
    const int NCH = p.K / S::KPC;
    const int blocks = (p.N + 15) / 16;
    // waves per workgroup: segments of at most RING chunks where possible, at least about
    // 2048 waves in the grid while each wave keeps 2 chunks or more; whole groups
    const int unit = S::GROUPED ? S::CPG : 1;
    int NW = min(GEMV_MAX_WAVES, max(1, (NCH + S::RING - 1) / S::RING));
    while (NW < GEMV_MAX_WAVES && (int64_t)blocks * NW < 2048 && NCH / (NW + 1) >= 2) ++NW;
    int seg = (NCH + NW - 1) / NW;
    seg = (seg + unit - 1) / unit * unit;
    NW = (NCH + seg - 1) / seg;
    // With x_q given, segments of equal length where a few more waves allow it: the int4
    // rows of K = 2560 (10 chunks) as 5 x 2 instead of 3 + 3 + 3 + 1 chunks (M=1, N=10240:
    // 6.51 -> 6.13 us per group, 5.71 -> 5.52 us per column). The fused layer keeps the
    // split above: every extra wave also copies and reduces its part of x (7.77 against
    // 7.95 us with five waves).
    if (FQ == 0 && NCH % seg != 0) {
        for (int nw = NW + 1; nw <= GEMV_MAX_WAVES; ++nw) {
            const int s = ((NCH + nw - 1) / nw + unit - 1) / unit * unit;
            if (s >= 2 && NCH % s == 0) {
                seg = s;
                NW = NCH / s;
                break;
            }
        }
    }
    const int table_groups = S::GROUPED ? ((seg * S::SPC + S::SPG - 1) / S::SPG + 1 + 3) & ~3 : 0;
    const size_t xl = XL ? (size_t)((p.M * seg * S::KPC + 1023) & ~1023) : 0;
    const size_t xh = FQ ? (size_t)((2 * p.M * seg * S::KPC + 1023) & ~1023) : 0;
    // ring slots: as many as fit while every workgroup of the grid is resident at once
    const int per_cu = (blocks + num_cus() - 1) / num_cus();
    const size_t budget = (size_t)160 * 1024 / per_cu;
    const size_t fixed = (size_t)NW * (table_groups * 16 * sizeof(float) + xl + xh) + (FQ ? (size_t)NW * 16 * 4 : 0);
    if (budget <= fixed) return hipErrorNotSupported;
    const int fit = (int)((budget - fixed) / ((size_t)NW * 2048));
    const int slots = min(min(S::RING, seg), fit);
    // the register-token variant cycles through min(RING, seg) slots; the LDS-token one
    // through `slots`, of which it needs 2 unless the segment is a single chunk
    if (!XL && slots < min(S::RING, seg)) return hipErrorNotSupported;
    if (slots < 2 && slots < seg) return hipErrorNotSupported;
    const size_t lds = (size_t)NW * slots * 2048 + fixed;
    if (lds > 160 * 1024 || slots < 1) return hipErrorNotSupported;
    hipLaunchKernelGGL((gemv_dma_kernel<GS, WK, XL, FQ>), dim3(blocks), dim3(64 * NW), lds, stream, p, seg, slots,
                       table_groups);
    return hipGetLastError();
}

template <int GS, int WK>
hipError_t launch_gemv_dma(const GemmProblem &p, hipStream_t stream) {
    {
        const hipError_t e = launch_gemv_dma_x<GS, WK, true>(p, stream);
        if (e != hipErrorNotSupported) return e;
    }
    return launch_gemv_dma_x<GS, WK, false>(p, stream);
}

template <int GS, int WK>
hipError_t launch_gemv_any(const GemmProblem &p, hipStream_t stream) {
    const hipError_t e = launch_gemv_dma<GS, WK>(p, stream);
    return e == hipErrorNotSupported ? launch_gemv<GS, WK>(p, stream) : e;
}

hipError_t dispatch_gemv(const GemmProblem &p, hipStream_t stream) {
    const int gs = p.out == OUT_I32 ? 0 : p.gs;
    if (p.wkind == W_INT4) {
        if (gs == 64) return launch_gemv_any<64, W_INT4>(p, stream);
        if (gs == 128) return launch_gemv_any<128, W_INT4>(p, stream);
        return launch_gemv_any<0, W_INT4>(p, stream);
    }
    if (gs == 64) return launch_gemv_any<64, W_INT8>(p, stream);
    if (gs == 128) return launch_gemv_any<128, W_INT8>(p, stream);
    return launch_gemv_any<0, W_INT8>(p, stream);
}

template <int FQ>
hipError_t linear_small_fq(const GemmProblem &p, hipStream_t stream) {
    const int gs = p.gs;
    if (p.wkind == W_INT4) {
        if (gs == 64) return launch_gemv_dma_x<64, W_INT4, true, FQ>(p, stream);
        if (gs == 128) return launch_gemv_dma_x<128, W_INT4, true, FQ>(p, stream);
        return launch_gemv_dma_x<0, W_INT4, true, FQ>(p, stream);
    }
    if (gs == 64) return launch_gemv_dma_x<64, W_INT8, true, FQ>(p, stream);
    if (gs == 128) return launch_gemv_dma_x<128, W_INT8, true, FQ>(p, stream);
    return launch_gemv_dma_x<0, W_INT8, true, FQ>(p, stream);
}

// ---- split-K: the sum of the slices and the dequantization ---------------------------
//
// Thread i covers the outputs (m, n .. n + 3) with m N + n = 4 i. The slices are added in
// slice order, up to eight loads in flight at a time. Per-channel (and I32 output): int32
// sums, exact in any order, then the arithmetic of the single-pass epilogue, so the result is
// bit-identical to the single-pass kernels. Per-group: the slices' fp32 folds are added,
// then y = t * s_x[m].
template <bool GROUPED>
__global__ __launch_bounds__(256) void splitk_finish_kernel(GemmProblem p) {
    const int N = p.N, S = p.ksplit;
    const int64_t quads = (int64_t)p.M * N / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < quads; i += (int64_t)gridDim.x * 256) {
        const int m = (int)(4 * i / N), n = (int)(4 * i - (int64_t)m * N);
        const int64_t off = (int64_t)m * p.ldy + n;
        if constexpr (GROUPED) {
            const float4 *ws = static_cast<const float4 *>(p.ws) + i;
            float4 t = ws[0];
            for (int s0 = 1; s0 < S; s0 += 8) {
                float4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (s0 + j < S) v[j] = ws[(s0 + j) * quads];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (s0 + j < S) {
                        t.x += v[j].x;
                        t.y += v[j].y;
                        t.z += v[j].z;
                        t.w += v[j].w;
                    }
            }
            const float sx = p.sx[m];
            store4(p.y, off, p.out, t.x * sx, t.y * sx, t.z * sx, t.w * sx);
        } else {
            const int4 *ws = static_cast<const int4 *>(p.ws) + i;
            int4 a = ws[0];
            for (int s0 = 1; s0 < S; s0 += 8) {
                int4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (s0 + j < S) v[j] = ws[(s0 + j) * quads];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (s0 + j < S) {
                        a.x += v[j].x;
                        a.y += v[j].y;
                        a.z += v[j].z;
                        a.w += v[j].w;
                    }
            }
            if (p.out == OUT_I32) {
                *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + off) = a;
            } else {
                const float sx = p.sx[m];
                const float4 sw = *reinterpret_cast<const float4 *>(p.sw + n);
                store4(p.y, off, p.out, ((float)a.x * sx) * sw.x, ((float)a.y * sx) * sw.y, ((float)a.z * sx) * sw.z,
                       ((float)a.w * sx) * sw.w);
            }
        }
    }
}

// ---- configuration table ------------------------------------------------------------

struct Config {
    int bm, bn, group_m;
};

// Index = config id for w8a8_debug_force_config.
constexpr Config kConfigs[] = {
    {128, 128, 4},  // 0: 4 waves, 64x64 per wave
    {256, 256, 4},  // 1: 8 waves, 128x64 per wave
    {256, 128, 4},  // 2: 4 waves, 128x64 per wave
    {128, 256, 4},  // 3: 4 waves, 64x128 per wave
    {64, 64, 4},    // 4: 4 waves, 32x32 per wave (small M / narrow N)
    {256, 256, 4},  // 5: direct-to-LDS, BN=256 BM=256, 2 stages, 8 waves (64 n x 128 m each)
    {256, 160, 4},  // 6: direct-to-LDS, BN=160 BM=256, 3 stages, 8 waves (80 n x 64 m each)
    {256, 128, 4},  // 7: direct-to-LDS, BN=128 BM=256, 3 stages, 8 waves (64 n x 64 m each)
    {256, 256, 4},  // 8: weights via 4-stage LDS ring, activations direct, 4 waves (256 n x 64 m each)
    {256, 256, 4},  // 9: weights via 4-stage LDS ring, activations direct, 8 waves (128 n x 64 m each)
    {16, 16, 1},    // 10: small-M weight-streaming GEMV (M <= 16)
    {256, 128, 4},  // 11: per-group / W4A8 on the direct-to-LDS pipeline, BN=128 BM=256 (per-channel: 7)
    {64, 64, 4},    // 12: direct-to-LDS, BN=64 BM=64, 4 stages, 4 waves (32 n x 32 m each); small M
    {256, 320, 8},  // 13: direct-to-LDS, BN=320 BM=256, 4 stages of 64, two wave groups in alternation
    {128, 128, 4},  // 14: direct-to-LDS, BN=128 BM=128, 4 stages, 4 waves (64 n x 64 m each)
    {128, 64, 4},   // 15: direct-to-LDS, BN=64 BM=128, 6 stages, 8 waves (32 n x 32 m each); mid M
    {256, 320, 8},  // 16: as 13 with two stages of 128-value K-tiles (128-byte DMA row segments)
    {256, 320, 8},  // 17: as 16 with int4 weights (per-channel scales or raw int32 sums) and the four-part epilogue; int8: 16
    {256, 256, 8},  // 18: as 16 with 256 x 256 tiles (64 x 128 per wave)
    {256, 320, 8},  // 19: as 16 with each wave's DMA of a stage split over two memory phases and the epilogue in four parts
    {256, 256, 8},  // 20: as 18 with the split DMA and four-part epilogue of 19
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

template <int BM, int BN, int WGM, int WGN, int GS, int WK>
hipError_t launch_cfg(const GemmProblem &p, int group_m, hipStream_t stream) {
    TileMap t;
    t.tiles_m = (p.M + BM - 1) / BM;
    t.tiles_n = (p.N + BN - 1) / BN;
    t.group_m = group_m;
    dim3 grid(t.tiles_m * t.tiles_n), block(64 * WGM * WGN);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, 128, WGM, WGN, GS, WK>), grid, block, 0, stream, p, t);
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_shape(const GemmProblem &p, int group_m, hipStream_t stream) {
    // I32 output is the raw sum over all of K: the ungrouped kernel.
    if (p.wkind == W_INT4) return launch_cfg<BM, BN, WGM, WGN, 0, W_INT4>(p, group_m, stream);
    return launch_cfg<BM, BN, WGM, WGN, 0, W_INT8>(p, group_m, stream);
}

// Grouped (per-group scale) kernels keep an fp32 accumulator beside the int32 one, so
// only the tile shapes whose registers hold both without spilling are instantiated.
template <int BM, int BN, int WGM, int WGN>
hipError_t launch_grouped(const GemmProblem &p, int group_m, hipStream_t stream) {
    if (p.wkind == W_INT4) {
        if (p.gs == 64) return launch_cfg<BM, BN, WGM, WGN, 64, W_INT4>(p, group_m, stream);
        return launch_cfg<BM, BN, WGM, WGN, 128, W_INT4>(p, group_m, stream);
    }
    if (p.gs == 64) return launch_cfg<BM, BN, WGM, WGN, 64, W_INT8>(p, group_m, stream);
    return launch_cfg<BM, BN, WGM, WGN, 128, W_INT8>(p, group_m, stream);
}

template <int BN, int BM, int STAGES, int WGN, int WGM, bool SPLIT = false>
hipError_t launch_ms(const GemmProblem &p, int group_m, hipStream_t stream) {
    TileMap t;
    t.tiles_m = (p.M + BM - 1) / BM;
    t.tiles_n = (p.N + BN - 1) / BN;
    t.group_m = group_m;
    dim3 grid(t.tiles_m * t.tiles_n * (SPLIT ? p.ksplit : 1)), block(64 * WGM * WGN);
    hipLaunchKernelGGL((gemm_ms_kernel<BN, BM, STAGES, WGN, WGM, SPLIT>), grid, block, 0, stream, p, t);
    return hipGetLastError();
}


template <int BN, int BM, int STAGES, int BKS = 64, int WK = W_INT8, int SPREAD = 0, int EPI = 2>
hipError_t launch_pp(const GemmProblem &p, int group_m, hipStream_t stream) {
    TileMap t;
    t.tiles_m = (p.M + BM - 1) / BM;
    t.tiles_n = (p.N + BN - 1) / BN;
    t.group_m = group_m;
    dim3 grid(t.tiles_m * t.tiles_n), block(512);
    hipLaunchKernelGGL((gemm_pp_kernel<BN, BM, STAGES, BKS, WK, SPREAD, EPI>), grid, block, 0, stream, p, t);
    return hipGetLastError();
}

template <int BN, int BM, int STAGES, int WGN, int WGM, int GS, int WK, bool SPLIT>
hipError_t launch_mg(const GemmProblem &p, int group_m, hipStream_t stream) {
    TileMap t;
    t.tiles_m = (p.M + BM - 1) / BM;
    t.tiles_n = (p.N + BN - 1) / BN;
    t.group_m = group_m;
    dim3 grid(t.tiles_m * t.tiles_n * (SPLIT ? p.ksplit : 1)), block(64 * WGM * WGN);
    hipLaunchKernelGGL((gemm_mg_kernel<BN, BM, STAGES, WGN, WGM, GS, WK, SPLIT>), grid, block, 0, stream, p, t);
    return hipGetLastError();
}

// Per-group / W4A8 on the DMA pipeline: 128 x 256 tiles, or 64 x 64 for small M.
template <bool SPLIT = false>
hipError_t dispatch_mg(const GemmProblem &p, bool small, int group_m, hipStream_t stream) {
    if (p.gs == 0 || p.out == OUT_I32) {
        // per-channel scales or the raw int32 sums: the GS = 0 form, int4 weights only
        // (int8 weights take the per-channel kernels)
        if (p.wkind != W_INT4) return hipErrorInvalidValue;
        return small ? launch_mg<64, 64, 4, 2, 2, 0, W_INT4, SPLIT>(p, group_m, stream)
                     : launch_mg<128, 256, 3, 2, 4, 0, W_INT4, SPLIT>(p, group_m, stream);
    }
    if (small) {
        if (p.wkind == W_INT4)
            return p.gs == 64 ? launch_mg<64, 64, 4, 2, 2, 64, W_INT4, SPLIT>(p, group_m, stream)
                              : launch_mg<64, 64, 4, 2, 2, 128, W_INT4, SPLIT>(p, group_m, stream);
        return p.gs == 64 ? launch_mg<64, 64, 4, 2, 2, 64, W_INT8, SPLIT>(p, group_m, stream)
                          : launch_mg<64, 64, 4, 2, 2, 128, W_INT8, SPLIT>(p, group_m, stream);
    }
    if (p.wkind == W_INT4) {
        // waves of 32 weight rows x 128 tokens: each packed weight fragment is unpacked by
        // two waves instead of four (gs=128 M=4096 N=10240 K=2560: 161 against 173 us with
        // 64 x 64 per wave; gs=64 197 against 214), for 25 % more fragment reads
        if (p.gs == 64) return launch_mg<128, 256, 3, 4, 2, 64, W_INT4, SPLIT>(p, group_m, stream);
        return launch_mg<128, 256, 3, 4, 2, 128, W_INT4, SPLIT>(p, group_m, stream);
    }
    if (p.gs == 64) return launch_mg<128, 256, 3, 2, 4, 64, W_INT8, SPLIT>(p, group_m, stream);
    return launch_mg<128, 256, 3, 2, 4, 128, W_INT8, SPLIT>(p, group_m, stream);
}

// The GS = 0 form of gemm_mg_kernel and the int4 form of gemm_pp_kernel serve int4 weights
// with per-channel scales, and the raw int32 sums of int4 weights (sums of 16 q).
bool mg_per_channel(const GemmProblem &p) {
    return p.wkind == W_INT4 && (p.gs == 0 || p.out == OUT_I32) && p.K % 128 == 0 && p.K <= kInt4X16MaxK;
}

int choose_config(const GemmProblem &p) {
    // Measured on MI355X (fp16 out, M = 32 .. 8192, N = 2560 .. 12288, K = 2560 .. 12288).
    if (p.M <= 16) return 10;  // weight-streaming GEMV
    const bool dma = p.K % 128 == 0;
    const int64_t cus = num_cus();
    if (mg_per_channel(p)) {
        // int4 weights, one scale per output channel (or the raw int32 sums): with enough tiles
        // the 320 x 256 ping-pong form with the unpack in its memory phase, or the per-group DMA
        // kernels without the fold, by rounds of tiles x tile area over the work rate per unit
        // area (1.44 : 1, measured: M = 4096, N = 10240, K = 2560 96.6 against 138.7 us; M =
        // 1024 45.1 against 55.6; M = 8192, N = 2560, K = 10240 153.1 against 282.7); few tiles:
        // as for per-group int4 weights
        const int64_t t11 = (int64_t)((p.M + 255) / 256) * ((p.N + 127) / 128);
        const int64_t t17 = (int64_t)((p.M + 255) / 256) * ((p.N + 319) / 320);
        if (t11 >= cus / 2) {
            const double c11 = (double)((t11 + cus - 1) / cus) * 128 * 256;
            const double c17 = (double)((t17 + cus - 1) / cus) * 320 * 256 / 1.44;
            return c17 < c11 ? 17 : 11;
        }
        return p.M <= 1024 ? 12 : 4;
    }
    if (p.gs > 0 && p.out != OUT_I32) {
        // per-group: the 128 x 256 DMA kernel once it has enough tiles to spread over the
        // chip, else 64 x 64 DMA tiles up to M = 768 (int8) / 1024 (int4), else the
        // register-staged 64 x 64 kernel (measured at N = 2560, K = 10240: M = 768 gs 128
        // 76.7 us against 86.6, M = 1024 148 against 95.6); without 128-value K-tiles the
        // register-staged kernels
        if (!dma) return p.M <= 128 ? 4 : 0;
        const int64_t t11 = (int64_t)((p.M + 255) / 256) * ((p.N + 127) / 128);
        if (t11 >= cus / 2) return 11;
        return p.M <= (p.wkind == W_INT4 ? 1024 : 768) ? 12 : 4;
    }
    if (!dma || p.wkind != W_INT8) return p.M <= 128 ? 4 : 1;
    // 16 < M <= 2048 (too few tiles for the large shapes): the largest of 128 x 128,
    // 64 x 128 and 64 x 64 whose full tiles make one round of workgroups that fills more
    // than half of the chip; measured on MI355X at M = 64 .. 2048, N = 1024 .. 10240,
    // K = 2560 .. 10240 (e.g. M = 128, N = 10240: 64 x 128 14.8 us against 16.2 for 64 x 64;
    // M = 256: 128 x 128 18.7 against 21.4; M = 768, N = 2560, K = 10240: 64 x 128 36.7
    // against 46.0; M = 1536: 128 x 128 53.9 against 71.5; M = 2048, N = 1024, K = 4096:
    // 64 x 128 16.6 against 19.2)
    if (p.M <= 2048) {
        const struct { int id, bm, bn; } one_round[] = {{14, 128, 128}, {15, 128, 64}, {12, 64, 64}};
        for (const auto &c : one_round) {
            const int64_t t = (int64_t)((p.M + c.bm - 1) / c.bm) * ((p.N + c.bn - 1) / c.bn);
            if (p.M % c.bm == 0 && t > cus / 2 && t <= cus) return c.id;
        }
    }
    // per-channel: among the DMA kernels, the fewest chip-wide rounds of tiles times tile
    // area over the kernel's work rate per unit area (320 x 256 in alternating wave
    // groups with 128-value stages: 1.2, 160 x 256: 1.0, 128 x 256: 0.9, 64 x 64: 0.4);
    // partial tiles and a partly filled last round cost whole ones. (With 1.2 the 320 x 256
    // form takes M = 2048, N = 6144, K = 4096: 54.6 against 56.8 us for 128 x 256; M = 1536,
    // N = 10240, K = 2560: 40.0 against 44.2; M = 2048, N = 10240: 45.3 against 47.6; and
    // ties 160 x 256 at M = 2048, N = 24576, K = 4096, 173.9 against 172.5 us.)
    // The 256 x 256 ping-pong form (18): 1.1, where its rounds fit better than the 320-wide
    // one's (M = 2048, N = 24576, K = 4096: 163.5 against 185.7 us for 160 x 256; M = 2048,
    // N = 6144, K = 4096: 52.7 against 58.4; M = 3072, N = 10240, K = 2560: 76.1 against 81.4;
    // every other shape of that sweep keeps its choice).
    const int64_t t13 = (int64_t)((p.M + 255) / 256) * ((p.N + 319) / 320);
    const int64_t t18 = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256);
    const int64_t t6 = (int64_t)((p.M + 255) / 256) * ((p.N + 159) / 160);
    const int64_t t7 = (int64_t)((p.M + 255) / 256) * ((p.N + 127) / 128);
    const int64_t t12 = (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
    const double c13 = (double)((t13 + cus - 1) / cus) * 320 * 256 / 1.2;
    const double c18 = (double)((t18 + cus - 1) / cus) * 256 * 256 / 1.1;
    const double c6 = (double)((t6 + cus - 1) / cus) * 160 * 256 / 1.0;
    const double c7 = (double)((t7 + cus - 1) / cus) * 128 * 256 / 0.9;
    const double c12 = (double)((t12 + cus - 1) / cus) * 64 * 64 / 0.4;
    // (the 320 x 256 ping-pong form with two stages of 128-value K-tiles, 16, against the same
    // tile with four 64-value stages, 13, which K % 128 == 0 always allows here: 91.4 against
    // 94.0 us at M = 4096, N = 10240, K = 2560; 148 against 150.5 us at M = 8192, N = 2560,
    // K = 10240; 177 against 183 us at M = 8192, N = 10240, K = 2560; whole 128-byte row
    // segments per DMA halve the L2 requests, and the chip holds a 6 % higher clock)
    if (c12 < c6 && c12 < c7 && c12 < c13 && c12 < c18) return 12;
    // (19 is 16 with each stage's DMA split over two memory phases of each group, outputs
    // identical: M = 4096, N = 10240, K = 2560 82.4 against 83.0 us, M = 8192, N = 2560,
    // K = 10240 139.6 against 141.2, M = 4096, N = 2560, K = 10240 111.8 against 116.3)
    if (c13 < c6 && c13 < c7 && c13 <= c18) return 19;
    // (20 is 18 with the split DMA of 19, outputs identical: M = 2048, N = 24576, K = 4096
    // 152.0 against 153.9 us, M = 2048, N = 6144, K = 4096 45.1 against 46.0, M = 1536,
    // N = 10240, K = 2560 36.6 against 37.4)
    if (c18 < c6 && c18 < c7) return 20;
    return c6 <= c7 ? 6 : 7;
}

// Tile configurations with a split-K form: per-channel 7, 12, 14 (gemm_ms_kernel), per-group
// 11 and 12 (gemm_mg_kernel).
bool split_config(const GemmProblem &p, int cfg) {
    if (p.gs > 0 && p.out != OUT_I32) return cfg == 11 || cfg == 12;
    return p.wkind == W_INT8 && (cfg == 7 || cfg == 12 || cfg == 14);
}

// Time model of the slice kernels, fitted to launches on MI355X (N = 2560 .. 10240,
// K = 2560 .. 12288, M = 32 .. 4096, every slice count up to 32; the chosen plan is within
// 20 % of the fastest measured one on every shape). A launch is bound either by its rounds
// of workgroups, each `fill_us + kt_us` per K-tile, or by the operand bytes all workgroups
// fetch into LDS over `fetch_tbs`; a split adds the finish pass and the partial results'
// traffic (written once, read once).
struct SplitCost {
    int bn, bm;
    int per_cu;        // workgroups that fit one CU (LDS)
    double fill_us;    // per workgroup: first stages' latency and the epilogue
    double kt_us;      // per 128-value K-tile
    double fetch_tbs;  // operand fetch rate of the whole chip, TB/s
};

SplitCost split_cost(const GemmProblem &p, int cfg) {
    const bool grouped = p.gs > 0 && p.out != OUT_I32, w4 = grouped && p.wkind == W_INT4;
    switch (cfg) {
        case 7: return {128, 256, 1, 1.81, 0.732, 14.4};
        case 14: return {128, 128, 1, 1.48, 0.565, 13.4};
        case 11: return w4 ? SplitCost{128, 256, 1, 0.77, 1.795, 6.6} : SplitCost{128, 256, 1, 1.04, 1.652, 9.6};
        default:
            if (!grouped) return {64, 64, 2, 0.96, 0.315, 20.7};
            return w4 ? SplitCost{64, 64, 2, 0.0, 0.685, 12.6} : SplitCost{64, 64, 2, 0.18, 0.798, 10.5};
    }
}

double split_time(const GemmProblem &p, int cfg, int slices) {
    const SplitCost c = split_cost(p, cfg);
    const int64_t units = (int64_t)((p.M + c.bm - 1) / c.bm) * ((p.N + c.bn - 1) / c.bn) * slices;
    const int64_t slots = (int64_t)num_cus() * c.per_cu;
    const int kt = (p.K / 128 + slices - 1) / slices;
    const double rounds = (double)((units + slots - 1) / slots) * (c.fill_us + c.kt_us * kt);
    const double fetch = (double)units * kt * (c.bn + c.bm) * 128 / (c.fetch_tbs * 1e6);
    double t = rounds > fetch ? rounds : fetch;
    if (slices > 1) t += 7.5 + 2.0 * slices * p.M * p.N * 4 / 6.15e6;  // finish; partials at 6.15 TB/s
    return t;
}

}  // namespace

int gemm_num_configs() { return kNumConfigs; }

SplitPlan splitk_plan(const GemmProblem &p, int force_cfg, int force_slices) {
    const SplitPlan none{-1, 1};
    // M <= 16 runs the weight-streaming GEMV, whose workgroups already cover the chip
    if (p.M <= 16 || p.N < 16 || p.K % 128 != 0) return none;
    const bool grouped = p.gs > 0 && p.out != OUT_I32;
    if (!grouped && p.wkind != W_INT8) return none;
    const int KTT = p.K / 128;
    if (KTT < 2) return none;
    if (force_cfg >= 0 && !split_config(p, force_cfg)) return none;
    if (force_slices == 1) return none;
    const int smax = force_slices > 1 ? min(force_slices, KTT) : min(KTT, 32);
    const int smin = force_slices > 1 ? smax : 1;
    static const int cands[] = {7, 12, 14, 11};
    SplitPlan best = none;
    double best_t = 0, single_t = 0;
    for (int cfg : cands) {
        if (!split_config(p, cfg) || (force_cfg >= 0 && cfg != force_cfg)) continue;
        const double t1 = split_time(p, cfg, 1);
        if (single_t == 0 || t1 < single_t) single_t = t1;
        for (int sl = smin; sl <= smax; ++sl) {
            const double t = split_time(p, cfg, sl);
            if (best.cfg < 0 || t < best_t) {
                best = {cfg, sl};
                best_t = t;
            }
        }
    }
    if (best.cfg < 0 || best.slices == 1) return none;
    // automatic: split only with a 10 % predicted gain over the best single pass modelled
    // (the per-channel single pass may also take tiles outside the model, 320 x 256 or
    // 160 x 256, which do better where the output has enough tiles)
    if (force_slices < 0 && best_t >= 0.9 * single_t) return none;
    return best;
}

int64_t splitk_workspace_bytes(const GemmProblem &p, const SplitPlan &plan) {
    return plan.slices > 1 ? (int64_t)plan.slices * p.M * p.N * 4 : 0;
}

// Scratch of the allocation-free split-K call (w8a8_gemm_splitk_noalloc): the slices'
// partial results, for callers that cannot allocate device memory. Each device that runs
// the library holds its own copy of this array, at its own address, until the process
// ends. Host code never passes the array's name to a kernel (on the host that name is a
// stand-in, not a device address): it takes the address per device from
// hipGetSymbolAddress, once, with that device current.
static __device__ __align__(256) int8_t scratch[kSplitScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t splitk_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);  // same value from any racing thread
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_gemm_splitk(GemmProblem p, const SplitPlan &plan, hipStream_t stream) {
    if (plan.slices < 2 || plan.slices > p.K / 128 || p.ws == nullptr || !split_config(p, plan.cfg))
        return hipErrorInvalidValue;
    p.ksplit = plan.slices;
    const bool grouped = p.gs > 0 && p.out != OUT_I32;
    const int gm = kConfigs[plan.cfg].group_m;
    hipError_t e;
    if (grouped) {
        e = dispatch_mg<true>(p, plan.cfg == 12, gm, stream);
    } else {
        switch (plan.cfg) {
            case 7: e = launch_ms<128, 256, 3, 2, 4, true>(p, gm, stream); break;
            case 14: e = launch_ms<128, 128, 4, 2, 2, true>(p, gm, stream); break;
            default: e = launch_ms<64, 64, 4, 2, 2, true>(p, gm, stream); break;
        }
    }
    if (e != hipSuccess) return e;
    const int64_t quads = (int64_t)p.M * p.N / 4;
    const int blocks = (int)min((quads + 255) / 256, (int64_t)num_cus() * 8);
    if (grouped)
        hipLaunchKernelGGL(splitk_finish_kernel<true>, dim3(blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(splitk_finish_kernel<false>, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_linear_small(const GemmProblem &p, hipStream_t stream) {
    if (p.x == nullptr || p.M < 1 || p.M > 16 || p.out == OUT_I32) return hipErrorNotSupported;
    return p.x_bf16 ? linear_small_fq<2>(p, stream) : linear_small_fq<1>(p, stream);
}

hipError_t launch_gemm(const GemmProblem &p, int force_cfg, hipStream_t stream) {
    int id = (force_cfg >= 0 && force_cfg < kNumConfigs) ? force_cfg : choose_config(p);
    if (id == 10) {
        if (p.M <= 16) return dispatch_gemv(p, stream);
        id = 4;
    }
    const bool grouped = p.gs > 0 && p.out != OUT_I32;
    if ((grouped || mg_per_channel(p)) && (id == 11 || id == 12) && p.K % 128 == 0)
        return dispatch_mg(p, id == 12, kConfigs[id].group_m, stream);
    // (int4 with the four-part epilogue: M=4096 N=10240 K=2560 91.1 against 91.7 us, M=8192
    // 178.1 against 179.7, M=2048 47.8 against 48.3; identical outputs)
    if (mg_per_channel(p) && id == 17) return launch_pp<320, 256, 2, 128, W_INT4, 0, 4>(p, kConfigs[17].group_m, stream);
    if (id == 17) id = 16;
    if (grouped) {
        if (id != 4) id = 0;
        const int gm = kConfigs[id].group_m;
        if (id == 4) return launch_grouped<64, 64, 2, 2>(p, gm, stream);
        return launch_grouped<128, 128, 2, 2>(p, gm, stream);
    }
    const int gm = kConfigs[id].group_m;
    const bool dma_ok = p.K % (id == 13 ? 64 : 128) == 0 && p.wkind == W_INT8;
    if (id >= 5 && !dma_ok) id = 1;
    switch (id) {
        case 11: return launch_ms<128, 256, 3, 2, 4>(p, gm, stream);
        case 12: return launch_ms<64, 64, 4, 2, 2>(p, gm, stream);
        case 13: return launch_pp<320, 256, 4>(p, gm, stream);
        case 16: return launch_pp<320, 256, 2, 128>(p, gm, stream);
        case 18: return launch_pp<256, 256, 2, 128>(p, gm, stream);
        case 20:
            if ((int64_t)p.N * p.K < ((int64_t)1 << 32) && (int64_t)p.M * p.K < ((int64_t)1 << 32))
                return launch_pp<256, 256, 2, 128, W_INT8, 4 * 16 + 4, 4>(p, gm, stream);
            return launch_pp<256, 256, 2, 128>(p, gm, stream);
        case 19:
            // 32-bit DMA offsets within each operand, else the same tile as 16
            if ((int64_t)p.N * p.K < ((int64_t)1 << 32) && (int64_t)p.M * p.K < ((int64_t)1 << 32))
                return launch_pp<320, 256, 2, 128, W_INT8, 5 * 16 + 5, 4>(p, gm, stream);
            return launch_pp<320, 256, 2, 128>(p, gm, stream);
        case 14: return launch_ms<128, 128, 4, 2, 2>(p, gm, stream);
        case 15: return launch_ms<64, 128, 6, 2, 4>(p, gm, stream);
        case 5: return launch_ms<256, 256, 2, 4, 2>(p, gm, stream);
        case 6: return launch_ms<160, 256, 3, 2, 4>(p, gm, stream);
        case 7: return launch_ms<128, 256, 3, 2, 4>(p, gm, stream);
        case 8: return launch_xd<1>(p, gm, stream);
        case 9: return launch_xd<2>(p, gm, stream);
        case 0: return launch_shape<128, 128, 2, 2>(p, gm, stream);
        case 1: return launch_shape<256, 256, 2, 4>(p, gm, stream);
        case 2: return launch_shape<256, 128, 2, 2>(p, gm, stream);
        case 3: return launch_shape<128, 256, 2, 2>(p, gm, stream);
        default: return launch_shape<64, 64, 2, 2>(p, gm, stream);
    }
}

}  // namespace w8a8
