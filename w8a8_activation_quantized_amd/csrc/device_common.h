// Device helpers shared by the kernel sources of libw8a8 (gfx950): vector types, the
// global -> LDS DMA forms, counted waits, the workgroup barrier and the output stores.
// Everything is file-local (anonymous namespace) in each source that includes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// fp32 -> fp16 bits, RNE, of an fp32 value that has been rounded to fp32 first. The empty
// asm pins the fp32 value in a register: without it the compiler may fold a preceding
// fp32 multiply and this conversion into one v_fma_mixlo_f16, which rounds the exact
// product once, straight to fp16, and differs from the two roundings at fp16 ties.
__device__ __forceinline__ uint32_t f16_bits(float f) {
    asm volatile("" : "+v"(f));
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Store four consecutive outputs y[m, n..n+3].
__device__ __forceinline__ void store4(void *y, int64_t off, int out, float v0, float v1, float v2,
                                       float v3) {
    if (out == OUT_F16) {
        uint2 w = make_uint2(f16_bits(v0) | (f16_bits(v1) << 16), f16_bits(v2) | (f16_bits(v3) << 16));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + off) = w;
    } else if (out == OUT_BF16) {
        uint2 w = make_uint2(bf16_rne(v0) | (bf16_rne(v1) << 16), bf16_rne(v2) | (bf16_rne(v3) << 16));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + off) = w;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(y) + off) = make_float4(v0, v1, v2, v3);
    }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

__device__ __forceinline__ void dma_16B(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds((gbl_void_t *)g, (lds_void_t *)l, 16, 0, 0);
}
// 4-byte form: lane i writes LDS bytes [4 i, 4 i + 4) of the block at l.
__device__ __forceinline__ void dma_4B(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds((gbl_void_t *)g, (lds_void_t *)l, 4, 0, 0);
}

// A 16-byte LDS read of data written by an earlier LDS DMA that the caller's own vmcnt wait
// has already retired, issued in inline asm and retired inside the same block. As an
// ordinary load the compiler cannot tell that region from the DMA targets still in flight
// and puts a wait for all of them in front of the read.
__device__ __forceinline__ float4 lds_read_f4_now(const float *p) {
    typedef float v4f_t __attribute__((ext_vector_type(4)));
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float *)p;
    v4f_t v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return make_float4(v[0], v[1], v[2], v[3]);
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding). The waits and
// the barrier are fenced with sched_barrier(0): the instruction scheduler otherwise moves
// MFMAs (which touch no memory) across them, so a wait meant to trail a run of MFMAs ends
// up ahead of it and exposes the latency it was placed to hide.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
    __builtin_amdgcn_sched_barrier(0);
}
// Workgroup barrier that the compiler may not move memory operations across. The
// s_barrier is written as asm, so the compiler adds no wait before it: this wave's LDS
// writes (and reads) are waited for here, else another wave may pass the barrier and
// read LDS that a write of this wave has not reached yet. DMA into LDS is counted by
// vmcnt and waited for separately.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace
}  // namespace w8a8
