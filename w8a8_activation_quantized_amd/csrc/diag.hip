// Measurement aid: the engine clock over an interval of stream time. Each workgroup of a
// probe launch records where it runs (the HW_ID register: compute unit, shader array and
// shader engine; the XCC_ID register: the XCD), the shader-clock counter (s_memtime, which
// counts at the current engine clock) and the constant 100 MHz counter (s_memrealtime).
// Two probes on one stream, before and after some work, give the mean engine clock over it
// on every compute unit that both probes visited: 100 MHz * (memtime difference) /
// (memrealtime difference), both counters read on the same compute unit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace w8a8 {
namespace {

// s_getreg_b32 operand: register id, bit offset 0, 32 bits
constexpr int kHwRegHwId = 4 | (31 << 11);
constexpr int kHwRegXccId = 20 | (31 << 11);

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t *out) {
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    const uint32_t hw = __builtin_amdgcn_s_getreg(kHwRegHwId);
    const uint32_t xcc = __builtin_amdgcn_s_getreg(kHwRegXccId);
    const int lane = threadIdx.x;
    // lanes 0..2 store (vector stores): location, shader clock, 100 MHz clock
    const uint64_t v = lane == 0 ? ((uint64_t)xcc << 32 | hw) : lane == 1 ? t : r;
    if (lane < 3) out[4 * blockIdx.x + lane] = v;
}

}  // namespace

hipError_t launch_clock_probe(uint64_t *out, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(64), 0, stream, out);
    return hipGetLastError();
}

}  // namespace w8a8
