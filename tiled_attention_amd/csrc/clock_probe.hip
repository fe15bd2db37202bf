// clock_probe.hip -- shader-clock probe for measurements.
//
// One wave counts shader-clock cycles (s_memtime) against the chip's fixed
// 100 MHz real-time counter (s_memrealtime) over a bounded interval. Enqueued
// between a workload's calls on their stream, it reads the clock the chip
// holds under that load, so a throughput can be set against the MFMA peak at
// that clock rather than at the 2.4 GHz peak clock.
#include "mxfa_internal.h"

namespace mxfa {
namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out, unsigned ticks) {
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1 = r0;
    // The real-time counter always advances; the iteration cap (far above
    // the <= 100,000 ticks the host allows) only bounds the loop by itself.
    for (int i = 0; i < (1 << 22) && r1 - r0 < ticks; ++i) {
        __builtin_amdgcn_s_sleep(1);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[0] = t1 - t0;
        out[1] = r1 - r0;
    }
}

}  // namespace

hipError_t launch_clock_probe(unsigned long long* out, unsigned ticks, hipStream_t stream) {
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, ticks);
    return hipGetLastError();
}

}  // namespace mxfa
