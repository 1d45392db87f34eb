// Shader-clock probe for the benchmark (libattn_probe.so, declared in
// include/attn_probe.h). Not part of the attention library.
//
// Every wave reads the shader cycle counter (s_memtime) and the constant-rate real-time
// counter (s_memrealtime) twice, a fixed number of real-time ticks apart, and stores
// cycles per tick. Enqueued right behind a stream of attention launches it reports the
// clock the chip held under that load: the power controller changes the clock on a
// millisecond scale, far slower than the probe's tens of microseconds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_probe.h"

namespace {

__global__ __launch_bounds__(64) void attn_probe_clock_kernel(float* out, int ticks) {
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    uint64_t r1 = r0;
    // Bounded: at most 2^16 polls of about 64 cycles of sleep each.
    for (int it = 0; it < (1 << 16) && r1 - r0 < (uint64_t)ticks; ++it) {
        __builtin_amdgcn_s_sleep(1);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0)
        out[blockIdx.x] = r1 > r0 ? (float)(double)(c1 - c0) / (float)(double)(r1 - r0) : 0.f;
}

}  // namespace

extern "C" {

int attn_probe_clock(float* out, int workgroups, int ticks, void* stream) {
    if (!out) return -1;
    if (workgroups < 1 || workgroups > (1 << 20) || ticks < 1 || ticks > (1 << 24)) return -2;
    hipLaunchKernelGGL(attn_probe_clock_kernel, dim3((unsigned)workgroups), dim3(64), 0,
                       reinterpret_cast<hipStream_t>(stream), out, ticks);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

double attn_probe_realtime_mhz(void) {
    int dev = 0;
    int khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0.0;
    }
    return khz / 1000.0;
}

}  // extern "C"
