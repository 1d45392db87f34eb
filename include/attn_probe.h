/*
 * attn_probe.h - shader-clock probe used by the benchmark (libattn_probe.so).
 * Measurement support only; not part of the attention library's ABI.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueues on `stream` (a hipStream_t) one wave per workgroup that measures the shader
 * clock over `ticks` ticks of the device's constant-rate real-time counter and writes
 * out[i] = shader cycles per real-time tick for workgroup i (0 if the counter did not
 * advance). Multiply by attn_probe_realtime_mhz() / 1000 for GHz.
 *   out:        device memory of the current device, `workgroups` floats, caller-owned
 *   workgroups: 1 .. 2^20; ticks: 1 .. 2^24 (the wait is also capped at 2^16 polls)
 * Returns 0, -1 (out is NULL), -2 (a count out of range) or -8 (launch failed).
 */
int attn_probe_clock(float* out, int workgroups, int ticks, void* stream);

/* Rate of the real-time counter of the current device in MHz (0.0 if unknown). */
double attn_probe_realtime_mhz(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
