/*
 * pa_probe.h - measurement probe of the benchmark (libpa_probe.so), not
 * part of the paged-attention library.
 *
 * pa_probe_read_stream reads `bytes` of device memory at `buf` once with
 * 16-byte nontemporal loads and computes nothing: `workgroups` one-wave
 * workgroups each stream one contiguous chunk with 16 KiB of loads in
 * flight.  The rate it reaches is the practical HBM read ceiling that the
 * decode kernels' bandwidth is compared with (the published peak being the
 * other reference).
 *   buf         device memory, 16-byte aligned, caller-owned
 *   bytes       a multiple of 16
 *   sink        device memory of `workgroups` uint32 values; written only
 *               in the (practically impossible) case that the folded data
 *               equals 0x9E3779B9, so that the loads cannot be removed
 *   workgroups  >= 1
 *   stream      a hipStream_t (NULL = the default stream); asynchronous
 * Returns 0, -1 for a null pointer or no workgroups, -4 for misalignment,
 * -6 when the launch fails.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int pa_probe_read_stream(const void* buf, size_t bytes, uint32_t* sink,
                         int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
