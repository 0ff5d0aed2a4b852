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
 *
 * pa_probe_scatter_v_store performs only the V stores of a KV append: for
 * each of the n tokens and each KV head, the head_size isolated elements of
 * the token's V column in the [head_size][16] tile of its slot's block
 * (constant values), threads mapped as the append maps its V items (16
 * tokens and one KV head per workgroup, tokens fastest).  Its time, next to
 * the append's on the same slots, says what share of the append the V
 * stores' pattern costs by itself.
 *   v_pool      device memory [num_blocks][num_kv_heads][head_size][16] of
 *               elem_bytes (2: bf16, 1: fp8) elements, caller-owned; its
 *               contents are overwritten at the slots' positions
 *   slots       device int32 [n]; negative or out-of-pool slots are skipped
 *   head_size   64, 128 or 256;  elem_bytes 1 or 2
 * Returns 0, -1 for a bad pointer or size, -2 for an unsupported head size
 * or element size, -6 when the launch fails.
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
int pa_probe_scatter_v_store(void* v_pool, const int32_t* slots, int n,
                             int num_kv_heads, int head_size, int num_blocks,
                             int elem_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
