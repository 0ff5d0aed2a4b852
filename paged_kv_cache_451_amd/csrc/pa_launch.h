// Host-side launchers of the libpa kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

// Everything one decode launch needs besides the split schedule.
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  void* out;
  float c_log2;   // scale * log2(e) * k_scale: scores in base-2 units
  float v_scale;  // applied to the output (1 for 16/32-bit pools)
  int Hq;
  int NB;
  SplitArgs s;
};

// Main pass: one 64-lane workgroup per (KV head, block range).
// Matrix-core kernel for bf16 q with bf16 (fp8 = false) or fp8 e4m3fn KV.
hipError_t launch_decode_mfma(bool fp8, int head_size, const DecodeArgs& a,
                              int num_workgroups, hipStream_t stream);
// Vector-ALU kernel for fp32 q and fp32 KV.
hipError_t launch_decode_valu(int head_size, const DecodeArgs& a,
                              int num_workgroups, hipStream_t stream);

// Merge pass over sequences whose blocks were split across ranges;
// grid = B * Hkv workgroups.  out_bf16 selects the output element type.
hipError_t launch_decode_merge(bool out_bf16, int head_size,
                               const DecodeArgs& a, hipStream_t stream);

// Byte copy of new tokens' K/V rows into pool slots.
hipError_t launch_kv_append(int elem_bytes, const void* k_new,
                            const void* v_new, const int32_t* slots,
                            void* k_pool, void* v_pool, int num_tokens,
                            int num_kv_heads, int head_size, int num_blocks,
                            hipStream_t stream);

}  // namespace pa
