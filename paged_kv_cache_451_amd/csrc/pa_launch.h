// Host-side launchers of the libpa kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

// Everything one decode launch needs.
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  int32_t* prefix;  // [B+1] exclusive prefix of per-sequence block counts
  float* part_ml;   // [W][2][G][2]  (m in log2 units, l)
  float* part_o;    // [W][2][G][D]
  // Fused append (s.len_bias = 1): the step's new token per sequence, its
  // pool slot, and the partials of sequences one range finished entirely.
  const void* k_new;       // [B][Hkv][D] pool element type
  const void* v_new;       // [B][Hkv][D]
  const int32_t* slots;    // [B]
  void* k_pool_w;          // the pools again, written by the merge pass
  void* v_pool_w;
  float* direct_ml;        // [B][Hq][2]
  float* direct_o;         // [B][Hq][D]
  Sched s;
};

// Main pass: one 64-lane workgroup per (KV head, block range).
// Matrix-core kernel for bf16 q with bf16 (fp8 = false) or fp8 e4m3fn KV.
hipError_t launch_decode_mfma(bool fp8, int head_size, const DecodeArgs& a,
                              int num_workgroups, hipStream_t stream);
// Vector-ALU kernel for fp32 q and fp32 KV.
hipError_t launch_decode_valu(int head_size, const DecodeArgs& a,
                              int num_workgroups, hipStream_t stream);
// Resident workgroups per compute unit of the main kernels (0 on error).
int occupancy_decode_mfma(bool fp8, int head_size);
int occupancy_decode_valu(int head_size);

// Merge pass over sequences whose blocks were split across ranges;
// grid = B * Hq workgroups.  out_bf16 selects the output element type.
hipError_t launch_decode_merge(bool out_bf16, int head_size,
                               const DecodeArgs& a, hipStream_t stream);
// Merge pass of the fused step: every (sequence, query head) combines its
// partials with the appended token, and the token's K/V go to their slot.
// kv_bytes: element size of the pools (4 = f32, 2 = bf16, 1 = fp8 e4m3fn).
hipError_t launch_decode_merge_append(int kv_bytes, int head_size,
                                      const DecodeArgs& a,
                                      hipStream_t stream);

// Byte copy of new tokens' K/V rows into pool slots: num_tokens *
// append_workgroups_per_token(...) workgroups of kAppendThreads threads.
constexpr int kAppendThreads = 256;
int append_workgroups_per_token(int elem_bytes, int num_kv_heads,
                                int head_size);
hipError_t launch_kv_append(int elem_bytes, const void* k_new,
                            const void* v_new, const int32_t* slots,
                            void* k_pool, void* v_pool, int num_tokens,
                            int num_kv_heads, int head_size, int num_blocks,
                            hipStream_t stream);

// Quantising append: bf16 rows into an fp8 e4m3fn pool (value / scale,
// nearest e4m3fn code, ties to even, saturating at 448).  Same grid as
// launch_kv_append with 2-byte input elements.
hipError_t launch_kv_append_quant(const void* k_new, const void* v_new,
                                  const int32_t* slots, void* k_pool,
                                  void* v_pool, int num_tokens,
                                  int num_kv_heads, int head_size,
                                  int num_blocks, float k_scale,
                                  float v_scale, hipStream_t stream);

// Chunked prefill (prefill_mfma.hip): query row tiles of
// kPrefillWaves waves * 32 rows per workgroup.
constexpr int kPrefillWaves = 4;
struct PrefillSched {
  int B;           // sequences
  int Hq, Hkv, G;  // heads
  int max_blocks;  // row length of block_tables
  int NB;          // pool blocks
  int T;           // packed query rows (q_start[B])
  float c_log2;    // scale * log2(e)
};
struct PrefillArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* q_start;
  void* out;
  PrefillSched s;
};
// Workgroups the prefill launch uses (an upper bound on the query tiles).
int64_t prefill_grid(int head_size, int64_t T, int G, int B, int Hkv);
hipError_t launch_prefill(int head_size, const PrefillArgs& a,
                          hipStream_t stream);

// Copy-on-write block copy: K and V block src[i] -> dst[i] for every pair
// (block_bytes per pool block, a multiple of 16).  Pairs with an id outside
// [0, num_blocks) are skipped.
int copy_workgroups_per_pair(int block_bytes);
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                              const int32_t* dst, int num_pairs,
                              int block_bytes, int num_blocks,
                              hipStream_t stream);

}  // namespace pa
