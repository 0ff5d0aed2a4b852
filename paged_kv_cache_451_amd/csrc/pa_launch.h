// Host-side launchers of the libpa kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

// Key ranges per group of the shared-prefix pass of cascade decode.
constexpr int kMaxSharedSplits = 16;

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
  // Cascade decode: partials of the shared-prefix pass, one per (sequence,
  // query head), folded in by the merge pass (null: no shared prefix), and
  // the true lengths for the merge when seq_lens holds suffix lengths.
  // (at most kMaxSharedSplits key ranges)
  const float* shared_ml;  // [shared_splits][B][Hq][2]
  const float* shared_o;   // [shared_splits][B][Hq][D]
  int shared_splits;
  const int32_t* full_lens;
  // Merge pass (plain, or fused without a shared prefix): one workgroup per
  // (sequence, pair of query heads) instead of per (sequence, query head).
  bool merge_pairs;
  // Measurement hook: when set, the main kernel's dispatch records these
  // events at its own start and end (no extra packets on the stream).
  hipEvent_t ev_start;
  hipEvent_t ev_stop;
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

// Merge pass over sequences whose blocks were split across ranges; one
// wave per (sequence, query head), or per (sequence, pair of query heads)
// with a.merge_pairs.
// out_bf16 selects the output element type.
hipError_t launch_decode_merge(bool out_bf16, int head_size,
                               const DecodeArgs& a, hipStream_t stream);
// Merge pass of the fused step: every (sequence, query head) combines its
// partials with the appended token, and the token's K/V go to their slot.
// kv_bytes: element size of the pools (4 = f32, 2 = bf16, 1 = fp8 e4m3fn).
hipError_t launch_decode_merge_append(int kv_bytes, int head_size,
                                      const DecodeArgs& a,
                                      hipStream_t stream);
// Resident waves per compute unit of the fused merge pass with one query
// head per wave (0 on error).
int occupancy_decode_merge_append(int kv_bytes, int head_size);
// The same for the plain merge pass.
int occupancy_decode_merge(bool out_bf16, int head_size);

// Byte copy of new tokens' K/V rows into pool slots: append_workgroups(...)
// workgroups of kAppendThreads threads (one per 16 tokens and KV head).
constexpr int kAppendThreads = 256;
int64_t append_workgroups(int64_t num_tokens, int num_kv_heads);
hipError_t launch_kv_append(int elem_bytes, const void* k_new,
                            const void* v_new, const int32_t* slots,
                            void* k_pool, void* v_pool, int num_tokens,
                            int num_kv_heads, int head_size, int num_blocks,
                            hipStream_t stream);

// Quantising append: bf16 rows into an fp8 e4m3fn pool (value / scale,
// nearest e4m3fn code, ties to even, saturating at 448).  Same grid as
// launch_kv_append.
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
  float c_log2;    // scale * log2(e) * k_scale
  float v_scale;   // fp8 pools: V dequantisation scale (else 1)
  int splits;      // shared-prefix pass: key ranges per group (else 1)
  int attn_grid;   // workgroups of the attention part (set by the launcher)
};
struct PrefillArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;  // shared-prefix pass: prefix blocks per group
  const int32_t* q_start;   // shared-prefix pass: group_start
  void* out;
  // shared-prefix pass only: the decode batch's lengths and the partials
  const int32_t* member_lens;  // [T]
  float* part_ml;              // [splits][T][Hq][2]
  float* part_o;               // [splits][T][Hq][D]
  int32_t* suffix_tables;      // [T][max_blocks]: the suffix view
  int32_t* suffix_lens;        // [T]
  PrefillSched s;
};
// Workgroups the prefill launch uses (an upper bound on the query tiles).
int64_t prefill_grid(int head_size, int64_t T, int G, int B, int Hkv);
// kv_fp8: the pools hold fp8 e4m3fn codes (else bf16).
hipError_t launch_prefill(int head_size, bool kv_fp8, const PrefillArgs& a,
                          hipStream_t stream);
// Shared-prefix pass of cascade decode (same kernel, s.B = groups, s.T =
// decode sequences), s.splits key ranges per group: partials
// [splits][T][Hq]; grid prefill_grid * splits, plus T workgroups that write
// each sequence's suffix view: suffix_tables[b][k] = block_tables[b][k +
// P_b] (-1 past the row), suffix_lens[b] = max(0, L_b - 16 P_b), where P_b
// is the prefix blocks of b's group (0 outside every group); sequences
// outside every group get empty partials (m = -inf, l = 0).
hipError_t launch_shared_prefix(int head_size, bool kv_fp8,
                                const PrefillArgs& a, hipStream_t stream);

// Copy-on-write block copy: K and V block src[i] -> dst[i] for every pair
// (block_bytes per pool block, a multiple of 16).  Pairs with an id outside
// [0, num_blocks) are skipped.
int copy_workgroups_per_pair(int block_bytes);
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                              const int32_t* dst, int num_pairs,
                              int block_bytes, int num_blocks,
                              hipStream_t stream);

}  // namespace pa
