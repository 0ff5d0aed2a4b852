// Device-side helpers shared by the decode kernels of libpa.
//
// Work split ("split context"): for every KV head g, the flattened sequence
// of that head's work units over all sequences (sequence-major, U units in
// total) is cut into Wh equal contiguous ranges, one per 64-lane workgroup.
// A unit is 2^shift consecutive KV blocks of one sequence - the step of the
// main kernel's loop (4 blocks for the matrix-core kernel, which computes
// two 2-block pairs per iteration; 1 for the vector kernel) - and a
// sequence of n blocks has ceil(n / 2^shift) units, its last one possibly
// partial.  Range k covers units [floor(k*U/Wh), floor((k+1)*U/Wh)), so
// every range boundary falls on a loop step and ranges cost the same
// number of steps up to one, whatever the length mix.  A workgroup walks
// every sequence that overlaps its range; a sequence wholly inside the
// range is finished in place (its output row written directly), one that
// crosses a range boundary leaves a partial (running max m, sum l and
// unnormalised output o) that the merge kernel combines.  Each workgroup
// leaves at most two partials: slot 0 for the sequence that started before
// its range, slot 1 for the one that continues after it.
//
// Workgroup w handles KV head g = w % Hkv, range k = w / Hkv; consecutive
// workgroup ids are dealt round-robin to the 8 XCDs, so with Hkv = 8 every
// XCD streams a single KV head and its L2 keeps that head's shared blocks.
//
// Every pointer reaches the kernels as its own __restrict__ parameter: the
// kernels store only to out / prefix / partials, so the compiler may read
// block tables through the scalar cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;  // tokens per KV block
constexpr int kWave = 64;   // lanes per wavefront on gfx950

// Scalars of one decode launch.
struct Sched {
  int B;           // sequences
  int max_blocks;  // row length of block_tables
  int Hq;          // query heads
  int Hkv;         // KV heads
  int G;           // Hq / Hkv
  int Wh;          // ranges (workgroups) per KV head
  int NB;          // physical blocks in the pool
  float c_log2;    // scale * log2(e) * k_scale: scores in base-2 units
  float v_scale;   // applied to the output (1 for 16/32-bit pools)
  int len_bias;    // newest tokens per sequence that are not read from the
                   // pool (1 when the step's appended token is folded in by
                   // the merge pass, else 0)
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Tokens of a sequence of length L that are read from the pool: L minus the
// tokens supplied separately, clamped to the table row.
__device__ __forceinline__ int pool_len(int L, int bias, int max_blocks) {
  const int cap = max_blocks * kBlock;
  L -= bias;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Work units of a sequence of length L (before the bias): its blocks read
// from the pool, in steps of 2^shift blocks.
__device__ __forceinline__ int seq_units(int L, int bias, int max_blocks,
                                         int shift) {
  const int nb = (pool_len(L, bias, max_blocks) + kBlock - 1) / kBlock;
  return (nb + (1 << shift) - 1) >> shift;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int range_begin(int k, int U, int Wh) {
  return (int)(((int64_t)k * U) / Wh);
}

// Range index k holding block u (0 <= u < U).
__device__ __forceinline__ int range_of(int u, int U, int Wh) {
  return (int)((((int64_t)u + 1) * Wh + U - 1) / U) - 1;
}

__device__ __forceinline__ int readlane(int v, int l) {
  return __builtin_amdgcn_readlane(v, l);
}

// Total units U per head (the sum of seq_units); when `prefix` is non-null
// the exclusive prefix is stored for the merge kernel.
// `first` (optional) receives this lane's units of sequence `lane` (the
// first chunk of kWave sequences), so that a cursor over the same
// sequences need not load them again.
__device__ inline int total_units(const int32_t* __restrict__ seq_lens,
                                  int B, int max_blocks, int bias, int shift,
                                  int32_t* __restrict__ prefix,
                                  int* first = nullptr) {
  const int lane = lane_id();
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int b = c0 + lane;
    const int nb =
        b < B ? seq_units(seq_lens[b], bias, max_blocks, shift) : 0;
    if (first && c0 == 0) *first = nb;
    const int incl = wave_incl_scan(nb) + carry;
    if (prefix && b < B) prefix[b] = incl - nb;
    carry = readlane(incl, kWave - 1);
  }
  if (first && B <= 0) *first = 0;
  if (prefix && lane == 0) prefix[B] = carry;
  return carry;
}

// Calls seg(b, Sb, Sb1) for every sequence b (in order) whose unit span
// [Sb, Sb1) overlaps [u0, u1) and is non-empty.  All arguments are uniform.
template <typename Seg>
__device__ inline void for_each_segment(const int32_t* __restrict__ seq_lens,
                                        int B, int max_blocks, int bias,
                                        int shift, int u0, int u1, Seg&& seg) {
  const int lane = lane_id();
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int b = c0 + lane;
    const int nb =
        b < B ? seq_units(seq_lens[b], bias, max_blocks, shift) : 0;
    const int incl = wave_incl_scan(nb) + carry;
    const int excl = incl - nb;
    const int chunk_end = readlane(incl, kWave - 1);
    if (chunk_end > u0) {
      uint64_t mask = __ballot(nb > 0 && excl < u1 && incl > u0);
      while (mask) {
        const int i = __builtin_ctzll(mask);
        mask &= mask - 1;
        seg(c0 + i, readlane(excl, i), readlane(incl, i));
      }
    }
    if (chunk_end >= u1) break;
    carry = chunk_end;
  }
}

// The same walk as for_each_segment, one segment per call, so that a kernel
// can look one segment ahead.  All state is uniform.
struct SegCursor {
  const int32_t* __restrict__ seq_lens;
  int B, max_blocks, bias, shift, u0, u1;
  int c0;          // first sequence of the scanned chunk of kWave sequences
  int chunk_end;   // units before the next chunk
  int excl, incl;  // per lane: unit span of sequence c0 + lane
  uint64_t mask;   // lanes of the chunk still to visit
  bool last;       // no later chunk can overlap [u0, u1)

  // first: this lane's units of sequence `lane`, as total_units returns
  // them (the first chunk is then not loaded again)
  __device__ SegCursor(const int32_t* __restrict__ lens, int B_, int mb,
                       int bias_, int shift_, int u0_, int u1_, int first)
      : seq_lens(lens), B(B_), max_blocks(mb), bias(bias_), shift(shift_),
        u0(u0_), u1(u1_), c0(0), chunk_end(0) {
    scan_units(first);
  }

  __device__ void scan() {
    const int b = c0 + lane_id();
    scan_units(b < B ? seq_units(seq_lens[b], bias, max_blocks, shift) : 0);
  }

  __device__ void scan_units(int nb) {
    incl = wave_incl_scan(nb) + chunk_end;
    excl = incl - nb;
    chunk_end = readlane(incl, kWave - 1);
    const uint64_t m = __ballot(nb > 0 && excl < u1 && incl > u0);
    mask = chunk_end > u0 ? m : 0;
    last = chunk_end >= u1 || c0 + kWave >= B;
  }

  // Next sequence b whose non-empty span [Sb, Sb1) overlaps [u0, u1).
  __device__ bool next(int& b, int& Sb, int& Sb1) {
    while (!mask) {
      if (last) return false;
      c0 += kWave;
      scan();
    }
    const int i = __builtin_ctzll(mask);
    mask &= mask - 1;
    b = c0 + i;
    Sb = readlane(excl, i);
    Sb1 = readlane(incl, i);
    return true;
  }
};

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// max(v[l], v[l ^ 16]) and max(v[l], v[l ^ 32]) with the gfx950 row/half
// swap instructions (plain VALU, no LDS traffic).  Each swap exchanges one
// half of the lanes between its two operands; passing the value as both
// operands puts each lane's partner value in one of the two results.
__device__ __forceinline__ float max_xor16(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]),
               __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float max_xor32(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]),
               __builtin_bit_cast(float, (unsigned)r[1]));
}

}  // namespace pa
