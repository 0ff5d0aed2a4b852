// Paged chunked-prefill attention on gfx950 matrix cores (bf16 q; bf16 or
// fp8 e4m3fn KV).
//
// Sequence b holds L cached tokens, the last C of which are this chunk's;
// query row (token i, head n) of the chunk attends to the keys at positions
// t <= p = L - C + i (causal within the chunk).  Queries are packed over
// the batch: rows q_start[b] .. q_start[b+1] of q.
//
// Work split.  A sequence's query rows are ordered token-major, head-minor
// (row = i * G + n), so a tile of COLS consecutive rows holds consecutive
// tokens and all G heads that share KV head g.  One workgroup of kPfWaves
// waves takes one (tile, KV head); each wave owns 32 rows.  Tiles differ in
// cost (the keys they attend grow along the chunk and with the context), so
// workgroups take them longest first: workgroup rank r picks the r-th tile
// in order of decreasing step count (ties in (sequence, tile) order), found
// by a search over step counts that every wave runs on the lengths alone.
//
// Products, per 64-key step, on v_mfma_f32_32x32x16_bf16:
//
//   S^T[32 keys][32 rows] = K[32 keys][D] . Q^T[D][32 rows]      (x2)
//   O^T[32 d][32 rows]   += V^T[32 d][16 keys] . P^T[16 keys][32 rows]
//
// Q^T stays in registers for the whole tile.  The K rows of each 32-key
// half are stored in LDS with bits 2 and 3 of the key index swapped, so
// that the S^T accumulator elements 8c .. 8c+7 of lane (n, h) are the
// scores of keys 16c + 8h .. 16c + 8h + 7 of that half: exactly lane
// (n, h)'s slots of the P^T operand of the PV product.  P never moves
// between lanes.
//
// K/V go through LDS: the workgroup copies the four 16-token K tiles
// ([16][D] each) and V tiles ([D][16] each) of KV head g of a step into
// one of two K and one of two V buffers while the waves compute on the
// others (K two steps ahead, V one step ahead).  The copies go from
// the pool straight into LDS (no registers on the way), wave w copying
// block w of the step; unpadded rows with XOR-swizzled 16-byte chunks keep
// the operand reads free of bank conflicts.  An fp8 e4m3fn pool takes a
// different road into the same LDS layout: each lane loads 16-byte pieces
// of its wave's tiles into registers, widens them exactly to bf16 and
// writes them to LDS before the step's barrier (k_scale is folded into the
// score scale, v_scale into the output).  Keys at or past the sequence
// end, or in blocks with an out-of-range id, get a -inf score, and their V
// is zeroed in LDS after the copy lands (a masked probability times them
// must be 0 even where the slot holds NaN).  The causal mask is applied only
// on steps that reach past the smallest query position of the wave.
//
// Each wave is software-pipelined: while the matrix cores compute step
// s + 1's scores, the vector unit turns step s's scores into probabilities;
// while they accumulate step s's PV products, it takes step s + 1's row
// maxima.  A scheduling fence after every product keeps the two kinds of
// work interleaved in the instruction stream.
//
// The same kernel runs the shared-prefix pass of cascade decode
// (kShared): a "chunk" is then a group of consecutive decode sequences that
// share their first P table entries, its query rows are the group's decode
// queries, every row attends to all 16 P prefix keys before its own newest
// token (no causal order inside the group), and the result is left as fp32
// partials (running max, sum, unnormalised output) for the decode merge.
//
// Online softmax in base 2 with a lazily updated running max: the
// accumulator is rescaled only when some row's max has grown by more than
// 8 (log2 units) since the last rescale, so probabilities stay below 256.
// The result is the same in exact arithmetic; only rounding differs.
#include <math.h>

#include <type_traits>

#include "pa_launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Fourth word of a raw buffer descriptor on gfx9-class GPUs: 32-bit data
// format, no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

constexpr int kPfWaves = kPrefillWaves;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kRows = 32;                // query rows per wave
constexpr int kCols = kPfWaves * kRows;  // query rows per workgroup
constexpr int kKeys = 64;                // keys per step: four blocks
constexpr float kLazy = 8.0f;            // rescale threshold (log2 units)

// LDS of one workgroup: two K buffers then two V buffers.  A K buffer holds
// a step's 64 key rows of D values (row k_lds_row(key)), a V buffer the
// step's four [D][16] V tiles back to back.  Rows are not padded: the
// 16-byte chunks of K row r sit at position chunk ^ kswz(r), those of V row
// d at half ^ ((d >> 3) & 1), which spreads every 16-lane group of operand
// reads over all banks.
template <int D>
struct PfLds {
  static constexpr int KRow = D * 2;           // bytes per K row
  static constexpr int KBytes = kKeys * KRow;  // one K buffer
  static constexpr int VTile = kBlock * D * 2;  // one block's V tile
  static constexpr int VBytes = 4 * VTile;      // one V buffer
  static constexpr int V0 = 2 * KBytes;         // V buffers follow both K
  static constexpr int Total = 2 * KBytes + 2 * VBytes;
};

// Chunk swizzle of K row r (16 chunks of 16 bytes per row at D = 128, 8 at
// D = 64).
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// One tile of `bytes` bytes at `tile` (uniform) into LDS: instruction m
// copies 16 bytes per lane from tile + src[m] to dst + 1024 m + 16 lane.
// The loads go through a buffer descriptor of the tile, so addresses are
// formed in scalar registers and no load can leave the tile.
template <int N>
__device__ __forceinline__ void copy_tile_to_lds(const char* tile, int bytes,
                                                 const uint32_t (&src)[N],
                                                 uint8_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(tile), 0, bytes, kBufferWord3);
#pragma unroll
  for (int m = 0; m < N; ++m)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 1024 * m),
                                             16, src[m], 0, 0, 0);
#endif
}

// Waits for every outstanding memory operation of the wave.
__device__ __forceinline__ void wait_all_memory() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0);
#endif
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keeps the 16-bit elements e of w (8 of them) with e < hi.
__device__ __forceinline__ u32x4 keep_below(u32x4 w, int hi) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned m = (2 * k < hi ? 0x0000FFFFu : 0u) |
                       (2 * k + 1 < hi ? 0xFFFF0000u : 0u);
    w[k] &= m;
  }
  return w;
}

// LDS row of key k of a step: bits 2 and 3 swapped within each 32-key half.
__device__ __forceinline__ int k_lds_row(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Clamped chunk of sequence b: rows [qs, qs + C) of q, L cached tokens.
struct Chunk {
  int qs, C, L;
};

// In the shared-prefix pass `seq_lens` holds each group's prefix blocks.
template <bool kShared>
__device__ __forceinline__ Chunk chunk_of(const int32_t* __restrict__ q_start,
                                          const int32_t* __restrict__ seq_lens,
                                          int b, const PrefillSched& sc) {
  int lo = q_start[b], hi = q_start[b + 1];
  lo = lo < 0 ? 0 : (lo > sc.T ? sc.T : lo);
  hi = hi < lo ? lo : (hi > sc.T ? sc.T : hi);
  int L;
  if (kShared) {
    const int p = seq_lens[b];
    L = (p < 0 ? 0 : (p > sc.max_blocks ? sc.max_blocks : p)) * kBlock;
  } else {
    const int cap = sc.max_blocks * kBlock;
    L = seq_lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
  }
  return Chunk{lo, hi - lo, L};
}

// Tiles of a chunk, and how many of them take at least W steps.  Tile t's
// last row is min(C*G, (t+1)*COLS) - 1, its largest query position
// L - C + that / G, and it takes ceil((position + 1) / 64) steps (0 when the
// position is negative).  The step count does not decrease along t, so the
// tiles taking >= W steps are a suffix.  In the shared-prefix pass every
// tile of a group takes ceil(L / 64) steps.
__device__ __forceinline__ int tiles_of(const Chunk& c, int G) {
  return (c.C * G + kCols - 1) / kCols;
}

template <bool kShared>
__device__ __forceinline__ int tiles_at_least(const Chunk& c, int G, int W) {
  const int nt = tiles_of(c, G);
  if (W <= 0) return nt;
  if (kShared) return (c.L + kKeys - 1) / kKeys >= W ? nt : 0;
  // need position >= (W - 1) * 64, i.e. last row / G >= Y
  const int Y = (W - 1) * kKeys - (c.L - c.C);
  if (Y < 0) return nt;
  if (Y >= c.C) return 0;
  // smallest t with min(C*G, (t+1)*COLS) >= Y*G + 1
  const int t_min = (Y * G + 1 + kCols - 1) / kCols - 1;
  return nt - (t_min < 0 ? 0 : t_min);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Total over all sequences of tiles_at_least(W).
template <bool kShared>
__device__ __forceinline__ int count_at_least(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ seq_lens,
    const PrefillSched& sc, int W) {
  const int lane = lane_id();
  int n = 0;
  for (int c0 = 0; c0 < sc.B; c0 += kWave) {
    const int b = c0 + lane;
    if (b < sc.B)
      n += tiles_at_least<kShared>(
          chunk_of<kShared>(q_start, seq_lens, b, sc), sc.G, W);
  }
  return wave_sum(n);
}

// The r-th tile in order of decreasing step count: sequence b and tile t, or
// b = -1 when r is past the last tile.  All arguments and results uniform.
template <bool kShared>
__device__ void tile_of_rank(const int32_t* __restrict__ q_start,
                             const int32_t* __restrict__ seq_lens,
                             const PrefillSched& sc, int r, int* b_out,
                             int* t_out) {
  *b_out = -1;
  *t_out = 0;
  if (sc.B <= kWave) {
    // Up to one sequence per lane: the sequences' chunks are loaded once
    // and every count of the search below runs on registers (with loads in
    // each count, the search's dependent round trips cost a few
    // microseconds per tile).
    const int lane = lane_id();
    const bool live = lane < sc.B;
    const Chunk c =
        live ? chunk_of<kShared>(q_start, seq_lens, lane, sc) : Chunk{0, 0, 0};
    auto count = [&](int W) {
      return wave_sum(live ? tiles_at_least<kShared>(c, sc.G, W) : 0);
    };
    if (r >= count(0)) return;
    int lo = 0, hi = (sc.max_blocks * kBlock + kKeys - 1) / kKeys + 1;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (count(mid) > r)
        lo = mid;
      else
        hi = mid;
    }
    const int W = lo;
    const int k = r - count(W + 1);
    int eq = 0, first = 0;
    if (live) {
      const int ge = tiles_at_least<kShared>(c, sc.G, W);
      eq = ge - tiles_at_least<kShared>(c, sc.G, W + 1);
      first = tiles_of(c, sc.G) - ge;
    }
    const int incl = wave_incl_scan(eq);
    const uint64_t hit = __ballot(eq > 0 && k < incl && k >= incl - eq);
    if (hit) {
      const int i = __builtin_ctzll(hit);
      *b_out = i;
      *t_out = readlane(first, i) + k - (readlane(incl, i) - readlane(eq, i));
    }
    return;
  }
  if (r >= count_at_least<kShared>(q_start, seq_lens, sc, 0)) return;
  // largest W with count_at_least(W) > r
  int lo = 0, hi = (sc.max_blocks * kBlock + kKeys - 1) / kKeys + 1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (count_at_least<kShared>(q_start, seq_lens, sc, mid) > r)
      lo = mid;
    else
      hi = mid;
  }
  const int W = lo;
  const int k = r - count_at_least<kShared>(q_start, seq_lens, sc, W + 1);
  // the k-th tile, in (sequence, tile) order, of those taking exactly W
  const int lane = lane_id();
  int carry = 0;
  for (int c0 = 0; c0 < sc.B; c0 += kWave) {
    const int b = c0 + lane;
    int eq = 0, first = 0;
    if (b < sc.B) {
      const Chunk c = chunk_of<kShared>(q_start, seq_lens, b, sc);
      const int ge = tiles_at_least<kShared>(c, sc.G, W);
      eq = ge - tiles_at_least<kShared>(c, sc.G, W + 1);
      first = tiles_of(c, sc.G) - ge;
    }
    const int incl = wave_incl_scan(eq) + carry;
    const uint64_t hit = __ballot(eq > 0 && k < incl && k >= incl - eq);
    if (hit) {
      const int i = __builtin_ctzll(hit);
      *b_out = c0 + i;
      *t_out = readlane(first, i) + k - (readlane(incl, i) - readlane(eq, i));
      return;
    }
    carry = readlane(incl, kWave - 1);
  }
}

__device__ __forceinline__ int clamp_to(int v, int hi) {
  return v < 0 ? 0 : (v > hi ? hi : v);
}

// Group j of sequence b (group_start[j] <= b < group_start[j + 1], values
// clamped to [0, B]), or -1.  A binary search over non-decreasing starts.
__device__ int group_of(const int32_t* __restrict__ gs, int ng, int B, int b) {
  int lo = 0, hi = ng - 1, j = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if (clamp_to(gs[mid], B) <= b) {
      j = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  if (j >= 0 && b >= clamp_to(gs[j + 1], B)) j = -1;
  return j;
}

// Suffix view of sequence b of a cascade batch, for the decode main pass:
// its table shifted left by its group's prefix blocks P (-1 past the row),
// its length less 16 P; a sequence outside every group gets empty
// shared-prefix partials (m = -inf, l = 0) in every key range.
__device__ void suffix_row(int b, const int32_t* __restrict__ tables,
                           const int32_t* __restrict__ lens,
                           const int32_t* __restrict__ gs,
                           const int32_t* __restrict__ gp,
                           const PrefillSched& sc,
                           int32_t* __restrict__ suffix_tables,
                           int32_t* __restrict__ suffix_lens,
                           float* __restrict__ part_ml) {
  const int j = group_of(gs, sc.B, sc.T, b);
  const int P = j >= 0 ? clamp_to(gp[j], sc.max_blocks) : 0;
  const int32_t* row = tables + (size_t)b * sc.max_blocks;
  int32_t* srow = suffix_tables + (size_t)b * sc.max_blocks;
  for (int k = threadIdx.x; k < sc.max_blocks; k += kPfThreads)
    srow[k] = k + P < sc.max_blocks ? row[k + P] : -1;
  if (threadIdx.x == 0) {
    const int L = clamp_to(lens[b], sc.max_blocks * kBlock);
    const int Ls = L - P * kBlock;
    suffix_lens[b] = Ls > 0 ? Ls : 0;
  }
  if (j < 0) {
    for (int i = threadIdx.x; i < sc.Hq * sc.splits; i += kPfThreads) {
      const int k = i / sc.Hq, hh = i - k * sc.Hq;
      const size_t r = ((size_t)k * sc.T + b) * sc.Hq + hh;
      part_ml[r * 2] = -INFINITY;
      part_ml[r * 2 + 1] = 0.f;
    }
  }
}

template <int D, bool kShared, bool kFP8>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_mfma_kernel(
    const __bf16* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_start, __bf16* __restrict__ out,
    const int32_t* __restrict__ member_lens, float* __restrict__ part_ml,
    float* __restrict__ part_o, int32_t* __restrict__ suffix_tables,
    int32_t* __restrict__ suffix_lens, PrefillSched sc) {
  typedef PfLds<D> Lay;
  constexpr int NK = D / 16;                  // 16-wide d chunks of Q^T
  constexpr int NX = D / 32;                  // 32-row d tiles of O^T
  __shared__ __attribute__((aligned(16))) uint8_t lds[Lay::Total];

  // the shared-prefix launch ends with one workgroup per decode sequence
  // that writes the sequence's suffix view
  if (kShared && (int)blockIdx.x >= sc.attn_grid) {
    suffix_row((int)blockIdx.x - sc.attn_grid, block_tables, member_lens,
               q_start, seq_lens, sc, suffix_tables, suffix_lens, part_ml);
    return;
  }
  const int tid = threadIdx.x;
  __builtin_assume(tid < kPfThreads);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n32 = lane & 31;
  const int h = lane >> 5;
  const int g = blockIdx.x % sc.Hkv;
  const int G = sc.G;

  // the shared-prefix pass also splits each group's keys into sc.splits
  // ranges (adjacent workgroup ranks), so that few groups still fill the
  // chip; each range leaves its own partial
  const int r2 = blockIdx.x / sc.Hkv;
  const int split = kShared ? r2 % sc.splits : 0;
  int b, t_in_b;
  tile_of_rank<kShared>(q_start, seq_lens, sc, kShared ? r2 / sc.splits : r2,
                        &b, &t_in_b);
  b = __builtin_amdgcn_readfirstlane(b);
  t_in_b = __builtin_amdgcn_readfirstlane(t_in_b);
  if (b < 0) return;

  const Chunk ck = chunk_of<kShared>(q_start, seq_lens, b, sc);
  const int qs = ck.qs, C = ck.C;
  // keys the pass may read: the chunk's context; in the shared-prefix pass
  // the prefix, cut at the first member's tokens before its newest (the
  // rows it reads through), so that no unwritten slot enters a product
  int L = ck.L;
  if (kShared) {
    const int lf = member_lens[qs] - 1;
    L = lf < 0 ? 0 : (lf < L ? lf : L);
  }
  const int rows_b = C * G;
  const int row0 = t_in_b * kCols;
  const int nblk = (L + kBlock - 1) / kBlock;

  // this lane's row: row0 + 32 * wave + n32
  const int row = row0 + kRows * wave + n32;
  const bool row_ok = row < rows_b;
  const int ti = row_ok ? row / G : 0;
  const int hn = row_ok ? row - ti * G : 0;
  // largest key position the row attends: causal within a prefill chunk;
  // in the shared-prefix pass every prefix key before the sequence's newest
  // token (which the merge adds)
  int pos;
  if (kShared) {
    const int lm = member_lens[qs + ti] - 1;  // keys before the newest
    pos = row_ok ? (lm < L ? lm : L) - 1 : -1;
  } else {
    pos = row_ok ? L - C + ti : -1;
  }
  bf16x8 qb[NK];
  {
    const __bf16* qrow =
        q + ((size_t)(qs + ti) * sc.Hq + (size_t)g * G + hn) * D + 8 * h;
    // loaded unconditionally (a row past the chunk reads the chunk's first
    // row) and zeroed after: loads under a branch leave the compiler's wait
    // counts unsure at the loop head
#pragma unroll
    for (int c = 0; c < NK; ++c) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * c);
      const bf16x8 z = {};
      qb[c] = row_ok ? v : z;
    }
  }
  const int last_row = (rows_b < row0 + kCols ? rows_b : row0 + kCols) - 1;
  int wp_min, kend;  // smallest position of the wave; keys needed
  if (kShared) {
    int v = row_ok ? pos : INT32_MAX;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_xor(v, o, kWave);
      v = t < v ? t : v;
    }
    wp_min = v;
    kend = L;
  } else {
    const int p_max = L - C + last_row / G;  // largest query position
    wp_min = L - C + (row0 + kRows * wave) / G;
    kend = p_max + 1 < L ? p_max + 1 : L;
  }
  const int nsteps = kend > 0 ? (kend + kKeys - 1) / kKeys : 0;
  // steps [s_begin, s_end) of this workgroup
  int s_begin = 0, s_end = nsteps;
  if (kShared) {
    const int per = (nsteps + sc.splits - 1) / sc.splits;
    s_begin = split * per < nsteps ? split * per : nsteps;
    s_end = s_begin + per < nsteps ? s_begin + per : nsteps;
  }

  f32x16 acc[NX];
#pragma unroll
  for (int X = 0; X < NX; ++X)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[X][i] = 0.f;
  float m_run = -INFINITY, lsum = 0.f;

  // the group's prefix is read through its first member's table row
  const int32_t* trow =
      block_tables + (size_t)(kShared ? qs : b) * sc.max_blocks;

  // Block ids: lane u % 4 holds the entry of block 4 s + u % 4 of a step.
  // They are loaded three steps ahead, so the K/V loads never wait on them.
  auto table_entry = [&](int s) -> int {
    const int blk = 4 * s + (lane & 3);
    return trow[blk < nblk ? blk : (nblk > 0 ? nblk - 1 : 0)];
  };

  // Copies go straight from the pool into LDS (buffer_load_dwordx4 ... lds:
  // lane l of a wave instruction fills bytes 16 l .. 16 l + 15 of a 1 KiB
  // LDS span, from any offset it names inside the tile).  Wave w copies
  // block w of each step: its K tile as IPT instructions of RPI rows each,
  // and its V tile as IPT instructions of 32 d rows each.
  constexpr int CPR = D / 8;             // 16-byte chunks per K row
  constexpr int RPI = kWave / CPR;       // K rows per instruction
  constexpr int IPT = kBlock / RPI;      // instructions per tile
  static_assert(kPfWaves == 4 && IPT * 1024 == kBlock * D * 2, "copy geometry");
  const size_t tile_bytes = (size_t)kBlock * D * (kFP8 ? 1 : 2);
  const char* kp = reinterpret_cast<const char*>(k_pool) + (size_t)g * tile_bytes;
  const char* vp = reinterpret_cast<const char*>(v_pool) + (size_t)g * tile_bytes;
  const size_t blk_stride = (size_t)sc.Hkv * tile_bytes;
  // per lane: the tile offsets of its chunks in instruction m
  uint32_t k_src[IPT], v_src[IPT];
#pragma unroll
  for (int m = 0; m < IPT; ++m) {
    const int kr = kBlock * wave + RPI * m + lane / CPR;  // LDS row
    const int key = k_lds_row(kr) & (kBlock - 1);         // token in block
    k_src[m] = (uint32_t)(key * Lay::KRow +
                          ((lane % CPR) ^ kswz<D>(kr)) * 16);
    const int d = 32 * m + (lane >> 1);
    v_src[m] = (uint32_t)(d * 32 + (((lane & 1) ^ ((d >> 3) & 1)) * 16));
  }

  // Valid tokens of the 4 blocks of step s (0 past the end or for a bad
  // id), from the step's table entries (lane u % 4 holds block 4 s + u % 4).
  auto valid_of = [&](int s, int ids_raw, int nvo[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int blk = 4 * s + u;
      const int raw = readlane(ids_raw, u);
      const bool ok = blk < nblk && (unsigned)raw < (unsigned)sc.NB;
      const int v = L - blk * kBlock;
      nvo[u] = ok ? (v > kBlock ? kBlock : v) : 0;
    }
  };
  // Issues the copies of a step's K tiles (table entries ids_raw) into K
  // buffer buf, and of its V tiles into V buffer buf.  Each wave's copy
  // reads one 16-token tile through a buffer descriptor built in scalar
  // registers for that tile, so the per-copy address arithmetic stays off
  // the vector unit; the lanes' offsets inside the tile are fixed.
  auto tile_copy = [&](const char* pool, int ids_raw, uint8_t* dst,
                       const uint32_t (&src)[IPT]) {
    const int raw = readlane(ids_raw, wave);
    const int id = (unsigned)raw < (unsigned)sc.NB ? raw : 0;
    copy_tile_to_lds<IPT>(pool + (size_t)id * blk_stride, (int)tile_bytes,
                          src, dst);
  };
  auto issue_k = [&](int buf, int ids_raw) {
    tile_copy(kp, ids_raw, lds + buf * Lay::KBytes + kBlock * wave * Lay::KRow,
              k_src);
  };
  auto issue_v = [&](int buf, int ids_raw) {
    tile_copy(vp, ids_raw,
              lds + Lay::V0 + buf * Lay::VBytes + wave * Lay::VTile, v_src);
  };
  // fp8 pools: lane l loads bytes 1024 m + 16 l (m < IPF) of its wave's K
  // tile and of its V tile into registers: 16 d values of one key, or the
  // 16 tokens of one d row.  Widened to bf16 they are two 16-byte chunks of
  // the bf16 layout above: kf_dst / vf_dst hold the LDS offset of the
  // first, the second sits at that offset ^ 16 (the chunks' positions
  // differ in their lowest bit).
  constexpr int IPF = kBlock * D / 1024;
  uint32_t kf_dst[IPF], vf_dst[IPF];
#pragma unroll
  for (int m = 0; m < IPF; ++m) {
    const int byte = 1024 * m + 16 * lane;
    const int tok = byte / D, u = (byte % D) / 16;
    const int kr = kBlock * wave + k_lds_row(tok);
    kf_dst[m] = (uint32_t)(kr * Lay::KRow + ((2 * u) ^ kswz<D>(kr)) * 16);
    const int d = byte / 16;
    vf_dst[m] = (uint32_t)(d * 32 + ((d >> 3) & 1) * 16);
  }
  typedef u32x4 Raw8[IPF];
#if defined(__HIP_DEVICE_COMPILE__)
  auto load_tile8 = [&](const char* pool, int ids_raw, Raw8& raw) {
    const int r = readlane(ids_raw, wave);
    const int id = (unsigned)r < (unsigned)sc.NB ? r : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(pool + (size_t)id * blk_stride), 0, (int)tile_bytes,
        kBufferWord3);
#pragma unroll
    for (int m = 0; m < IPF; ++m)
      raw[m] = __builtin_amdgcn_raw_buffer_load_b128(rs, 1024 * m + 16 * lane,
                                                     0, 0);
  };
#else
  auto load_tile8 = [](const char*, int, Raw8&) {};
#endif
  // 16 fp8 e4m3fn codes -> 16 bf16 (exact: every e4m3fn value is a bf16
  // value, written directly by the scaled conversion with scale 1), stored
  // as two LDS chunks
  auto widen_store = [&](const Raw8& raw, uint8_t* base,
                         const uint32_t (&dst)[IPF]) {
#pragma unroll
    for (int m = 0; m < IPF; ++m) {
      unsigned w[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[2 * k] = __builtin_bit_cast(
            unsigned,
            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[m][k], 1.0f, false));
        w[2 * k + 1] = __builtin_bit_cast(
            unsigned,
            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[m][k], 1.0f, true));
      }
      *reinterpret_cast<u32x4*>(base + dst[m]) = u32x4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(base + (dst[m] ^ 16u)) =
          u32x4{w[4], w[5], w[6], w[7]};
    }
  };
  uint8_t* const v_wave = lds + Lay::V0 + wave * Lay::VTile;

  // Zeroes V of tokens at or past nvs[u] in the V tiles of buffer buf (a
  // masked probability times them must be 0, also where the slot holds NaN).
  auto zero_v_tail = [&](int buf, const int nvs[4]) {
    constexpr int CH = kBlock * D * 2 / 16;  // 16-byte chunks per V tile
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (nvs[u] >= kBlock) continue;
      for (int c = tid; c < CH; c += kPfThreads) {
        const int d = c >> 1;
        const int half = (c & 1) ^ ((d >> 3) & 1);  // tokens 8 half .. + 7
        u32x4* p = reinterpret_cast<u32x4*>(lds + Lay::V0 + buf * Lay::VBytes +
                                            u * Lay::VTile + 16 * c);
        *p = keep_below(*p, nvs[u] - 8 * half);
      }
    }
  };
  auto partial = [](const int nvs[4]) {
    return nvs[0] < kBlock || nvs[1] < kBlock || nvs[2] < kBlock ||
           nvs[3] < kBlock;
  };

  // lane-constant LDS offsets of the operands: K row n32 of each 32-key
  // half, d = 8h + 16c; V row d = n32 of each 32-row tile, keys 8h + 16c
  const int k_off = n32 * Lay::KRow;
  const int k_sw = kswz<D>(n32);  // the same for row 32 + n32
  const int v_off = Lay::V0 + n32 * 32 + 16 * (h ^ ((n32 >> 3) & 1));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  constexpr int NS = 2 * NK;  // score products per step
  constexpr int NP = 4 * NX;  // PV products per step
  // LDS fragments are read this many products ahead (fewer in the
  // shared-prefix pass, whose partial outputs need more registers)
  constexpr int kAhead = kShared ? 2 : 4;

  // K fragment of score product t (d chunk t / 2, key half t % 2) in K
  // buffer kb; V fragment of PV product t (16-key chunk t / NX, d tile
  // t % NX) in V buffer vb.
  auto kfrag = [&](int kb, int t) {
    const int chunk = (2 * (t >> 1) + h) ^ k_sw;
    return *reinterpret_cast<const bf16x8*>(
        lds + kb * Lay::KBytes + k_off + (t & 1) * 32 * Lay::KRow + 16 * chunk);
  };
  // K fragment of key half hf, d chunk kc (16 d values) in K buffer kb.
  auto kfrag_hc = [&](int kb, int hf, int kc) {
    const int chunk = (2 * kc + h) ^ k_sw;
    return *reinterpret_cast<const bf16x8*>(
        lds + kb * Lay::KBytes + k_off + hf * 32 * Lay::KRow + 16 * chunk);
  };
  auto vfrag = [&](int vb, int t) {
    return *reinterpret_cast<const bf16x8*>(
        lds + vb * Lay::VBytes + v_off + (t / NX) * Lay::VTile +
        (t % NX) * 32 * 32);
  };
  auto zero_scores = [](f32x16 (&sv)[2]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[hf][i] = 0.f;
  };
  // Scores of a step on their own (the first step of a tile).
  auto scores = [&](int kb, f32x16 (&sv)[2]) {
    zero_scores(sv);
    bf16x8 ring[kAhead];
#pragma unroll
    for (int t = 0; t < kAhead; ++t) ring[t] = kfrag(kb, t);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const bf16x8 ka = ring[t % kAhead];
      if (t + kAhead < NS) ring[t % kAhead] = kfrag(kb, t + kAhead);
      sv[t & 1] = mfma32(ka, qb[t >> 1], sv[t & 1]);
    }
  };
  // Whether step s needs no mask: four full blocks, all keys at or before
  // the wave's smallest query position.
  auto unmasked = [&](int s, const int nv[4]) {
    return nv[0] == kBlock && nv[1] == kBlock && nv[2] == kBlock &&
           nv[3] == kBlock && s * kKeys + kKeys - 1 <= wp_min;
  };
  // Element pair q (elements 2q, 2q + 1) of a step's scores: -inf past the
  // row's position or a block's valid tokens.  Element 8c + j of half hf is
  // key key0 + 32 hf + 16 c + 8 h + j, in block 2 hf + c at offset 8 h + j.
  auto mask_pair = [&](f32x16 (&sv)[2], int q, int key0, const int nv[4]) {
    const int hf = q >> 3, c = (q >> 2) & 1, j = 2 * (q & 3);
    const int lim = pos - (key0 + 32 * hf + 16 * c + 8 * h) + 1;
    const int nvb = nv[2 * hf + c] - 8 * h;
    const int thr = lim < nvb ? lim : nvb;
    sv[hf][8 * c + j] = j < thr ? sv[hf][8 * c + j] : -INFINITY;
    sv[hf][8 * c + j + 1] = j + 1 < thr ? sv[hf][8 * c + j + 1] : -INFINITY;
  };
  auto max_pair = [](const f32x16 (&sv)[2], int q, float mx) {
    const int hf = q >> 3, e = 2 * (q & 7);
    mx = fmaxf(mx, sv[hf][e]);
    return fmaxf(mx, sv[hf][e + 1]);
  };
  // Probabilities of element pair q into the P operand (one packed word of
  // two bf16), and their sum.
  auto exp_pair = [&](const f32x16 (&sv)[2], int q, float m_use,
                      unsigned (&pw)[2][2][4]) {
    const int hf = q >> 3, c = (q >> 2) & 1, j = 2 * (q & 3);
    const f32x2 e = {
        fast_exp2(fmaf(sv[hf][8 * c + j], sc.c_log2, -m_use)),
        fast_exp2(fmaf(sv[hf][8 * c + j + 1], sc.c_log2, -m_use))};
    const bf16x2 pp = __builtin_convertvector(e, bf16x2);
    pw[hf][c][j >> 1] = __builtin_bit_cast(unsigned, pp);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
  };
  // The P operand of 16-key chunk ch.
  auto p_operand = [](const unsigned (&pw)[2][2][4], int ch) {
    const u32x4 w = {pw[ch >> 1][ch & 1][0], pw[ch >> 1][ch & 1][1],
                     pw[ch >> 1][ch & 1][2], pw[ch >> 1][ch & 1][3]};
    return __builtin_bit_cast(bf16x8, w);
  };

  // The phases below are written as groups of one product, its share of
  // the vector work and the LDS read of a later fragment; a scheduling
  // fence after each group keeps that order, so that the matrix cores and
  // the vector unit work side by side and no fragment is read far ahead.
  auto fence = []() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_barrier(0);
#endif
  };

  // Software pipeline.  Iteration s turns step s's scores into
  // probabilities while the matrix cores compute step s + 1's scores, then
  // accumulates step s's PV products while the vector unit masks step
  // s + 1's scores and takes their row maxima: each wave keeps its own
  // products and vector work in flight together.  K therefore runs one step
  // ahead of V: iteration s copies K of step s + 2 (into the buffer that
  // held K of step s) and V of step s + 1, and both land behind the
  // iteration's closing barrier.
  int nv_nxt[4] = {0, 0, 0, 0};
  // scores of the current and the next step, in two register sets that
  // swap roles from step to step (the loop is unrolled by two)
  f32x16 s_a[2], s_b[2];
  zero_scores(s_a);
  float m_cand = -INFINITY;  // step s's row maximum (log2 units)
  int e1 = 0, e2 = 0;        // table entries of steps s + 1 and s + 2
  const int last = s_end - 1;
  if (s_end > s_begin) {
    const int e0 = table_entry(s_begin);
    e1 = table_entry(last < s_begin + 1 ? last : s_begin + 1);
    Raw8 k0, v0, k1;
    if constexpr (kFP8) {
      load_tile8(kp, e0, k0);
      load_tile8(vp, e0, v0);
      if (last > s_begin) load_tile8(kp, e1, k1);
    } else {
      issue_k(0, e0);
      issue_v(0, e0);
      if (last > s_begin) issue_k(1, e1);
    }
    int nv0[4];
    valid_of(s_begin, e0, nv0);
    e2 = table_entry(last < s_begin + 2 ? last : s_begin + 2);
    wait_all_memory();
    if constexpr (kFP8) {
      widen_store(k0, lds, kf_dst);
      widen_store(v0, v_wave, vf_dst);
      if (last > s_begin) widen_store(k1, lds + Lay::KBytes, kf_dst);
    }
    __syncthreads();
    if (partial(nv0)) {
      zero_v_tail(0, nv0);
      __syncthreads();
    }
    scores(0, s_a);
    if (!unmasked(s_begin, nv0)) {
#pragma unroll
      for (int q = 0; q < 16; ++q) mask_pair(s_a, q, s_begin * kKeys, nv0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = max_pair(s_a, q, mx);
    m_cand = max_xor32(mx) * sc.c_log2;
    __syncthreads();  // K buffer 0 is refilled by the first iteration
  }

  // PV products of step s from V buffer vb, with `extra(t)` (vector work
  // on the next step's scores) after product t.
  auto pv_products = [&](int vb, const unsigned (&pw)[2][2][4], auto extra) {
    bf16x8 vring[kAhead];
#pragma unroll
    for (int t = 0; t < kAhead; ++t) vring[t] = vfrag(vb, t);
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const bf16x8 va = vring[t % kAhead];
      if (t + kAhead < NP) vring[t % kAhead] = vfrag(vb, t + kAhead);
      const int ch = t / NX;
      acc[t % NX] = mfma32(va, p_operand(pw, ch), acc[t % NX]);
      extra(t);
      fence();
    }
  };

  // One step: s_cur holds its scores, s_nxt receives step s + 1's; cb_tag
  // is (s - s_begin) & 1, the buffer pair it reads; kMore: step s + 1
  // exists (its scores are computed here).
  auto step = [&](int s, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], auto cb_tag,
                  auto more_tag) {
    constexpr bool kMore = decltype(more_tag)::value;
    constexpr int cb = decltype(cb_tag)::value, nb = cb ^ 1;
    // the table entries of step s + 3 are loaded before this step's copies
    // are issued, so that waiting for them leaves the copies in flight
    const int e3 = table_entry(s + 3 < last ? s + 3 : last);
    Raw8 kraw, vraw;  // fp8 pools: the copies, held until the step's end
    if (kMore) {
      if constexpr (kFP8) {
        if (s + 2 <= last) load_tile8(kp, e2, kraw);
        load_tile8(vp, e1, vraw);
      } else {
        if (s + 2 <= last) issue_k(cb, e2);
        issue_v(nb, e1);
      }
      valid_of(s + 1, e1, nv_nxt);
    }

    // rescale when some row's max grew by more than kLazy (or was unset)
    if (__ballot(m_cand > m_run + kLazy ||
                 (m_run == -INFINITY && m_cand > -INFINITY))) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha =
          fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
      lsum *= alpha;
#pragma unroll
      for (int X = 0; X < NX; ++X) acc[X] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;

    unsigned pw[2][2][4];
    if constexpr (!kMore) {
      // last step: probabilities, then the PV products
#pragma unroll
      for (int q = 0; q < 16; ++q) exp_pair(s_cur, q, m_use, pw);
      pv_products(cb, pw, [](int) {});
    } else {
      // Phase A: probabilities of step s, scores of step s + 1 (the two key
      // halves' products alternate, so that back-to-back products use
      // independent accumulators).
      {
        constexpr int kPer = 16 / NS;  // probability pairs per product
        bf16x8 ring[kAhead];
#pragma unroll
        for (int t = 0; t < kAhead; ++t) ring[t] = kfrag_hc(nb, t & 1, t >> 1);
        fence();
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const int hf = t & 1, kc = t >> 1;
          const bf16x8 ka = ring[t % kAhead];
          if (t + kAhead < NS)
            ring[t % kAhead] =
                kfrag_hc(nb, (t + kAhead) & 1, (t + kAhead) >> 1);
          const f32x16 zero = {};
          s_nxt[hf] = mfma32(ka, qb[kc], kc == 0 ? zero : s_nxt[hf]);
#pragma unroll
          for (int u = 0; u < kPer; ++u)
            exp_pair(s_cur, t * kPer + u, m_use, pw);
          fence();
        }
      }
      // Phase B: PV products of step s; row maxima of step s + 1 (after
      // its mask, on the rare steps that need one).
      float mx = -INFINITY;
      if (unmasked(s + 1, nv_nxt)) {
        pv_products(cb, pw, [&](int t) {
#pragma unroll
          for (int u = 0; u < 16 / NP; ++u)
            mx = max_pair(s_nxt, t * (16 / NP) + u, mx);
        });
      } else {
        pv_products(cb, pw, [](int) {});
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          mask_pair(s_nxt, q, (s + 1) * kKeys, nv_nxt);
          mx = max_pair(s_nxt, q, mx);
        }
      }
      m_cand = max_xor32(mx) * sc.c_log2;

      wait_all_memory();
      if constexpr (kFP8) {
        if (s + 2 <= last) widen_store(kraw, lds + cb * Lay::KBytes, kf_dst);
        widen_store(vraw, v_wave + nb * Lay::VBytes, vf_dst);
      }
      __syncthreads();
      if (partial(nv_nxt)) {
        zero_v_tail(nb, nv_nxt);
        __syncthreads();
      }
      e1 = e2;
      e2 = e3;
    }
  };
  typedef std::integral_constant<int, 0> Buf0;
  typedef std::integral_constant<int, 1> Buf1;
  int s = s_begin;
  for (; s + 1 < last; s += 2) {
    step(s, s_a, s_b, Buf0(), std::true_type());
    step(s + 1, s_b, s_a, Buf1(), std::true_type());
  }
  if (s < last) {
    step(s, s_a, s_b, Buf0(), std::true_type());
    step(last, s_b, s_a, Buf1(), std::false_type());
  } else if (s == last) {
    step(last, s_a, s_b, Buf0(), std::false_type());
  }

  // lane (n, h) holds O[row n][32 X + 8 a + 4 h + i] in element 4 a + i
  const float ltot = lsum + __shfl_xor(lsum, 32, kWave);
  if (kShared) {
    if (row_ok) {
      const size_t hrow =
          ((size_t)split * sc.T + qs + ti) * sc.Hq + (size_t)g * G + hn;
      if (h == 0) {
        part_ml[hrow * 2] = m_run;
        part_ml[hrow * 2 + 1] = ltot;
      }
      float* orow = part_o + hrow * D + 4 * h;
      const float vs = kFP8 ? sc.v_scale : 1.f;
#pragma unroll
      for (int X = 0; X < NX; ++X)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float4 o = {acc[X][4 * a] * vs, acc[X][4 * a + 1] * vs,
                            acc[X][4 * a + 2] * vs, acc[X][4 * a + 3] * vs};
          *reinterpret_cast<float4*>(orow + 32 * X + 8 * a) = o;
        }
    }
    return;
  }
  if (row_ok) {
    const float inv = ltot > 0.f ? (kFP8 ? sc.v_scale : 1.f) / ltot : 0.f;
    __bf16* orow =
        out + ((size_t)(qs + ti) * sc.Hq + (size_t)g * G + hn) * D + 4 * h;
#pragma unroll
    for (int X = 0; X < NX; ++X)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[X][4 * a + i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * X + 8 * a) = o;
      }
  }
}

template <int D, bool kShared, bool kFP8>
void launch_pf(const PrefillArgs& a, hipStream_t stream) {
  const int tiles =
      (int)(((int64_t)a.s.T * a.s.G + kCols - 1) / kCols) + a.s.B;
  const int splits = kShared ? a.s.splits : 1;
  PrefillSched s = a.s;
  s.attn_grid = tiles * a.s.Hkv * splits;
  const int grid = s.attn_grid + (kShared ? a.s.T : 0);
  hipLaunchKernelGGL((prefill_mfma_kernel<D, kShared, kFP8>),
                     dim3((unsigned)grid), dim3(kPfThreads), 0, stream,
                     reinterpret_cast<const __bf16*>(a.q), a.k_pool, a.v_pool,
                     a.block_tables,
                     a.seq_lens, a.q_start, reinterpret_cast<__bf16*>(a.out),
                     a.member_lens, a.part_ml, a.part_o, a.suffix_tables,
                     a.suffix_lens, s);
}

template <bool kShared>
hipError_t launch_pf_any(int head_size, bool kv_fp8, const PrefillArgs& a,
                         hipStream_t stream) {
  if (a.s.B == 0 || a.s.T == 0) return hipSuccess;
  switch (head_size * 2 + (kv_fp8 ? 1 : 0)) {
    case 128: launch_pf<64, kShared, false>(a, stream); break;
    case 129: launch_pf<64, kShared, true>(a, stream); break;
    case 256: launch_pf<128, kShared, false>(a, stream); break;
    case 257: launch_pf<128, kShared, true>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t prefill_grid(int head_size, int64_t T, int G, int B, int Hkv) {
  (void)head_size;
  return ((T * G + kCols - 1) / kCols + B) * Hkv;
}

hipError_t launch_prefill(int head_size, bool kv_fp8, const PrefillArgs& a,
                          hipStream_t stream) {
  return launch_pf_any<false>(head_size, kv_fp8, a, stream);
}

hipError_t launch_shared_prefix(int head_size, bool kv_fp8,
                                const PrefillArgs& a, hipStream_t stream) {
  return launch_pf_any<true>(head_size, kv_fp8, a, stream);
}

}  // namespace pa
