// Paged decode attention on gfx950 matrix cores (bf16 q; bf16 or fp8 KV).
//
// One 64-lane workgroup streams one KV head's blocks over its range of the
// split schedule (pa_device.h) two blocks (32 tokens) at a time.  With
// G = Hq/Hkv query heads sharing the KV head, each pair of blocks is two
// dense contractions:
//
//   S^T[32 tok][G] = K[32 tok][D] . Q^T[D][G]        (D/32 MFMAs per 16 tok)
//   O^T[D][G]     += V^T[D][32 tok] . P^T[32 tok][G]  (D/16 MFMAs)
//
// both with v_mfma_f32_16x16x32_bf16 (heads padded to 16 columns).  The
// operands come straight from HBM in the MFMA register layout - no LDS:
//
// * MFMA operand lane l holds row (l % 16) and the 8 consecutive k-values of
//   group (l / 16).  A contraction is indifferent to the order of its k
//   index, so k-slots are mapped to whatever bytes are contiguous in memory.
// * QK: A = K rows.  Row m of MFMA set s (s = 0, 1) is token
//   8*((m/4)%2) + 4*s + m%4 of block m/8 of the pair; k-slots are 8
//   consecutive d values.  With the 16x16 output layout (lane l holds rows
//   4*(l/16)+i, column l%16), lane (n, j) = (l%16, l/16) then owns the 8
//   consecutive tokens 8*(j%2) .. 8*(j%2)+7 of block j/2 for query head n.
// * PV: B = P^T with exactly those 8 tokens as lane (n, j)'s k-slots, and
//   A = V^T rows: since V is stored [D][16 tokens] per block and head, lane
//   (m, j) loads the same 8 tokens of row d = 16*X + m as 16 contiguous
//   bytes (8 for fp8).  No data moves between lanes except the per-head
//   max reduction of the online softmax (xor 16 and xor 32).
//
// The loop is software-pipelined over pairs: the K/V loads of pair i+1 and
// the block-table entries of pair i+2 are issued before pair i is computed,
// so each wave keeps a pair (16 KiB of bf16) in flight while it works.  The
// loads sit outside any branch so the compiler's wait before pair i's math
// leaves pair i+1's loads outstanding.  fp8 bytes stay raw in registers
// until their pair is computed.
//
// The softmax is the usual online one in base 2: scores are scaled by
// scale*log2(e) (times k_scale for fp8), a running max m and sum l are kept
// per head and the accumulator is rescaled when m grows (skipped when no
// head's max changed).  P is rounded to bf16 for the matrix core; l sums the
// rounded values, so the weights applied to V sum exactly to the
// normaliser.  fp8 e4m3fn codes widen exactly to bf16 (v_cvt_pk_f32_fp8 then
// v_cvt_pk_bf16_f32); k_scale is folded into the score scale and v_scale
// into the output.
//
// Masking: tokens at or past seq_len, the second block of a pair that lies
// outside the range, and out-of-range block ids contribute nothing: their
// scores become -inf and their V values are zeroed in registers, so NaN or
// stale bytes in unused slots never reach the result.  Such blocks are read
// from a valid block address (the pair's first block, or block 0).  A pair
// that is never computed (the software pipeline's loads past the last pair
// of the range) reads a zero tile in device memory instead (idle_tile below).
#include <math.h>

#include <hip/hip_ext.h>

#include "pa_launch.h"

namespace pa {
namespace {

// Largest (block, KV head) tile the kernel reads: 16 tokens x 256 values of
// 2 bytes.  Every lane's loads of a pair stay inside one tile (checked at
// compile time in Pair), so loads pointed at this array with the lanes'
// tile offsets stay in bounds.  It is read-only and never written: it
// holds zeros for the whole life of the process, a few lines that stay in
// the caches.
constexpr int kIdleTileBytes = 16 * 256 * 2;
__device__ __align__(256) uint8_t idle_tile[kIdleTileBytes];

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 fp8 e4m3fn codes (little-endian bytes of w) -> 8 bf16, exact: every
// e4m3fn value is a bf16 value, and the scaled conversion with scale 1
// writes it directly (one instruction per two codes instead of a float32
// conversion and a bf16 rounding).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(unsigned w0, unsigned w1) {
  bf16x8 r;
  const unsigned w[2] = {w0, w1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, true);
    r[4 * h + 0] = lo[0];
    r[4 * h + 1] = lo[1];
    r[4 * h + 2] = hi[0];
    r[4 * h + 3] = hi[1];
  }
  return r;
}

// K/V bytes are read once per call: nontemporal loads keep them from
// displacing reused lines (block tables, q, partials) in the caches and
// measurably raise the sustained read rate of a pure stream.
template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
  return __builtin_nontemporal_load(p);
}

// Zero elements e >= nv of an 8-element bf16 vector.
__device__ __forceinline__ bf16x8 keep_first(bf16x8 v, int nv) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    unsigned m = (2 * w < nv ? 0x0000FFFFu : 0u) |
                 (2 * w + 1 < nv ? 0xFFFF0000u : 0u);
    u[w] &= m;
  }
  return __builtin_bit_cast(bf16x8, u);
}

// Raw block-table entries of the pair starting at logical block `blk`.  The
// indices are clamped to the segment's last block hi - 1, so the loads are
// always in bounds and need no branch; the second block of a pair that ends
// the segment repeats the first, so its loads fall on the same lines.
struct RawIds {
  int e0, e1;
};

__device__ __forceinline__ RawIds raw_ids(const int32_t* __restrict__ trow,
                                          int blk, int hi) {
  const int last = hi - 1;
  return RawIds{trow[blk < last ? blk : last],
                trow[blk + 1 < last ? blk + 1 : last]};
}

// Physical ids to read, made safe: an id outside [0, NB) becomes block 0.
__device__ __forceinline__ int safe_id(int p, int NB) {
  return (unsigned)p < (unsigned)NB ? p : 0;
}

// Valid tokens of the two blocks of the pair at `blk` (uniform); a pair at
// or past the segment end `hi` has none.
__device__ __forceinline__ void pair_valid(const RawIds& r, int blk, int hi,
                                           int L, int NB, int& nv0,
                                           int& nv1) {
  const bool ok0 = blk < hi && (unsigned)r.e0 < (unsigned)NB;
  const bool ok1 = blk + 1 < hi && (unsigned)r.e1 < (unsigned)NB;
  const int a = L - blk * kBlock;
  const int b = a - kBlock;
  nv0 = ok0 ? (a > kBlock ? kBlock : a) : 0;
  nv1 = ok1 ? (b > kBlock ? kBlock : (b < 0 ? 0 : b)) : 0;
}

// Lane-constant element offsets, inside one (block, KV head) tile, of lane
// (m, j) = (l % 16, l / 16)'s K and V loads (layout at the top of this
// file): K token row 8*((m/4)%2) + m%4 (MFMA set s adds 4 rows), columns
// from kColJ * j; V row d = m of the [D][16] tile (each further MFMA adds
// 16 rows), tokens from 8*(j%2).  Which block of the pair a lane reads is
// chosen by its base address (m >= 8 for K, j >= 2 for V).
__host__ __device__ constexpr int k_lane_offset(int r16, int j, int D,
                                                int col_j) {
  return (((r16 >> 2) & 1) * 8 + (r16 & 3)) * D + col_j * j;
}
__host__ __device__ constexpr int v_lane_offset(int r16, int j) {
  return r16 * kBlock + 8 * (j & 1);
}

// Storage-type specific register sets of one pair.  bf16: K chunk c of a row
// is the 8 values at d = 32c + 8j; fp8: one 16-byte load at d = 64c' + 16j
// feeds MFMAs 2c' (low 8 bytes) and 2c'+1 (high 8 bytes).  Q uses the same d
// sets (qcol).  k_off / v_off give the element offset of each load from the
// lane's base address, and kKVec / kVVec its width in elements.
template <bool FP8, int D>
struct Pair;

template <int D>
struct Pair<false, D> {
  typedef __bf16 T;
  static constexpr int NC = D / 32, NX = D / 16, kColJ = 8;
  static constexpr int kKLoads = NC, kKVec = 8, kVVec = 8;
  bf16x8 k[2][NC];
  bf16x8 v[NX];
  __host__ __device__ static constexpr int k_off(int s, int c) {
    return 4 * D * s + 32 * c;
  }
  __host__ __device__ static constexpr int v_off(int x) { return 256 * x; }
  __device__ static __forceinline__ int qcol(int c, int j) {
    return 32 * c + 8 * j;
  }
  __device__ __forceinline__ void load(const T* kl, const T* vl) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        k[s][c] = stream_load(reinterpret_cast<const bf16x8*>(kl + k_off(s, c)));
#pragma unroll
    for (int x = 0; x < NX; ++x)
      v[x] = stream_load(reinterpret_cast<const bf16x8*>(vl + v_off(x)));
  }
  __device__ __forceinline__ bf16x8 kop(int s, int c) const { return k[s][c]; }
  __device__ __forceinline__ bf16x8 vop(int x) const { return v[x]; }
};

template <int D>
struct Pair<true, D> {
  typedef uint8_t T;
  static constexpr int NC = D / 32, NX = D / 16, kColJ = 16;
  static constexpr int kKLoads = D / 64, kKVec = 16, kVVec = 8;
  u32x4 k[2][D / 64];
  u32x2 v[NX];
  __host__ __device__ static constexpr int k_off(int s, int c) {
    return 4 * D * s + 64 * c;
  }
  __host__ __device__ static constexpr int v_off(int x) { return 256 * x; }
  __device__ static __forceinline__ int qcol(int c, int j) {
    return 64 * (c >> 1) + 16 * j + 8 * (c & 1);
  }
  __device__ __forceinline__ void load(const T* kl, const T* vl) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < D / 64; ++c)
        k[s][c] = stream_load(reinterpret_cast<const u32x4*>(kl + k_off(s, c)));
#pragma unroll
    for (int x = 0; x < NX; ++x)
      v[x] = stream_load(reinterpret_cast<const u32x2*>(vl + v_off(x)));
  }
  __device__ __forceinline__ bf16x8 kop(int s, int c) const {
    const u32x4 w = k[s][c >> 1];
    return (c & 1) ? fp8x8_to_bf16(w[2], w[3]) : fp8x8_to_bf16(w[0], w[1]);
  }
  __device__ __forceinline__ bf16x8 vop(int x) const {
    return fp8x8_to_bf16(v[x][0], v[x][1]);
  }
};

// True when every load of every lane of a pair stays inside one
// (block, KV head) tile of 16 * D elements, for K and for V: then a pair
// read from any valid tile (or from idle_tile) never leaves it.
template <bool FP8, int D>
constexpr bool pair_stays_in_tile() {
  typedef Pair<FP8, D> P;
  for (int l = 0; l < kWave; ++l) {
    const int r16 = l & 15, j = l >> 4;
    const int kb = k_lane_offset(r16, j, D, P::kColJ);
    for (int s = 0; s < 2; ++s)
      for (int c = 0; c < P::kKLoads; ++c) {
        const int o = kb + P::k_off(s, c);
        if (o < 0 || o + P::kKVec > kBlock * D) return false;
      }
    const int vb = v_lane_offset(r16, j);
    for (int x = 0; x < P::NX; ++x) {
      const int o = vb + P::v_off(x);
      if (o < 0 || o + P::kVVec > kBlock * D) return false;
    }
  }
  return kBlock * D * (int)sizeof(typename P::T) <= kIdleTileBytes;
}

// Blocks per work unit of the split schedule (pa_device.h): one loop step,
// two pairs of blocks.
constexpr int kUnitShift = 2;

// One sequence b of a workgroup's range: the part [lo, hi) of its blocks
// that the range covers (its units [Sb, Sb1) clipped to the range's units,
// in blocks; the sequence's last unit may hold fewer than 4), its pool
// length L, and which partial slot it leaves (-1: the range holds all of
// it, 0: it started in an earlier range, 1: it continues in a later one).
struct Seg {
  int b, lo, hi, L, slot;
  __device__ __forceinline__ void bind(const int32_t* __restrict__ lens,
                                       const Sched& sc, int Sb, int Sb1,
                                       int u0, int u1) {
    L = pool_len(lens[b], sc.len_bias, sc.max_blocks);
    const int nb = (L + kBlock - 1) / kBlock;
    lo = ((Sb > u0 ? Sb : u0) - Sb) << kUnitShift;
    hi = ((Sb1 < u1 ? Sb1 : u1) - Sb) << kUnitShift;
    hi = hi < nb ? hi : nb;
    slot = Sb < u0 ? 0 : (Sb1 > u1 ? 1 : -1);
  }
};

// Minimum resident waves per SIMD the register budget is held to.
template <int D>
constexpr int min_waves() { return D > 128 ? 1 : 2; }

template <bool FP8, int D>
__global__ __launch_bounds__(64, min_waves<D>()) void decode_mfma_kernel(
    const __bf16* __restrict__ q, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, __bf16* __restrict__ out,
    int32_t* __restrict__ prefix, float* __restrict__ part_ml,
    float* __restrict__ part_o, float* __restrict__ direct_ml,
    float* __restrict__ direct_o, Sched sc) {
  typedef Pair<FP8, D> P;
  typedef typename P::T T;
  constexpr int NC = P::NC;
  constexpr int NX = P::NX;

  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int j = lane >> 4;
  const int w = blockIdx.x;
  const int g = w % sc.Hkv;
  const int k = w / sc.Hkv;
  const int G = sc.G;

  int first_units;
  const int U = total_units(seq_lens, sc.B, sc.max_blocks, sc.len_bias,
                            kUnitShift, w == 0 ? prefix : nullptr,
                            &first_units);
  const int u0 = range_begin(k, U, sc.Wh);
  const int u1 = range_begin(k + 1, U, sc.Wh);
  if (u0 >= u1) return;

  const T* kpool = reinterpret_cast<const T*>(k_pool);
  const T* vpool = reinterpret_cast<const T*>(v_pool);
  const size_t tile = (size_t)kBlock * D;  // elements of one (block, head) tile
  const size_t gtile = (size_t)g * tile;
  const size_t btile = (size_t)sc.Hkv * tile;
  // lane-constant parts of the K and V addresses
  static_assert(pair_stays_in_tile<FP8, D>(),
                "a lane's loads must stay inside one (block, head) tile");
  const int k_lane = k_lane_offset(r16, j, D, P::kColJ);
  const int v_lane = v_lane_offset(r16, j);
  const bool k_hi = r16 >= 8;  // K row from the pair's second block
  const bool v_hi = j >= 2;    // V tokens from the pair's second block

  // The range's sequences ("segments") in order, one ahead of the one being
  // computed: the last loads a segment issues are the next segment's first
  // pair, so the wave's stream of loads does not stop between sequences.
  SegCursor cursor(seq_lens, sc.B, sc.max_blocks, sc.len_bias, kUnitShift,
                   u0, u1, first_units);
  Seg cur, nxt;
  int Sb, Sb1;
  if (!cursor.next(cur.b, Sb, Sb1)) return;
  cur.bind(seq_lens, sc, Sb, Sb1, u0, u1);
  bool more = cursor.next(nxt.b, Sb, Sb1);
  if (more) nxt.bind(seq_lens, sc, Sb, Sb1, u0, u1);
  // block-table row of sequence b
  auto trow = [&](int b) { return block_tables + (size_t)b * sc.max_blocks; };

  // Q as the B operand of QK: lane (n, j) holds head g*G + n.
  auto load_q = [&](bf16x8* qv, int b) {
    const int n = r16;
    const __bf16* qrow = q + ((size_t)b * sc.Hq + (size_t)g * G + n) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      qv[c] = n < G ? *reinterpret_cast<const bf16x8*>(qrow + P::qcol(c, j))
                    : z;
    }
  };

  P A, B;
  // Table entries of the pairs ahead (see the loop invariant below).
  RawIds ia = raw_ids(trow(cur.b), cur.lo, cur.hi);
  RawIds ib, ic, id;
  // Loads of pair pblk of the current segment, or, at and past its loop
  // end `blk_end`, of the next segment's pair at nxt.lo + (pblk - blk_end).
  // A pair past both is never computed: its loads go to idle_tile (a few
  // cached lines) instead of HBM, at the same lane offsets, which keep them
  // inside it (pair_stays_in_tile).
  const T* idle = reinterpret_cast<const T*>(idle_tile);
  auto issue = [&](P& pr, const RawIds& ids, int pblk, const Seg& s,
                   int blk_end) {
    const size_t base0 = (size_t)safe_id(ids.e0, sc.NB) * btile + gtile;
    const size_t base1 = (size_t)safe_id(ids.e1, sc.NB) * btile + gtile;
    const bool live =
        pblk < s.hi ||
        (more && pblk >= blk_end && nxt.lo + (pblk - blk_end) < nxt.hi);
    pr.load((live ? kpool + (k_hi ? base1 : base0) : idle) + k_lane,
            (live ? vpool + (v_hi ? base1 : base0) : idle) + v_lane);
  };
  issue(A, ia, cur.lo, cur, cur.lo + 4);
  ib = raw_ids(trow(cur.b), cur.lo + 2, cur.hi);

  bf16x8 qb[NC], qn[NC];
  load_q(qb, cur.b);

  f32x4 acc[NX];
  float m, lsum;

  for (;;) {  // segments
    // first pair index the pair loop below does not compute
    const int blk_end = cur.lo + 4 * ((cur.hi - cur.lo + 3) >> 2);
    const int L = cur.L;
    const int hi = cur.hi;
    if (more) load_q(qn, nxt.b);
    auto ids_at = [&](int pblk) {
      const bool here = pblk < blk_end || !more;
      return raw_ids(trow(here ? cur.b : nxt.b),
                     here ? pblk : nxt.lo + (pblk - blk_end),
                     here ? hi : nxt.hi);
    };

#pragma unroll
    for (int x = 0; x < NX; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    lsum = 0.f;

    auto compute = [&](const P& pr, const RawIds& ids, int blk) {
      int nv0, nv1;
      pair_valid(ids, blk, hi, L, sc.NB, nv0, nv1);
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        s0 = mfma16x16x32(pr.kop(0, c), qb[c], s0);
        s1 = mfma16x16x32(pr.kop(1, c), qb[c], s1);
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = s0[i] * sc.c_log2;
        x[4 + i] = s1[i] * sc.c_log2;
      }
      // this lane's 8 tokens: 8*(j%2) + e of block j/2
      const bool partial = nv0 + nv1 < 2 * kBlock;
      int nv = (v_hi ? nv1 : nv0) - 8 * (j & 1);
      nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
      if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = e < nv ? x[e] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      bf16x8 pb;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pe = (__bf16)fast_exp2(x[e] - m_use);
        pb[e] = pe;
        psum += (float)pe;
      }
      lsum = lsum * alpha + psum;
      m = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int xx = 0; xx < NX; ++xx) acc[xx] *= alpha;
      }
#pragma unroll
      for (int xx = 0; xx < NX; ++xx) {
        bf16x8 vv = pr.vop(xx);
        if (partial) vv = keep_first(vv, nv);
        acc[xx] = mfma16x16x32(vv, pb, acc[xx]);
      }
    };

    // Loop invariant: A holds the loads of pair blk, ia its table entries,
    // ib the entries of pair blk + 2.  Loads are issued unconditionally
    // (see raw_ids), and the loop leaves only after computing both register
    // sets: when a segment has an odd number of pairs, the last B pair lies
    // past its end and is computed with every token masked.  The loop
    // leaves with A holding the next segment's first pair, the same state
    // as at its back edge, so the compiler's wait before each pair's math
    // leaves the following pair's loads outstanding.
    // The scheduling barriers keep each pair's loads issued before the
    // other pair's math: left free, the scheduler may sink them below it,
    // which leaves a pair's loads no time in flight.
    int blk = cur.lo;
    for (;;) {
      issue(B, ib, blk + 2, cur, blk_end);
      __builtin_amdgcn_sched_barrier(0);
      ic = ids_at(blk + 4);
      compute(A, ia, blk);
      blk += 2;
      issue(A, ic, blk + 2, cur, blk_end);
      __builtin_amdgcn_sched_barrier(0);
      id = ids_at(blk + 4);
      compute(B, ib, blk);
      blk += 2;
      if (blk >= hi) break;
      ia = ic;
      ib = id;
    }

    // lane (n, j) holds O[head n][16X + 4j + i]
    float ltot = lsum + __shfl_xor(lsum, 16, kWave);
    ltot += __shfl_xor(ltot, 32, kWave);
    const int n = r16;
    const int b = cur.b;
    if (n < G) {
      const bool split = cur.slot >= 0;
      if (!split && sc.len_bias) {
        // the merge pass still has to fold in the appended token
        const size_t row = (size_t)b * sc.Hq + (size_t)g * G + n;
        float* po = direct_o + row * D + 4 * j;
#pragma unroll
        for (int xx = 0; xx < NX; ++xx)
          *reinterpret_cast<f32x4*>(po + 16 * xx) = acc[xx] * sc.v_scale;
        if (j == 0) {
          direct_ml[row * 2 + 0] = m;
          direct_ml[row * 2 + 1] = ltot;
        }
      } else if (!split) {
        const float inv = ltot > 0.f ? sc.v_scale / ltot : 0.f;
        __bf16* orow = out + ((size_t)b * sc.Hq + (size_t)g * G + n) * D +
                       4 * j;
#pragma unroll
        for (int xx = 0; xx < NX; ++xx) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[xx][i] * inv);
          *reinterpret_cast<bf16x4*>(orow + 16 * xx) = o;
        }
      } else {
        const size_t row = ((size_t)w * 2 + cur.slot) * G + n;
        float* po = part_o + row * D + 4 * j;
#pragma unroll
        for (int xx = 0; xx < NX; ++xx)
          *reinterpret_cast<f32x4*>(po + 16 * xx) = acc[xx] * sc.v_scale;
        if (j == 0) {
          part_ml[row * 2 + 0] = m;
          part_ml[row * 2 + 1] = ltot;
        }
      }
    }

    if (!more) break;
    cur = nxt;
    more = cursor.next(nxt.b, Sb, Sb1);
    if (more) nxt.bind(seq_lens, sc, Sb, Sb1, u0, u1);
    ia = ic;
    ib = id;
#pragma unroll
    for (int c = 0; c < NC; ++c) qb[c] = qn[c];
  }
}

template <bool FP8, int D>
void launch_one(const DecodeArgs& a, int nwg, hipStream_t stream) {
  hipExtLaunchKernelGGL((decode_mfma_kernel<FP8, D>), dim3(nwg), dim3(64), 0,
                        stream, a.ev_start, a.ev_stop, 0,
                        reinterpret_cast<const __bf16*>(a.q), a.k_pool,
                     a.v_pool, a.block_tables, a.seq_lens,
                     reinterpret_cast<__bf16*>(a.out), a.prefix, a.part_ml,
                     a.part_o, a.direct_ml, a.direct_o, a.s);
}

template <bool FP8, int D>
int occupancy_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(decode_mfma_kernel<FP8, D>), 64,
          0) != hipSuccess)
    return 0;
  return n;
}

template <bool FP8>
int occupancy_d(int head_size) {
  switch (head_size) {
    case 64: return occupancy_one<FP8, 64>();
    case 128: return occupancy_one<FP8, 128>();
    case 256: return occupancy_one<FP8, 256>();
  }
  return 0;
}

template <bool FP8>
hipError_t launch_d(int head_size, const DecodeArgs& a, int nwg,
                    hipStream_t stream) {
  switch (head_size) {
    case 64: launch_one<FP8, 64>(a, nwg, stream); break;
    case 128: launch_one<FP8, 128>(a, nwg, stream); break;
    case 256: launch_one<FP8, 256>(a, nwg, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int occupancy_decode_mfma(bool fp8, int head_size) {
  return fp8 ? occupancy_d<true>(head_size) : occupancy_d<false>(head_size);
}

hipError_t launch_decode_mfma(bool fp8, int head_size, const DecodeArgs& a,
                              int nwg, hipStream_t stream) {
  return fp8 ? launch_d<true>(head_size, a, nwg, stream)
             : launch_d<false>(head_size, a, nwg, stream);
}

}  // namespace pa
