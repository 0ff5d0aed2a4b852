// Merge pass of the split schedule: combines the partials of every sequence
// whose blocks were divided between ranges, and zeroes the rows of empty
// sequences.  Partials hold a base-2 running max m, the sum l of
// 2^(score - m) and the matching unnormalised output o; with
// M = max_i m_i and w_i = 2^(m_i - M):
//     out = sum_i w_i o_i / sum_i w_i l_i.
// One 64-lane wave per (sequence, query head), kMergeWaves waves per
// workgroup (fewer, larger workgroups dispatch faster; the waves are
// independent).  The partials' (m, l) pairs are read by all lanes at once
// (lane i takes partial i) and reduced across the wave; the output rows
// are summed with lane l owning columns d = l + 64 r.  When a batch has more (sequence, query head) pairs than the
// GPU holds merge workgroups at once, the *_pair_kernel forms run instead:
// one workgroup per (sequence, pair of query heads), each half of the wave
// doing the same for one head with 32 lanes (columns d = l + 32 r), so the
// grid still fits in one round of waves.
#include <math.h>

#include "pa_launch.h"

namespace pa {
namespace {

// Waves per workgroup of the one-head-per-wave merge kernels (without
// shared-prefix partials).  Measured on MI355X, fused step of the
// Llama-shaped batch (2048 waves): 4 per workgroup 86.5 us against 87.3 us
// with 1; fp8 long-context batch 217.7 against 218.2 us.  The cascade form,
// which holds the shared partials in registers, stays at 1 (4 was 0.6 us
// slower).
constexpr int kMergeWaves = 4;

// The (sequence, query head) row of this wave, or -1 past the last row.
__device__ __forceinline__ int merge_row(int waves, int rows) {
  const int r = (int)blockIdx.x * waves +
                __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  return r < rows ? r : -1;
}

// Value of lane l ^ 1, l ^ 2 (quad permutations), of the other quad of the
// lane's 8 (row half-mirror) and of the other 8 of its 16 (row mirror):
// DPP moves, without an LDS round trip.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                         0xF, 0xF, false));
}

// Sum or maximum over the 64 lanes, left in every lane.  After the two quad
// steps every lane of a quad holds the quad's result; each mirror step then
// pairs a group with the other half of its row, and the two swaps pair a
// row with the rows 16 and 32 lanes away.
template <bool kMax>
__device__ __forceinline__ float wave_all(float v) {
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));  // row_half_mirror
  v = op(v, dpp_move<0x140>(v));  // row_mirror
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = op(__builtin_bit_cast(float, (unsigned)r16[0]),
         __builtin_bit_cast(float, (unsigned)r16[1]));
  const unsigned w = __builtin_bit_cast(unsigned, v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return op(__builtin_bit_cast(float, (unsigned)r32[0]),
            __builtin_bit_cast(float, (unsigned)r32[1]));
}

// Row of partial `k` (a range index) for the sequence whose span of work
// units starts at Sb, or -1 when range k is empty and left no partial.
__device__ __forceinline__ int partial_row(int k, int Sb, int U, int g,
                                           int n, const Sched& s) {
  const int r0 = range_begin(k, U, s.Wh);
  if (r0 == range_begin(k + 1, U, s.Wh)) return -1;
  const int slot = Sb < r0 ? 0 : 1;
  return ((g + s.Hkv * k) * 2 + slot) * s.G + n;
}

// Folds the range partials kf..kl of sequence span [Sb, ...) (head n of
// KV head g) into the running (M, lsum, o).  Partials are consumed 64 at a
// time (lane i holds partial i0 + i's m and l) with a running max across
// batches; their output rows are read kRows at a time, the first batch
// issued before the (m, l) reductions so that both loads share one memory
// round trip.
template <int D>
__device__ inline void fold_range_partials(
    int kf, int kl, int Sb, int U, int g, int n, const Sched& s,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    float& M, float& lsum, float (&o)[D / 64]) {
  constexpr int NR = D / 64;
  constexpr int kRows = 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int np = kl - kf + 1;
  for (int i0 = 0; i0 < np; i0 += kWave) {
    const int cnt = np - i0 < kWave ? np - i0 : kWave;
    const int row = lane < cnt ? partial_row(kf + i0 + lane, Sb, U, g, n, s)
                               : -1;
    float mi = -INFINITY, li = 0.f;
    if (row >= 0) {
      mi = part_ml[(size_t)row * 2];
      li = part_ml[(size_t)row * 2 + 1];
    }
    float v[kRows][NR];
    auto load_rows = [&](int t0) {
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int rr = t0 + u < cnt ? readlane(row, t0 + u) : -1;
        const float* po = part_o + (size_t)(rr < 0 ? 0 : rr) * D + lane;
#pragma unroll
        for (int r = 0; r < NR; ++r) v[u][r] = rr < 0 ? 0.f : po[64 * r];
      }
    };
    load_rows(0);
    const float mx = wave_all<true>(mi);
    const float m_new = fmaxf(M, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(M - m_use);
    const float wi = row >= 0 ? fast_exp2(mi - m_use) : 0.f;
    const float wl = wave_all<false>(wi * li);
    lsum = lsum * alpha + wl;
#pragma unroll
    for (int r = 0; r < NR; ++r) o[r] *= alpha;
    M = m_new;
    for (int t0 = 0; t0 < cnt; t0 += kRows) {
      if (t0 > 0) load_rows(t0);
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const float w = __builtin_bit_cast(
            float, readlane(__builtin_bit_cast(int, wi), t0 + u < cnt ? t0 + u
                                                                       : 0));
#pragma unroll
        for (int r = 0; r < NR; ++r) o[r] = fmaf(w, v[u][r], o[r]);
      }
    }
  }
}

template <typename OT, int D>
__global__ __launch_bounds__(kWave * kMergeWaves) void decode_merge_kernel(
    OT* __restrict__ out_all, const int32_t* __restrict__ prefix,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    Sched s) {
  constexpr int NR = D / 64;  // output columns per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int G = s.G;
  const int rid = merge_row(kMergeWaves, s.B * s.Hq);
  if (rid < 0) return;
  const int n = rid % G;
  const int bg = rid / G;
  const int b = bg / s.Hkv;
  const int g = bg % s.Hkv;
  const int Sb = prefix[b];
  const int Sb1 = prefix[b + 1];
  const int U = prefix[s.B];
  OT* out = out_all + ((size_t)b * s.Hq + (size_t)g * G + n) * D;

  if (Sb1 == Sb) {
#pragma unroll
    for (int r = 0; r < NR; ++r) out[lane + 64 * r] = (OT)0.f;
    return;
  }
  const int kf = range_of(Sb, U, s.Wh);
  const int kl = range_of(Sb1 - 1, U, s.Wh);
  if (kf == kl) return;  // finished by the main pass

  float M = -INFINITY, lsum = 0.f;
  float o[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) o[r] = 0.f;
  fold_range_partials<D>(kf, kl, Sb, U, g, n, s, part_ml, part_o, M, lsum,
                         o);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) out[lane + 64 * r] = (OT)(o[r] * inv);
}

// Storage element of a K/V pool: raw bits for the byte copy, and the value.
template <int KB>
struct KvElem;
template <>
struct KvElem<4> {
  typedef uint32_t raw;
  typedef float io;  // q and out element type paired with this pool
  __device__ static float value(raw r) { return __builtin_bit_cast(float, r); }
};
template <>
struct KvElem<2> {
  typedef uint16_t raw;
  typedef __bf16 io;
  __device__ static float value(raw r) {
    return __builtin_bit_cast(float, (uint32_t)r << 16);
  }
};
template <>
struct KvElem<1> {
  typedef uint8_t raw;
  typedef __bf16 io;
  __device__ static float value(raw r) {
    return __builtin_amdgcn_cvt_f32_fp8((int)r, 0);
  }
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The newest token's V column, written as whole rows.  In the [D][16] V
// tile each row d holds 16 tokens, so the token is one element per row:
// written alone, that is D isolated stores of 1-4 bytes and a partly
// written cache line per 4-16 rows, which measured about 3 us per fused step
// of the Llama-shaped batch (512 columns).  Instead each lane reads its
// rows d = first + kStride r (all 16 tokens, 16 KB bytes each), replaces
// token `off` and writes the rows back: consecutive lanes write consecutive
// rows, so every store instruction covers whole cache lines.  The other 15
// tokens of each row keep their bytes (the block belongs to this sequence
// only, and nothing else writes it during the call).  The stores, and those
// of the token's K row, are nontemporal: nothing reads the lines before the
// next step's main pass streams them from HBM (measured: 0.2 us less per
// step of the Llama-shaped batch, 0.5 us on the 256-sequence one).
template <int KB, int D, int kStride>
struct VRows {
  typedef typename KvElem<KB>::raw RT;
  static constexpr int NR = D / kStride;  // rows per lane
  static constexpr int CH = KB;           // 16-byte chunks per row
  u32x4 row[NR][CH];
  __device__ __forceinline__ void load(const RT* v_tile, int first) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          v_tile + (size_t)(first + kStride * r) * kBlock);
#pragma unroll
      for (int c = 0; c < CH; ++c) row[r][c] = src[c];
    }
  }
  __device__ __forceinline__ void store(RT* v_tile, int first, int off,
                                        const RT (&v)[NR]) {
    constexpr int EPD = 4 / KB;  // elements per dword
    const int dw = off / EPD;
    const int shift = 8 * KB * (off % EPD);
    const unsigned mask =
        KB == 4 ? 0xFFFFFFFFu : (((1u << (8 * KB)) - 1u) << shift);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const unsigned val = ((unsigned)v[r] << shift) & mask;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          row[r][c][e] = (4 * c + e == dw)
                             ? ((row[r][c][e] & ~mask) | val)
                             : row[r][c][e];
      u32x4* dst = reinterpret_cast<u32x4*>(
          v_tile + (size_t)(first + kStride * r) * kBlock);
#pragma unroll
      for (int c = 0; c < CH; ++c) __builtin_nontemporal_store(row[r][c], dst + c);
    }
  }
};

// Merge pass of the fused append + decode step, one 64-lane workgroup per
// (sequence, query head).  The main pass attended to every cached token but
// the newest one (len_bias = 1) and left partials: range partials for
// sequences split between ranges, a direct partial for a sequence one range
// finished.  This pass
//   * writes the newest token's K row and V column for KV head g into its
//     slot (the workgroup of the group's first query head; a byte copy),
//   * scores that token from k_new (s = scale * log2e * k_scale * <q, k>),
//   * and folds it into the sequence's partials as one more term of the
//     online softmax:  out = (sum_i w_i o_i + 2^(s-M) v_scale v_new) /
//                            (sum_i w_i l_i + 2^(s-M)).
// The pool slot is not read by this call's main pass (its position is at or
// past the attended length), so the write needs no ordering with it.
// In cascade decode the main pass covered only each sequence's suffix
// blocks; the shared-prefix pass's partial is folded in as one more term
// (when it holds any weight), and `full_lens` gives the true lengths.
// kShared selects the cascade form at compile time, so that the plain step
// holds no registers for the shared partials.
template <int KB, int D, bool kShared>
__global__ __launch_bounds__(kWave * (kShared ? 1 : kMergeWaves)) void
decode_merge_append_kernel(
    typename KvElem<KB>::io* __restrict__ out_all,
    const typename KvElem<KB>::io* __restrict__ q,
    const int32_t* __restrict__ prefix, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ slots,
    const typename KvElem<KB>::raw* __restrict__ k_new,
    const typename KvElem<KB>::raw* __restrict__ v_new,
    typename KvElem<KB>::raw* __restrict__ k_pool,
    typename KvElem<KB>::raw* __restrict__ v_pool,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    const float* __restrict__ direct_ml, const float* __restrict__ direct_o,
    const float* __restrict__ shared_ml, const float* __restrict__ shared_o,
    int shared_splits, const int32_t* __restrict__ full_lens, Sched s) {
  typedef KvElem<KB> E;
  typedef typename E::io OT;
  typedef typename E::raw RT;
  constexpr int NR = D / 64;
  const int lane = threadIdx.x & (kWave - 1);
  const int G = s.G;
  const int rid = merge_row(kShared ? 1 : kMergeWaves, s.B * s.Hq);
  if (rid < 0) return;
  const int n = rid % G;
  const int bg = rid / G;
  const int b = bg / s.Hkv;
  const int g = bg % s.Hkv;
  const size_t h_row = (size_t)b * s.Hq + (size_t)g * G + n;
  const size_t kv_row = ((size_t)b * s.Hkv + g) * D;

  // independent loads: one memory round trip
  const int Sb = prefix[b];
  const int Sb1 = prefix[b + 1];
  const int U = prefix[s.B];
  const int L = full_lens ? full_lens[b] : seq_lens[b];
  const int slot = slots[b];
  // shared-prefix partials, one per key range (all issued up front)
  constexpr int NS = kShared ? kMaxSharedSplits : 1;
  float sh_m[NS], sh_l[NS];
  float sh_o[NS][NR];
  const size_t split_rows = (size_t)s.B * s.Hq;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const bool live = kShared && k < shared_splits;
    const size_t r = (size_t)k * split_rows + h_row;
    sh_m[k] = live ? shared_ml[r * 2] : -INFINITY;
    sh_l[k] = live ? shared_ml[r * 2 + 1] : 0.f;
#pragma unroll
    for (int x = 0; x < NR; ++x)
      sh_o[k][x] = live ? shared_o[r * D + lane + 64 * x] : 0.f;
  }
  RT kr[NR], vr[NR];
  float qf[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int d = lane + 64 * r;
    kr[r] = k_new[kv_row + d];
    vr[r] = v_new[kv_row + d];
    qf[r] = (float)q[h_row * D + d];
  }
  // the wave of the group's first query head writes the token's slot; its
  // V rows are read with the loads above (one round trip) and written back
  // after the partials are read, so that waiting for them does not delay
  // the second round trip (measured: 0.7 us less per cascade step)
  const bool writes = n == 0 && slot >= 0 && slot < s.NB * kBlock;
  const size_t tile =
      writes ? ((size_t)(slot >> 4) * s.Hkv + g) * kBlock * D : 0;
  VRows<KB, D, kWave> vrows;
  if (writes) vrows.load(v_pool + tile, lane);

  float dot = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) dot = fmaf(qf[r], E::value(kr[r]), dot);
  dot = wave_all<false>(dot);

  float M = -INFINITY, lsum = 0.f;
  float o[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) o[r] = 0.f;
  if (Sb1 > Sb) {
    const int kf = range_of(Sb, U, s.Wh);
    const int kl = range_of(Sb1 - 1, U, s.Wh);
    if (kf == kl) {
      M = direct_ml[h_row * 2];
      lsum = direct_ml[h_row * 2 + 1];
#pragma unroll
      for (int r = 0; r < NR; ++r) o[r] = direct_o[h_row * D + lane + 64 * r];
    } else {
      fold_range_partials<D>(kf, kl, Sb, U, g, n, s, part_ml, part_o, M,
                             lsum, o);
    }
  }
  if (writes) {
    const int off = slot & (kBlock - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r)
      __builtin_nontemporal_store(kr[r], k_pool + tile + (size_t)off * D + lane + 64 * r);
    vrows.store(v_pool + tile, lane, off, vr);
  }
  if constexpr (kShared) {  // the shared prefix's partials, as more terms
    float m_new = M;
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (sh_l[k] > 0.f) m_new = fmaxf(m_new, sh_m[k]);
    if (m_new > -INFINITY) {
      const float alpha = fast_exp2(M - m_new);
      lsum *= alpha;
#pragma unroll
      for (int r = 0; r < NR; ++r) o[r] *= alpha;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        // a range with no weight is skipped, not multiplied by zero: its
        // output row was never written
        if (!(sh_l[k] > 0.f)) continue;
        const float w = fast_exp2(sh_m[k] - m_new);
        lsum = fmaf(w, sh_l[k], lsum);
#pragma unroll
        for (int r = 0; r < NR; ++r) o[r] = fmaf(w, sh_o[k][r], o[r]);
      }
      M = m_new;
    }
  }
  if (L >= 1) {  // the newest token, from k_new / v_new
    const float sn = dot * s.c_log2;
    const float m_new = fmaxf(M, sn);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(M - m_use);
    const float w = fast_exp2(sn - m_use);
    lsum = lsum * alpha + w;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      o[r] = fmaf(w * s.v_scale, E::value(vr[r]), o[r] * alpha);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  OT* out = out_all + h_row * D;
#pragma unroll
  for (int r = 0; r < NR; ++r) out[lane + 64 * r] = (OT)(o[r] * inv);
}

// Sum or maximum over each half (32 lanes) of the wave, left in every lane
// of that half: the quad and mirror steps of wave_all, then the swap with
// the row 16 lanes away.
template <bool kMax>
__device__ __forceinline__ float half_all(float v) {
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));  // row_half_mirror
  v = op(v, dpp_move<0x140>(v));  // row_mirror
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return op(__builtin_bit_cast(float, (unsigned)r16[0]),
            __builtin_bit_cast(float, (unsigned)r16[1]));
}

// Value of lane `base + t` for lanes of the first half, `32 + base + t`
// for the second (t uniform).
__device__ __forceinline__ int half_lane(int v, int t, bool upper) {
  const int lo = readlane(v, t);
  const int hi = readlane(v, 32 + t);
  return upper ? hi : lo;
}

// The range partials kf..kl of sequence span [Sb, ...) folded into the
// running (M, lsum, o) of one query head per half wave (KV head g, head n
// within its group).  Partials are consumed 32 at a time (half lane i holds
// partial i0 + i's m and l); their output rows are read kRows at a time,
// the first batch issued before the (m, l) reductions so that both loads
// share one memory round trip.  Lane il of a half owns columns il + 32 r.
template <int D>
__device__ inline void fold_range_partials_half(
    int kf, int kl, int Sb, int U, int g, int n, bool upper, const Sched& s,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    float& M, float& lsum, float (&o)[D / 32]) {
  constexpr int NR = D / 32;
  constexpr int kRows = 4;
  const int il = threadIdx.x & 31;
  const int np = kl - kf + 1;
  for (int i0 = 0; i0 < np; i0 += 32) {
    const int cnt = np - i0 < 32 ? np - i0 : 32;
    const int row = il < cnt ? partial_row(kf + i0 + il, Sb, U, g, n, s) : -1;
    float mi = -INFINITY, li = 0.f;
    if (row >= 0) {
      mi = part_ml[(size_t)row * 2];
      li = part_ml[(size_t)row * 2 + 1];
    }
    float v[kRows][NR];
    auto load_rows = [&](int t0) {
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int rr = t0 + u < cnt ? half_lane(row, t0 + u, upper) : -1;
        const float* po = part_o + (size_t)(rr < 0 ? 0 : rr) * D + il;
#pragma unroll
        for (int r = 0; r < NR; ++r) v[u][r] = rr < 0 ? 0.f : po[32 * r];
      }
    };
    load_rows(0);
    const float mx = half_all<true>(mi);
    const float m_new = fmaxf(M, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(M - m_use);
    const float wi = row >= 0 ? fast_exp2(mi - m_use) : 0.f;
    const float wl = half_all<false>(wi * li);
    lsum = lsum * alpha + wl;
#pragma unroll
    for (int r = 0; r < NR; ++r) o[r] *= alpha;
    M = m_new;
    for (int t0 = 0; t0 < cnt; t0 += kRows) {
      if (t0 > 0) load_rows(t0);
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int tt = t0 + u < cnt ? t0 + u : 0;
        const float w = __builtin_bit_cast(
            float, half_lane(__builtin_bit_cast(int, wi), tt, upper));
#pragma unroll
        for (int r = 0; r < NR; ++r) o[r] = fmaf(w, v[u][r], o[r]);
      }
    }
  }
}

// The newest token's K row and V column for KV head g, written by all G
// query heads of its group together (the two-heads-per-wave merge) when G
// is a power of two and each head has at most one 16-byte chunk of the V
// rows per lane: head n takes rows [n D/G, (n + 1) D/G), lane i the i-th
// 16-byte chunk of those rows (both chunks of a row are rewritten, so the
// head's stores cover whole cache lines) and K element n D/G + i.  The
// chunk is read with the first round trip of loads and written back after
// the partials are folded; only the loaded values are held through the
// fold, the offsets are recomputed from (tile, n, G, i).
template <int KB, int D, int kLanes>
struct TokenShare {
  typedef typename KvElem<KB>::raw RT;
  static constexpr int kTokPerChunk = 16 / KB;  // tokens per 16-byte chunk
  __device__ static bool usable(int G) {
    return G >= 1 && (G & (G - 1)) == 0 && G <= D && (D / G) * KB <= kLanes;
  }
  u32x4 chunk;
  RT v, k;
  __device__ __forceinline__ static int chunk_at(int n, int G, int i) {
    const int rph = D / G;  // rows per head
    return (n * rph + i / KB) * kBlock + (i % KB) * kTokPerChunk;
  }
  __device__ __forceinline__ void load(const RT* __restrict__ v_pool,
                                       const RT* __restrict__ k_new,
                                       const RT* __restrict__ v_new,
                                       size_t kv_row, size_t tile, int n,
                                       int G, int i) {
    const int rph = D / G;
    const bool has_chunk = i < rph * KB;
    chunk = has_chunk ? *reinterpret_cast<const u32x4*>(
                            v_pool + tile + chunk_at(n, G, i))
                      : u32x4{0, 0, 0, 0};
    v = has_chunk ? v_new[kv_row + n * rph + i / KB] : RT(0);
    k = i < rph ? k_new[kv_row + n * rph + i] : RT(0);
  }
  __device__ __forceinline__ void store(RT* __restrict__ k_pool,
                                        RT* __restrict__ v_pool, size_t tile,
                                        int off, int n, int G, int i) {
    const int rph = D / G;
    if (i < rph)
      __builtin_nontemporal_store(k, k_pool + tile + (size_t)off * D +
                                         n * rph + i);
    if (i >= rph * KB) return;
    if (i % KB == off / kTokPerChunk) {
      constexpr int EPD = 4 / KB;  // elements per dword
      const int within = off % kTokPerChunk;
      const int dw = within / EPD;
      const int shift = 8 * KB * (within % EPD);
      const unsigned mask =
          KB == 4 ? 0xFFFFFFFFu : (((1u << (8 * KB)) - 1u) << shift);
      const unsigned val = ((unsigned)v << shift) & mask;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        chunk[e] = e == dw ? ((chunk[e] & ~mask) | val) : chunk[e];
    }
    __builtin_nontemporal_store(
        chunk, reinterpret_cast<u32x4*>(v_pool + tile + chunk_at(n, G, i)));
  }
};

// The same merge pass with one 64-lane workgroup per (sequence, pair of
// query heads), for batches whose (sequence, query head) count exceeds the
// waves the GPU holds at once: the first half of the wave takes head 2p,
// the second head 2p + 1, so the sequence's lengths and ranges are read
// once for both and half as many waves run.  (When the batch fits in one
// round, one head per wave is faster: more loads in flight.)  The main
// pass attended to every cached token but the newest one
// (len_bias = 1) and left partials: range partials for sequences split
// between ranges, a direct partial for a sequence one range finished.  For
// its query head, each half
//   * writes the newest token's K row and V column for KV head g into its
//     slot (the half of the group's first query head; a byte copy),
//   * scores that token from k_new (s = scale * log2e * k_scale * <q, k>),
//   * and folds it into the sequence's partials as one more term of the
//     online softmax:  out = (sum_i w_i o_i + 2^(s-M) v_scale v_new) /
//                            (sum_i w_i l_i + 2^(s-M)).
// The pool slot is not read by this call's main pass (its position is at or
// past the attended length), so the write needs no ordering with it.
// (The cascade form always uses one head per wave.)  With an odd number of
// query heads the second half of the last workgroup of a sequence has no head:
// it loads from a valid row and stores nothing.
template <int KB, int D>
__global__ __launch_bounds__(64) void decode_merge_append_pair_kernel(
    typename KvElem<KB>::io* __restrict__ out_all,
    const typename KvElem<KB>::io* __restrict__ q,
    const int32_t* __restrict__ prefix, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ slots,
    const typename KvElem<KB>::raw* __restrict__ k_new,
    const typename KvElem<KB>::raw* __restrict__ v_new,
    typename KvElem<KB>::raw* __restrict__ k_pool,
    typename KvElem<KB>::raw* __restrict__ v_pool,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    const float* __restrict__ direct_ml, const float* __restrict__ direct_o,
    Sched s) {
  typedef KvElem<KB> E;
  typedef typename E::io OT;
  typedef typename E::raw RT;
  constexpr int NR = D / 32;
  const int lane = threadIdx.x;
  const bool upper = lane >= 32;
  const int il = lane & 31;
  const int G = s.G;
  const int pairs = (s.Hq + 1) >> 1;
  const int b = blockIdx.x / pairs;
  const int h_raw = 2 * (blockIdx.x % pairs) + (upper ? 1 : 0);
  const bool has_head = h_raw < s.Hq;
  const int h = has_head ? h_raw : s.Hq - 1;  // a valid row to read
  const int g = h / G;
  const int n = h % G;
  const size_t h_row = (size_t)b * s.Hq + h;
  const size_t kv_row = ((size_t)b * s.Hkv + g) * D;

  // independent loads: one memory round trip
  const int Sb = prefix[b];
  const int Sb1 = prefix[b + 1];
  const int U = prefix[s.B];
  const int L = seq_lens[b];
  const int slot = slots[b];
  RT kr[NR], vr[NR];
  float qf[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int d = il + 32 * r;
    kr[r] = k_new[kv_row + d];
    vr[r] = v_new[kv_row + d];
    qf[r] = (float)q[h_row * D + d];
  }
  // The token's slot: written by every head of the group together
  // (TokenShare: one 16-byte chunk per lane, read with the loads above),
  // else by the half of the group's first query head at the end (whole V
  // rows: reading them up front would hold 32 more registers through the
  // fold, and this kernel must stay within 64, 8 waves per SIMD, so that
  // the grid runs in one round).
  const bool slot_ok = has_head && slot >= 0 && slot < s.NB * kBlock;
  const size_t tile =
      slot_ok ? ((size_t)(slot >> 4) * s.Hkv + g) * kBlock * D : 0;
  const int off = slot & (kBlock - 1);
  typedef TokenShare<KB, D, 32> Share;
  const bool shared_write = slot_ok && Share::usable(G);
  Share share;
  if (shared_write)
    share.load(v_pool, k_new, v_new, kv_row, tile, n, G, il);

  float dot = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) dot = fmaf(qf[r], E::value(kr[r]), dot);
  dot = half_all<false>(dot);

  float M = -INFINITY, lsum = 0.f;
  float o[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) o[r] = 0.f;
  if (Sb1 > Sb) {
    const int kf = range_of(Sb, U, s.Wh);
    const int kl = range_of(Sb1 - 1, U, s.Wh);
    if (kf == kl) {
      M = direct_ml[h_row * 2];
      lsum = direct_ml[h_row * 2 + 1];
#pragma unroll
      for (int r = 0; r < NR; ++r) o[r] = direct_o[h_row * D + il + 32 * r];
    } else {
      fold_range_partials_half<D>(kf, kl, Sb, U, g, n, upper, s, part_ml,
                                  part_o, M, lsum, o);
    }
  }
  if (L >= 1) {  // the newest token, from k_new / v_new
    const float sn = dot * s.c_log2;
    const float m_new = fmaxf(M, sn);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(M - m_use);
    const float w = fast_exp2(sn - m_use);
    lsum = lsum * alpha + w;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      o[r] = fmaf(w * s.v_scale, E::value(vr[r]), o[r] * alpha);
  }
  if (!has_head) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  OT* out = out_all + h_row * D;
#pragma unroll
  for (int r = 0; r < NR; ++r) out[il + 32 * r] = (OT)(o[r] * inv);
  if (shared_write) {
    share.store(k_pool, v_pool, tile, off, n, G, il);
  } else if (slot_ok && n == 0) {
    VRows<KB, D, 32> vrows;
    vrows.load(v_pool + tile, il);
#pragma unroll
    for (int r = 0; r < NR; ++r)
      __builtin_nontemporal_store(kr[r], k_pool + tile + (size_t)off * D + il + 32 * r);
    vrows.store(v_pool + tile, il, off, vr);
  }
}

// The plain merge pass with one 64-lane workgroup per (sequence, pair of
// query heads), for batches with more (sequence, query head) pairs than the
// GPU holds merge workgroups at once: the first half of the wave takes head
// 2p, the second head 2p + 1.  With an odd number of query heads the second
// half of a sequence's last workgroup has no head and stores nothing.
template <typename OT, int D>
__global__ __launch_bounds__(64) void decode_merge_pair_kernel(
    OT* __restrict__ out_all, const int32_t* __restrict__ prefix,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    Sched s) {
  constexpr int NR = D / 32;
  const int lane = threadIdx.x;
  const bool upper = lane >= 32;
  const int il = lane & 31;
  const int G = s.G;
  const int pairs = (s.Hq + 1) >> 1;
  const int b = blockIdx.x / pairs;
  const int h_raw = 2 * (blockIdx.x % pairs) + (upper ? 1 : 0);
  const bool has_head = h_raw < s.Hq;
  const int h = has_head ? h_raw : s.Hq - 1;
  const int g = h / G;
  const int n = h % G;
  const int Sb = prefix[b];
  const int Sb1 = prefix[b + 1];
  const int U = prefix[s.B];
  OT* out = out_all + ((size_t)b * s.Hq + h) * D;

  if (Sb1 == Sb) {
    if (has_head) {
#pragma unroll
      for (int r = 0; r < NR; ++r) out[il + 32 * r] = (OT)0.f;
    }
    return;
  }
  const int kf = range_of(Sb, U, s.Wh);
  const int kl = range_of(Sb1 - 1, U, s.Wh);
  if (kf == kl) return;  // finished by the main pass

  float M = -INFINITY, lsum = 0.f;
  float o[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) o[r] = 0.f;
  fold_range_partials_half<D>(kf, kl, Sb, U, g, n, upper, s, part_ml, part_o,
                              M, lsum, o);
  if (!has_head) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) out[il + 32 * r] = (OT)(o[r] * inv);
}

template <typename OT, int D>
void launch_one(const DecodeArgs& a, hipStream_t stream) {
  if (a.merge_pairs) {
    const dim3 grid((unsigned)(a.s.B * ((a.s.Hq + 1) / 2)));
    hipLaunchKernelGGL((decode_merge_pair_kernel<OT, D>), grid, dim3(64), 0,
                       stream, reinterpret_cast<OT*>(a.out), a.prefix,
                       a.part_ml, a.part_o, a.s);
    return;
  }
  const int rows = a.s.B * a.s.Hq;
  const dim3 grid((unsigned)((rows + kMergeWaves - 1) / kMergeWaves));
  hipLaunchKernelGGL((decode_merge_kernel<OT, D>), grid,
                     dim3(kWave * kMergeWaves), 0, stream,
                     reinterpret_cast<OT*>(a.out), a.prefix, a.part_ml,
                     a.part_o, a.s);
}

template <typename OT>
hipError_t launch_m(int head_size, const DecodeArgs& a, hipStream_t stream) {
  switch (head_size) {
    case 64: launch_one<OT, 64>(a, stream); break;
    case 128: launch_one<OT, 128>(a, stream); break;
    case 256: launch_one<OT, 256>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB, int D, bool kShared>
void launch_append_k(const DecodeArgs& a, hipStream_t stream) {
  typedef KvElem<KB> E;
  constexpr int waves = kShared ? 1 : kMergeWaves;
  const int rows = a.s.B * a.s.Hq;
  const dim3 grid((unsigned)((rows + waves - 1) / waves));
  hipLaunchKernelGGL(
      (decode_merge_append_kernel<KB, D, kShared>), grid, dim3(kWave * waves),
      0, stream,
      reinterpret_cast<typename E::io*>(a.out),
      reinterpret_cast<const typename E::io*>(a.q), a.prefix, a.seq_lens,
      a.slots, reinterpret_cast<const typename E::raw*>(a.k_new),
      reinterpret_cast<const typename E::raw*>(a.v_new),
      reinterpret_cast<typename E::raw*>(a.k_pool_w),
      reinterpret_cast<typename E::raw*>(a.v_pool_w), a.part_ml, a.part_o,
      a.direct_ml, a.direct_o, a.shared_ml, a.shared_o, a.shared_splits,
      a.full_lens, a.s);
}

template <int KB, int D>
void launch_append_one(const DecodeArgs& a, hipStream_t stream) {
  if (a.shared_ml) {
    launch_append_k<KB, D, true>(a, stream);
  } else if (a.merge_pairs) {
    typedef KvElem<KB> E;
    const dim3 grid((unsigned)(a.s.B * ((a.s.Hq + 1) / 2)));
    hipLaunchKernelGGL(
        (decode_merge_append_pair_kernel<KB, D>), grid, dim3(64), 0, stream,
        reinterpret_cast<typename E::io*>(a.out),
        reinterpret_cast<const typename E::io*>(a.q), a.prefix, a.seq_lens,
        a.slots, reinterpret_cast<const typename E::raw*>(a.k_new),
        reinterpret_cast<const typename E::raw*>(a.v_new),
        reinterpret_cast<typename E::raw*>(a.k_pool_w),
        reinterpret_cast<typename E::raw*>(a.v_pool_w), a.part_ml, a.part_o,
        a.direct_ml, a.direct_o, a.s);
  } else {
    launch_append_k<KB, D, false>(a, stream);
  }
}

template <int KB>
hipError_t launch_append_d(int head_size, const DecodeArgs& a,
                           hipStream_t stream) {
  switch (head_size) {
    case 64: launch_append_one<KB, 64>(a, stream); break;
    case 128: launch_append_one<KB, 128>(a, stream); break;
    case 256: launch_append_one<KB, 256>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_merge_append(int kv_bytes, int head_size,
                                      const DecodeArgs& a,
                                      hipStream_t stream) {
  if (a.s.B == 0) return hipSuccess;
  switch (kv_bytes) {
    case 4: return launch_append_d<4>(head_size, a, stream);
    case 2: return launch_append_d<2>(head_size, a, stream);
    case 1: return launch_append_d<1>(head_size, a, stream);
  }
  return hipErrorInvalidValue;
}

int occupancy_decode_merge_append(int kv_bytes, int head_size) {
  const void* f = nullptr;
#define PA_MERGE_KERNEL(KB, D) \
  reinterpret_cast<const void*>(decode_merge_append_kernel<KB, D, false>)
  switch (kv_bytes * 1000 + head_size) {
    case 4064: f = PA_MERGE_KERNEL(4, 64); break;
    case 4128: f = PA_MERGE_KERNEL(4, 128); break;
    case 4256: f = PA_MERGE_KERNEL(4, 256); break;
    case 2064: f = PA_MERGE_KERNEL(2, 64); break;
    case 2128: f = PA_MERGE_KERNEL(2, 128); break;
    case 2256: f = PA_MERGE_KERNEL(2, 256); break;
    case 1064: f = PA_MERGE_KERNEL(1, 64); break;
    case 1128: f = PA_MERGE_KERNEL(1, 128); break;
    case 1256: f = PA_MERGE_KERNEL(1, 256); break;
    default: return 0;
  }
#undef PA_MERGE_KERNEL
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, f, kWave * kMergeWaves, 0) != hipSuccess)
    return 0;
  return n * kMergeWaves;
}

int occupancy_decode_merge(bool out_bf16, int head_size) {
  const void* f = nullptr;
  switch (head_size) {
    case 64:
      f = out_bf16 ? reinterpret_cast<const void*>(decode_merge_kernel<__bf16, 64>)
                   : reinterpret_cast<const void*>(decode_merge_kernel<float, 64>);
      break;
    case 128:
      f = out_bf16 ? reinterpret_cast<const void*>(decode_merge_kernel<__bf16, 128>)
                   : reinterpret_cast<const void*>(decode_merge_kernel<float, 128>);
      break;
    case 256:
      f = out_bf16 ? reinterpret_cast<const void*>(decode_merge_kernel<__bf16, 256>)
                   : reinterpret_cast<const void*>(decode_merge_kernel<float, 256>);
      break;
    default: return 0;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, f, kWave * kMergeWaves, 0) != hipSuccess)
    return 0;
  return n * kMergeWaves;
}

hipError_t launch_decode_merge(bool out_bf16, int head_size,
                               const DecodeArgs& a, hipStream_t stream) {
  if (a.s.B == 0) return hipSuccess;
  return out_bf16 ? launch_m<__bf16>(head_size, a, stream)
                  : launch_m<float>(head_size, a, stream);
}

}  // namespace pa
