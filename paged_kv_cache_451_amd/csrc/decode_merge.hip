// Merge pass of the split schedule: combines the partials of every sequence
// whose blocks were divided between ranges, and zeroes the rows of empty
// sequences.  Partials hold a base-2 running max m, the sum l of
// 2^(score - m) and the matching unnormalised output o; with
// M = max_i m_i and w_i = 2^(m_i - M):
//     out = sum_i w_i o_i / sum_i w_i l_i.
// One 64-lane workgroup per (sequence, query head).  The partials' (m, l)
// pairs are read by all lanes at once (lane i takes partial i) and reduced
// across the wave; the output rows are summed with lane l owning columns
// d = l + 64 r.
#include <math.h>

#include "pa_launch.h"

namespace pa {
namespace {

// Row of partial `k` (a range index) for sequence span starting at block
// Sb, or -1 when range k is empty and left no partial.
__device__ __forceinline__ int partial_row(int k, int Sb, int U, int g,
                                           int n, const Sched& s) {
  const int r0 = range_begin(k, U, s.Wh);
  if (r0 == range_begin(k + 1, U, s.Wh)) return -1;
  const int slot = Sb < r0 ? 0 : 1;
  return ((g + s.Hkv * k) * 2 + slot) * s.G + n;
}

template <typename OT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    OT* __restrict__ out_all, const int32_t* __restrict__ prefix,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    Sched s) {
  constexpr int NR = D / 64;    // output columns per lane
  constexpr int kRows = 16;     // partial rows loaded per batch
  const int lane = threadIdx.x;
  const int G = s.G;
  const int n = blockIdx.x % G;
  const int bg = blockIdx.x / G;
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
  const int np = kl - kf + 1;

  // Partials are consumed 64 at a time (lane i holds partial i0 + i's m and
  // l) with a running max across batches; their output rows are read
  // kRows at a time, the first batch issued before the (m, l) reductions so
  // that both loads share one memory round trip.
  float M = -INFINITY, lsum = 0.f;
  float o[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) o[r] = 0.f;
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
    float mx = mi;
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1) mx = fmaxf(mx, __shfl_xor(mx, x, kWave));
    const float m_new = fmaxf(M, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(M - m_use);
    const float wi = row >= 0 ? fast_exp2(mi - m_use) : 0.f;
    float wl = wi * li;
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1) wl += __shfl_xor(wl, x, kWave);
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
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) out[lane + 64 * r] = (OT)(o[r] * inv);
}

template <typename OT, int D>
void launch_one(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.s.B * a.s.Hq));
  hipLaunchKernelGGL((decode_merge_kernel<OT, D>), grid, dim3(64), 0, stream,
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

}  // namespace

hipError_t launch_decode_merge(bool out_bf16, int head_size,
                               const DecodeArgs& a, hipStream_t stream) {
  if (a.s.B == 0) return hipSuccess;
  return out_bf16 ? launch_m<__bf16>(head_size, a, stream)
                  : launch_m<float>(head_size, a, stream);
}

}  // namespace pa
