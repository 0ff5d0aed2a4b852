// Merge pass of the split schedule: combines the partials of every sequence
// whose blocks were divided between ranges, and zeroes the rows of empty
// sequences.  Partials hold a base-2 running max m, the sum l of
// 2^(score - m) and the matching unnormalised output o; with
// M = max_i m_i and w_i = 2^(m_i - M):
//     out = sum_i w_i o_i / sum_i w_i l_i.
// One 64-lane workgroup per (sequence, query head).  The partials' (m, l)
// pairs are read by all lanes at once (lane i takes partial i) and reduced
// across the wave; the output rows are then summed with lane l owning
// columns d = l + 64 r, four partial rows loaded per step.
#include <math.h>

#include "pa_launch.h"

namespace pa {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <typename OT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    OT* __restrict__ out_all, const int32_t* __restrict__ prefix,
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    Sched s) {
  constexpr int NR = D / 64;
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

  // row of partial kf + i, or -1 for an empty range (no partial written)
  auto row_of = [&](int i) -> int {
    const int k = kf + i;
    const int r0 = range_begin(k, U, s.Wh);
    if (r0 == range_begin(k + 1, U, s.Wh)) return -1;
    const int slot = Sb < r0 ? 0 : 1;
    return ((g + s.Hkv * k) * 2 + slot) * G + n;
  };

  float M = -INFINITY;
  for (int i0 = 0; i0 < np; i0 += kWave) {
    const int i = i0 + lane;
    const int row = i < np ? row_of(i) : -1;
    const float mi = row >= 0 ? part_ml[(size_t)row * 2] : -INFINITY;
    M = fmaxf(M, wave_max(mi));
  }
  float lsum = 0.f;
  float o[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) o[r] = 0.f;
  if (M != -INFINITY) {
    for (int i0 = 0; i0 < np; i0 += kWave) {
      const int i = i0 + lane;
      const int row = i < np ? row_of(i) : -1;
      float wi = 0.f;
      if (row >= 0) {
        wi = fast_exp2(part_ml[(size_t)row * 2] - M);
        lsum += wi * part_ml[(size_t)row * 2 + 1];
      }
      const int cnt = np - i0 < kWave ? np - i0 : kWave;
      int t = 0;
      for (; t + 4 <= cnt; t += 4) {
        float w4[4], v4[4][NR];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rr = __builtin_amdgcn_readlane(row, t + u);
          w4[u] = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wi),
                                               t + u));
          const float* po = part_o + (size_t)(rr < 0 ? 0 : rr) * D + lane;
#pragma unroll
          for (int r = 0; r < NR; ++r) v4[u][r] = rr < 0 ? 0.f : po[64 * r];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < NR; ++r) o[r] += w4[u] * v4[u][r];
      }
      for (; t < cnt; ++t) {
        const int rr = __builtin_amdgcn_readlane(row, t);
        const float wt = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wi), t));
        const float* po = part_o + (size_t)(rr < 0 ? 0 : rr) * D + lane;
#pragma unroll
        for (int r = 0; r < NR; ++r) o[r] += rr < 0 ? 0.f : wt * po[64 * r];
      }
    }
    lsum = wave_sum(lsum);
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
