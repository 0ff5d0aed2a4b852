// Merge pass of the split schedule: combines the partials of every sequence
// whose blocks were divided between ranges, and zeroes the rows of empty
// sequences.  Partials hold a base-2 running max m, the sum l of
// 2^(score - m) and the matching unnormalised output o; with
// M = max_i m_i and w_i = 2^(m_i - M):
//     out = sum_i w_i o_i / sum_i w_i l_i.
// One 64-lane workgroup per (sequence, KV head); lane l owns d = l + 64 r.
#include <math.h>

#include "pa_launch.h"

namespace pa {
namespace {

template <typename OT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int NR = D / 64;
  const SplitArgs& s = a.s;
  const int lane = threadIdx.x;
  const int b = blockIdx.x / s.Hkv;
  const int g = blockIdx.x % s.Hkv;
  const int G = s.G;
  const int Sb = s.prefix[b];
  const int Sb1 = s.prefix[b + 1];
  const int U = s.prefix[s.B];
  OT* out = reinterpret_cast<OT*>(a.out) +
            ((size_t)b * a.Hq + (size_t)g * G) * D;

  if (Sb1 == Sb) {
    for (int i = lane; i < G * D; i += kWave) out[i] = (OT)0.f;
    return;
  }
  const int kf = range_of(Sb, U, s.Wh);
  const int kl = range_of(Sb1 - 1, U, s.Wh);
  if (kf == kl) return;  // finished by the main pass

  for (int n = 0; n < G; ++n) {
    float M = -INFINITY;
    for (int k = kf; k <= kl; ++k) {
      const int r0 = range_begin(k, U, s.Wh);
      if (r0 == range_begin(k + 1, U, s.Wh)) continue;  // empty range
      const int slot = Sb < r0 ? 0 : 1;
      const size_t row = ((size_t)(g + s.Hkv * k) * 2 + slot) * G + n;
      M = fmaxf(M, s.part_ml[row * 2]);
    }
    float lsum = 0.f;
    float o[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) o[r] = 0.f;
    if (M != -INFINITY) {
      for (int k = kf; k <= kl; ++k) {
        const int r0 = range_begin(k, U, s.Wh);
        if (r0 == range_begin(k + 1, U, s.Wh)) continue;
        const int slot = Sb < r0 ? 0 : 1;
        const size_t row = ((size_t)(g + s.Hkv * k) * 2 + slot) * G + n;
        const float wgt = fast_exp2(s.part_ml[row * 2] - M);
        lsum += wgt * s.part_ml[row * 2 + 1];
#pragma unroll
        for (int r = 0; r < NR; ++r)
          o[r] += wgt * s.part_o[row * D + lane + 64 * r];
      }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) out[n * D + lane + 64 * r] = (OT)(o[r] * inv);
  }
}

template <typename OT>
hipError_t launch_m(int head_size, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.s.B * a.s.Hkv));
  switch (head_size) {
    case 64:
      hipLaunchKernelGGL((decode_merge_kernel<OT, 64>), grid, dim3(64), 0,
                         stream, a);
      break;
    case 128:
      hipLaunchKernelGGL((decode_merge_kernel<OT, 128>), grid, dim3(64), 0,
                         stream, a);
      break;
    case 256:
      hipLaunchKernelGGL((decode_merge_kernel<OT, 256>), grid, dim3(64), 0,
                         stream, a);
      break;
    default:
      return hipErrorInvalidValue;
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
