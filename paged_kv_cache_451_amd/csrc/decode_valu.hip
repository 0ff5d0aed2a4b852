// Paged decode attention for fp32 q and fp32 KV on the vector ALUs.
//
// Same split schedule and partial format as the matrix-core kernel
// (pa_device.h), one 16-token block per step:
//
// * scores: lane (t, j) = (l % 16, l / 16) reads quarter j of token t's K
//   row and forms the partial dot product with each of the G query heads
//   (q staged in LDS); two xor-shuffles (16, 32) complete the sum, so every
//   lane of row t holds s_t.
// * online softmax in base 2 per head, reductions over the 16 token lanes.
// * values: lane l owns output columns d = l + 64 r; it reads the D x 16 V
//   tile row d (16 contiguous tokens) and accumulates sum_t p_t V[d][t] with
//   the block's weights broadcast from LDS.
//
// Tokens past seq_len (or in blocks with an out-of-range id) get -inf scores
// and zeroed V values.
#include <math.h>

#include "pa_launch.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxG = 8;

template <int D>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeArgs a) {
  constexpr int DQ = D / 4;   // K values per lane (a quarter row)
  constexpr int NR = D / 64;  // output columns per lane
  __shared__ float qs[kMaxG][D];
  __shared__ float ps[kMaxG][kBlock];

  const SplitArgs& s = a.s;
  const int lane = threadIdx.x;
  const int t = lane & 15;
  const int j = lane >> 4;
  const int w = blockIdx.x;
  const int g = w % s.Hkv;
  const int k = w / s.Hkv;
  const int G = s.G;

  const int U = total_blocks(s, w == 0);
  const int u0 = range_begin(k, U, s.Wh);
  const int u1 = range_begin(k + 1, U, s.Wh);
  if (u0 >= u1) return;

  const float* kpool = reinterpret_cast<const float*>(a.k_pool);
  const float* vpool = reinterpret_cast<const float*>(a.v_pool);
  const size_t tile = (size_t)kBlock * D;

  for_each_segment(s, u0, u1, [&](int b, int Sb, int Sb1) {
    const int L = clamped_len(s, b);
    const int lo = (Sb > u0 ? Sb : u0) - Sb;
    const int hi = (Sb1 < u1 ? Sb1 : u1) - Sb;
    const int32_t* trow = s.block_tables + (size_t)b * s.max_blocks;

    __syncthreads();
    const float* qrow = reinterpret_cast<const float*>(a.q) +
                        ((size_t)b * a.Hq + (size_t)g * G) * D;
    for (int i = lane; i < G * D; i += kWave) qs[i / D][i % D] = qrow[i];
    __syncthreads();

    float o[kMaxG][NR];
    float m[kMaxG], l[kMaxG], alpha[kMaxG];
#pragma unroll
    for (int n = 0; n < kMaxG; ++n) {
      m[n] = -INFINITY;
      l[n] = 0.f;
#pragma unroll
      for (int r = 0; r < NR; ++r) o[n][r] = 0.f;
    }

    for (int blk = lo; blk < hi; ++blk) {
      int p = trow[blk];
      int nv = (unsigned)p < (unsigned)a.NB ? L - blk * kBlock : 0;
      nv = nv > kBlock ? kBlock : nv;
      if ((unsigned)p >= (unsigned)a.NB) p = 0;
      const size_t base = ((size_t)p * s.Hkv + g) * tile;

      float kr[DQ];
      const float* kp = kpool + base + (size_t)t * D + j * DQ;
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        f32x4 v = *reinterpret_cast<const f32x4*>(kp + i);
        kr[i] = v[0]; kr[i + 1] = v[1]; kr[i + 2] = v[2]; kr[i + 3] = v[3];
      }
      float vr[NR][kBlock];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float* vp = vpool + base + (size_t)(lane + 64 * r) * kBlock;
#pragma unroll
        for (int c = 0; c < kBlock; c += 4) {
          f32x4 v = *reinterpret_cast<const f32x4*>(vp + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) vr[r][c + e] = c + e < nv ? v[e] : 0.f;
        }
      }

      __syncthreads();  // previous block's weights are no longer read
#pragma unroll
      for (int n = 0; n < kMaxG; ++n) {
        if (n >= G) break;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DQ; ++i) dot = fmaf(qs[n][j * DQ + i], kr[i], dot);
        dot += __shfl_xor(dot, 16, kWave);
        dot += __shfl_xor(dot, 32, kWave);
        float x = t < nv ? dot * a.c_log2 : -INFINITY;
        float mx = x;
#pragma unroll
        for (int o2 = 1; o2 < 16; o2 <<= 1) mx = wave_max_xor(mx, o2);
        const float m_new = fmaxf(m[n], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        alpha[n] = fast_exp2(m[n] - m_use);
        const float p_t = fast_exp2(x - m_use);
        float psum = p_t;
#pragma unroll
        for (int o2 = 1; o2 < 16; o2 <<= 1)
          psum += __shfl_xor(psum, o2, kWave);
        l[n] = l[n] * alpha[n] + psum;
        m[n] = m_new;
        if (j == 0) ps[n][t] = p_t;
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < kMaxG; ++n) {
        if (n >= G) break;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          float acc = o[n][r] * alpha[n];
#pragma unroll
          for (int tt = 0; tt < kBlock; ++tt)
            acc = fmaf(ps[n][tt], vr[r][tt], acc);
          o[n][r] = acc;
        }
      }
    }

    const bool split = Sb < u0 || Sb1 > u1;
#pragma unroll
    for (int n = 0; n < kMaxG; ++n) {
      if (n >= G) break;
      if (!split) {
        const float inv = l[n] > 0.f ? a.v_scale / l[n] : 0.f;
        float* orow = reinterpret_cast<float*>(a.out) +
                      ((size_t)b * a.Hq + (size_t)g * G + n) * D;
#pragma unroll
        for (int r = 0; r < NR; ++r) orow[lane + 64 * r] = o[n][r] * inv;
      } else {
        const int slot = Sb < u0 ? 0 : 1;
        const size_t row = ((size_t)w * 2 + slot) * G + n;
#pragma unroll
        for (int r = 0; r < NR; ++r)
          s.part_o[row * D + lane + 64 * r] = o[n][r] * a.v_scale;
        if (lane == 0) {
          s.part_ml[row * 2 + 0] = m[n];
          s.part_ml[row * 2 + 1] = l[n];
        }
      }
    }
  });
}

}  // namespace

hipError_t launch_decode_valu(int head_size, const DecodeArgs& a, int nwg,
                              hipStream_t stream) {
  switch (head_size) {
    case 64:
      hipLaunchKernelGGL(decode_valu_kernel<64>, dim3(nwg), dim3(64), 0,
                         stream, a);
      break;
    case 128:
      hipLaunchKernelGGL(decode_valu_kernel<128>, dim3(nwg), dim3(64), 0,
                         stream, a);
      break;
    case 256:
      hipLaunchKernelGGL(decode_valu_kernel<256>, dim3(nwg), dim3(64), 0,
                         stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
