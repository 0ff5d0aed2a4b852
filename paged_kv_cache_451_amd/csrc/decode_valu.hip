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
// and zeroed V values.  K/V are read with nontemporal loads (each byte is
// used once per call).
#include <math.h>

#include <hip/hip_ext.h>

#include "pa_launch.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxG = 8;

template <int D>
__global__ __launch_bounds__(64) void decode_valu_kernel(
    const float* __restrict__ q, const float* __restrict__ kpool,
    const float* __restrict__ vpool, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, float* __restrict__ out,
    int32_t* __restrict__ prefix, float* __restrict__ part_ml,
    float* __restrict__ part_o, float* __restrict__ direct_ml,
    float* __restrict__ direct_o, Sched sc) {
  constexpr int DQ = D / 4;   // K values per lane (a quarter row)
  constexpr int NR = D / 64;  // output columns per lane
  __shared__ float qs[kMaxG][D];
  __shared__ float ps[kMaxG][kBlock];

  const int lane = threadIdx.x;
  const int t = lane & 15;
  const int j = lane >> 4;
  const int w = blockIdx.x;
  const int g = w % sc.Hkv;
  const int k = w / sc.Hkv;
  const int G = sc.G;

  // one block per loop step: work units of one block
  const int U = total_units(seq_lens, sc.B, sc.max_blocks, sc.len_bias, 0,
                            w == 0 ? prefix : nullptr);
  const int u0 = range_begin(k, U, sc.Wh);
  const int u1 = range_begin(k + 1, U, sc.Wh);
  if (u0 >= u1) return;

  const size_t tile = (size_t)kBlock * D;

  for_each_segment(seq_lens, sc.B, sc.max_blocks, sc.len_bias, 0, u0, u1,
                   [&](int b, int Sb, int Sb1) {
    const int L = pool_len(seq_lens[b], sc.len_bias, sc.max_blocks);
    const int lo = (Sb > u0 ? Sb : u0) - Sb;
    const int hi = (Sb1 < u1 ? Sb1 : u1) - Sb;
    const int32_t* trow = block_tables + (size_t)b * sc.max_blocks;

    __syncthreads();
    const float* qrow = q + ((size_t)b * sc.Hq + (size_t)g * G) * D;
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
      int nv = (unsigned)p < (unsigned)sc.NB ? L - blk * kBlock : 0;
      nv = nv > kBlock ? kBlock : nv;
      if ((unsigned)p >= (unsigned)sc.NB) p = 0;
      const size_t base = ((size_t)p * sc.Hkv + g) * tile;

      float kr[DQ];
      const float* kp = kpool + base + (size_t)t * D + j * DQ;
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        f32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(kp + i));
        kr[i] = v[0]; kr[i + 1] = v[1]; kr[i + 2] = v[2]; kr[i + 3] = v[3];
      }
      float vr[NR][kBlock];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float* vp = vpool + base + (size_t)(lane + 64 * r) * kBlock;
#pragma unroll
        for (int c = 0; c < kBlock; c += 4) {
          f32x4 v = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4*>(vp + c));
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
        float x = t < nv ? dot * sc.c_log2 : -INFINITY;
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
      if (!split && sc.len_bias) {
        // the merge pass still has to fold in the appended token
        const size_t row = (size_t)b * sc.Hq + (size_t)g * G + n;
#pragma unroll
        for (int r = 0; r < NR; ++r)
          direct_o[row * D + lane + 64 * r] = o[n][r] * sc.v_scale;
        if (lane == 0) {
          direct_ml[row * 2 + 0] = m[n];
          direct_ml[row * 2 + 1] = l[n];
        }
      } else if (!split) {
        const float inv = l[n] > 0.f ? sc.v_scale / l[n] : 0.f;
        float* orow = out + ((size_t)b * sc.Hq + (size_t)g * G + n) * D;
#pragma unroll
        for (int r = 0; r < NR; ++r) orow[lane + 64 * r] = o[n][r] * inv;
      } else {
        const int slot = Sb < u0 ? 0 : 1;
        const size_t row = ((size_t)w * 2 + slot) * G + n;
#pragma unroll
        for (int r = 0; r < NR; ++r)
          part_o[row * D + lane + 64 * r] = o[n][r] * sc.v_scale;
        if (lane == 0) {
          part_ml[row * 2 + 0] = m[n];
          part_ml[row * 2 + 1] = l[n];
        }
      }
    }
  });
}

template <int D>
void launch_one(const DecodeArgs& a, int nwg, hipStream_t stream) {
  hipExtLaunchKernelGGL(decode_valu_kernel<D>, dim3(nwg), dim3(64), 0, stream,
                        a.ev_start, a.ev_stop, 0,
                        reinterpret_cast<const float*>(a.q),
                     reinterpret_cast<const float*>(a.k_pool),
                     reinterpret_cast<const float*>(a.v_pool), a.block_tables,
                     a.seq_lens, reinterpret_cast<float*>(a.out), a.prefix,
                     a.part_ml, a.part_o, a.direct_ml, a.direct_o, a.s);
}

template <int D>
int occupancy_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(decode_valu_kernel<D>), 64, 0) !=
      hipSuccess)
    return 0;
  return n;
}

}  // namespace

int occupancy_decode_valu(int head_size) {
  switch (head_size) {
    case 64: return occupancy_one<64>();
    case 128: return occupancy_one<128>();
    case 256: return occupancy_one<256>();
  }
  return 0;
}

hipError_t launch_decode_valu(int head_size, const DecodeArgs& a, int nwg,
                              hipStream_t stream) {
  switch (head_size) {
    case 64: launch_one<64>(a, nwg, stream); break;
    case 128: launch_one<128>(a, nwg, stream); break;
    case 256: launch_one<256>(a, nwg, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
