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
//   max/sum reductions of the online softmax (xor 16 and xor 32).
//
// The softmax is the usual online one in base 2: scores are scaled by
// scale*log2(e) (times k_scale for fp8), a running max m and sum l are kept
// per head and the accumulator is rescaled when m grows.  P is rounded to
// bf16 for the matrix core; l sums the rounded values, so the weights used
// for V sum exactly to the normaliser.  fp8 e4m3fn codes widen exactly to
// bf16 (v_cvt_pk_f32_fp8 then v_cvt_pk_bf16_f32); k_scale is folded into the
// score scale and v_scale into the output.
//
// Masking: tokens at or past seq_len, the second block of a pair that lies
// outside the range, and out-of-range block ids contribute nothing: their
// scores become -inf and their V values are zeroed in registers, so NaN or
// stale bytes in unused slots never reach the result.  Such blocks are read
// from a valid block address (the pair's first block, or block 0).
#include <math.h>

#include "pa_launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 fp8 e4m3fn codes (little-endian bytes of w) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  bf16x8 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], true);
    r[4 * h + 0] = (__bf16)lo[0];
    r[4 * h + 1] = (__bf16)lo[1];
    r[4 * h + 2] = (__bf16)hi[0];
    r[4 * h + 3] = (__bf16)hi[1];
  }
  return r;
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

// Storage-type specific loads.  For bf16 a K row chunk for MFMA c is the 8
// values at d = 32c + 8j; for fp8 one 16-byte load at d = 64c' + 16j feeds
// MFMAs 2c' (low 8 bytes) and 2c'+1 (high 8 bytes).  Q uses the same d sets.
template <bool FP8>
struct Kv;

template <>
struct Kv<false> {
  typedef __bf16 T;
  static constexpr int kColJ = 8;  // element offset of k-group j in a row
  __device__ static __forceinline__ int qcol(int c, int j) {
    return 32 * c + 8 * j;
  }
  template <int D>
  __device__ static __forceinline__ void load_k(const T* p, bf16x8* k) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      k[c] = *reinterpret_cast<const bf16x8*>(p + 32 * c);
  }
  template <int D>
  __device__ static __forceinline__ void load_v(const T* p, bf16x8* v) {
#pragma unroll
    for (int x = 0; x < D / 16; ++x)
      v[x] = *reinterpret_cast<const bf16x8*>(p + 256 * x);
  }
};

template <>
struct Kv<true> {
  typedef uint8_t T;
  static constexpr int kColJ = 16;
  __device__ static __forceinline__ int qcol(int c, int j) {
    return 64 * (c >> 1) + 16 * j + 8 * (c & 1);
  }
  template <int D>
  __device__ static __forceinline__ void load_k(const T* p, bf16x8* k) {
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      u32x4 w = *reinterpret_cast<const u32x4*>(p + 64 * c);
      k[2 * c] = fp8x8_to_bf16(u32x2{w[0], w[1]});
      k[2 * c + 1] = fp8x8_to_bf16(u32x2{w[2], w[3]});
    }
  }
  template <int D>
  __device__ static __forceinline__ void load_v(const T* p, bf16x8* v) {
#pragma unroll
    for (int x = 0; x < D / 16; ++x)
      v[x] = fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(p + 256 * x));
  }
};

template <bool FP8, int D>
__global__ __launch_bounds__(64) void decode_mfma_kernel(DecodeArgs a) {
  typedef Kv<FP8> KV;
  typedef typename KV::T T;
  constexpr int NC = D / 32;  // QK MFMAs per 16 tokens
  constexpr int NX = D / 16;  // PV MFMAs (16-row tiles of d)

  const SplitArgs& s = a.s;
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int j = lane >> 4;
  const int w = blockIdx.x;
  const int g = w % s.Hkv;
  const int k = w / s.Hkv;
  const int G = s.G;

  const int U = total_blocks(s, w == 0);
  const int u0 = range_begin(k, U, s.Wh);
  const int u1 = range_begin(k + 1, U, s.Wh);
  if (u0 >= u1) return;

  const T* kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* vpool = reinterpret_cast<const T*>(a.v_pool);
  const size_t tile = (size_t)kBlock * D;  // elements of one (block, head) tile
  // lane-constant parts of the K and V addresses
  const int k_lane = (((r16 >> 2) & 1) * 8 + (r16 & 3)) * D + KV::kColJ * j;
  const int v_lane = r16 * kBlock + 8 * (j & 1);
  const bool k_hi = r16 >= 8;  // K row from the pair's second block
  const bool v_hi = j >= 2;    // V tokens from the pair's second block

  for_each_segment(s, u0, u1, [&](int b, int Sb, int Sb1) {
    const int L = clamped_len(s, b);
    const int lo = (Sb > u0 ? Sb : u0) - Sb;
    const int hi = (Sb1 < u1 ? Sb1 : u1) - Sb;
    const int32_t* trow = s.block_tables + (size_t)b * s.max_blocks;

    // Q as the B operand of QK: lane (n, j) holds head g*G + n.
    bf16x8 qb[NC];
    {
      const int n = r16;
      const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) +
                           ((size_t)b * a.Hq + (size_t)g * G + n) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 z = {};
        qb[c] = n < G ? *reinterpret_cast<const bf16x8*>(qrow + KV::qcol(c, j))
                      : z;
      }
    }

    f32x4 acc[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float lsum = 0.f;

    for (int blk = lo; blk < hi; blk += 2) {
      const bool has1 = blk + 1 < hi;
      int p0 = trow[blk];
      int p1 = has1 ? trow[blk + 1] : p0;
      int nv0 = (unsigned)p0 < (unsigned)a.NB ? L - blk * kBlock : 0;
      int nv1 = has1 && (unsigned)p1 < (unsigned)a.NB
                    ? L - (blk + 1) * kBlock : 0;
      nv0 = nv0 > kBlock ? kBlock : nv0;
      nv1 = nv1 > kBlock ? kBlock : (nv1 < 0 ? 0 : nv1);
      if ((unsigned)p0 >= (unsigned)a.NB) p0 = 0;
      if ((unsigned)p1 >= (unsigned)a.NB) p1 = p0;

      const size_t base0 = ((size_t)p0 * s.Hkv + g) * tile;
      const size_t base1 = ((size_t)p1 * s.Hkv + g) * tile;
      const T* kl = kpool + (k_hi ? base1 : base0) + k_lane;
      const T* vl = vpool + (v_hi ? base1 : base0) + v_lane;

      bf16x8 kr0[NC], kr1[NC], vr[NX];
      KV::template load_k<D>(kl, kr0);
      KV::template load_k<D>(kl + 4 * D, kr1);
      KV::template load_v<D>(vl, vr);

      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        s0 = mfma16x16x32(kr0[c], qb[c], s0);
        s1 = mfma16x16x32(kr1[c], qb[c], s1);
      }

      // this lane's 8 tokens: 8*(j%2) + e of block j/2
      const int nvb = v_hi ? nv1 : nv0;
      int nv = nvb - 8 * (j & 1);
      nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = s0[i] * a.c_log2;
        x[4 + i] = s1[i] * a.c_log2;
      }
      if (nv0 + nv1 < 2 * kBlock) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = e < nv ? x[e] : -INFINITY;
#pragma unroll
        for (int xx = 0; xx < NX; ++xx) vr[xx] = keep_first(vr[xx], nv);
      }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      bf16x8 pb;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 pe = (__bf16)fast_exp2(x[e] - m_use);
        pb[e] = pe;
        psum += (float)pe;
      }
      lsum = lsum * alpha + psum;
      m = m_new;
#pragma unroll
      for (int xx = 0; xx < NX; ++xx) {
        acc[xx] *= alpha;
        acc[xx] = mfma16x16x32(vr[xx], pb, acc[xx]);
      }
    }

    // lane (n, j) holds O[head n][16X + 4j + i]
    float ltot = lsum + __shfl_xor(lsum, 16, kWave);
    ltot += __shfl_xor(ltot, 32, kWave);
    const int n = r16;
    if (n < G) {
      const bool split = Sb < u0 || Sb1 > u1;
      if (!split) {
        const float inv = ltot > 0.f ? a.v_scale / ltot : 0.f;
        __bf16* orow = reinterpret_cast<__bf16*>(a.out) +
                       ((size_t)b * a.Hq + (size_t)g * G + n) * D + 4 * j;
#pragma unroll
        for (int xx = 0; xx < NX; ++xx) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[xx][i] * inv);
          *reinterpret_cast<bf16x4*>(orow + 16 * xx) = o;
        }
      } else {
        const int slot = Sb < u0 ? 0 : 1;
        const size_t row = ((size_t)w * 2 + slot) * G + n;
        float* po = s.part_o + row * D + 4 * j;
#pragma unroll
        for (int xx = 0; xx < NX; ++xx)
          *reinterpret_cast<f32x4*>(po + 16 * xx) = acc[xx] * a.v_scale;
        if (j == 0) {
          s.part_ml[row * 2 + 0] = m;
          s.part_ml[row * 2 + 1] = ltot;
        }
      }
    }
  });
}

template <bool FP8>
hipError_t launch_d(int head_size, const DecodeArgs& a, int nwg,
                    hipStream_t stream) {
  switch (head_size) {
    case 64:
      hipLaunchKernelGGL((decode_mfma_kernel<FP8, 64>), dim3(nwg), dim3(64),
                         0, stream, a);
      break;
    case 128:
      hipLaunchKernelGGL((decode_mfma_kernel<FP8, 128>), dim3(nwg), dim3(64),
                         0, stream, a);
      break;
    case 256:
      hipLaunchKernelGGL((decode_mfma_kernel<FP8, 256>), dim3(nwg), dim3(64),
                         0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(bool fp8, int head_size, const DecodeArgs& a,
                              int nwg, hipStream_t stream) {
  return fp8 ? launch_d<true>(head_size, a, nwg, stream)
             : launch_d<false>(head_size, a, nwg, stream);
}

}  // namespace pa
