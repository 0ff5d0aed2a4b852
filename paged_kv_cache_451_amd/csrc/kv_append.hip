// KV append: each new token's K row goes to its slot's row of the K tile
// ([16][D] per block and KV head) and its V values to the slot's column of
// the V tile ([D][16]); a byte copy, or, for the quantising append, bf16
// values divided by their tensor's scale and stored as fp8 e4m3fn codes.
//
// One workgroup per (group of kGroup = 16 consecutive tokens, KV head).  A
// thread item is one 16-byte chunk of a token's input row for that head:
// its values go to one row of the K tile (a contiguous store) or to VPI rows
// of the V tile, one element each.  K items are laid out chunk-fastest, so a
// wave writes whole K rows; V items token-fastest, so 16 neighbouring lanes
// hold the 16 tokens of the group at the same d: when those tokens fill
// consecutive slots of one block (a prefill chunk), each V store instruction
// writes contiguous 16-element row segments instead of isolated elements.
// Every thread issues all of its chunk loads together with the slot loads,
// so one memory round trip precedes its stores.  K rows are stored
// nontemporally (whole 8- or 16-byte pieces that nothing reads back soon:
// 15% faster on slot runs); V elements are not, since nontemporal partial
// writes of scattered slots measured 8x slower.
#include "pa_launch.h"

namespace pa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 16;  // tokens per workgroup

// Clamp of a float32 value that is not NaN to the e4m3fn range: magnitudes
// above 448 become 448, so the hardware conversion to the nearest e4m3fn
// value (ties to the even code) never overflows.
__device__ __forceinline__ float e4m3fn_clamp(float a) {
  return __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
}

// The IEEE float32 quotient x / scale of a bfloat16 value x (its bits in
// the upper half of `bits`), computed as the float64 product of x with
// rcp = the float64 reciprocal of scale (correctly rounded), rounded to
// float32.  The result is the correctly rounded quotient whenever scale is
// finite and positive.  The product differs from x / scale by a relative
// error below 2^-52 (two float64 roundings).  x has at most 8 significant
// bits and scale at most 24, so x / scale is either a float32 value itself
// or lies at relative distance at least about 2^-49 from every midpoint
// between neighbouring float32 values: for a midpoint M, x - M * scale is
// zero or a non-zero multiple of the lower of the last bits of x and of
// M * scale (a product of at most 25 + 24 bits).  No midpoint therefore
// separates the product from the exact quotient, and both round to the
// same float32 value.  Every intermediate stays in the normal float64
// range for all float32 x and scale.
__device__ __forceinline__ float bf16_quotient(uint32_t bits, double rcp) {
  return (float)((double)__uint_as_float(bits) * rcp);
}

// Non-zero when one of the two bfloat16 values in w is a NaN (bit 15 for
// the low value, bit 31 for the high one): adding 0x7F to a half's
// magnitude carries into its top bit exactly when the magnitude exceeds
// 0x7F80 (exponent all ones, mantissa non-zero).
__device__ __forceinline__ uint32_t bf16_nan_bits(uint32_t w) {
  return ((w & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u;
}

// Stored values of one 16-byte input chunk: a copy (TI = TO) ...
template <typename TI, typename TO>
struct Chunk {
  static constexpr int N = 16 / (int)sizeof(TI);
  TO v[N];
  __device__ __forceinline__ Chunk(const u32x4& raw, double) {
    __builtin_memcpy(v, &raw, sizeof(raw));
  }
  __device__ __forceinline__ TO elem(int e) const { return v[e]; }
};

// ... or the e4m3fn codes of 8 bfloat16 values divided by their scale
// (rcp: the float64 reciprocal of the scale), value e in byte e of the two
// words, a NaN stored as 0x7F.
template <>
struct Chunk<uint16_t, uint8_t> {
  u32x2 w;
  __device__ __forceinline__ Chunk(const u32x4& raw, double rcp) {
    uint32_t nan = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t lo = raw[2 * i], hi = raw[2 * i + 1];
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(
          e4m3fn_clamp(bf16_quotient(lo << 16, rcp)),
          e4m3fn_clamp(bf16_quotient(lo & 0xFFFF0000u, rcp)), 0, false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(
          e4m3fn_clamp(bf16_quotient(hi << 16, rcp)),
          e4m3fn_clamp(bf16_quotient(hi & 0xFFFF0000u, rcp)), c, true);
      w[i] = (uint32_t)c;
      nan |= bf16_nan_bits(lo) | bf16_nan_bits(hi);
    }
    if (nan) {  // rare: recode the NaNs
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t m0 = bf16_nan_bits(raw[2 * i]);
        const uint32_t m1 = bf16_nan_bits(raw[2 * i + 1]);
        const uint32_t mask = ((m0 >> 15) & 1u) * 0x000000FFu |
                              (m0 >> 31) * 0x0000FF00u |
                              ((m1 >> 15) & 1u) * 0x00FF0000u |
                              (m1 >> 31) * 0xFF000000u;
        w[i] = (w[i] & ~mask) | (0x7F7F7F7Fu & mask);
      }
    }
  }
  __device__ __forceinline__ uint8_t elem(int e) const {
    return (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
  }
};

template <typename TI, typename TO, int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const TI* __restrict__ k_new, const TI* __restrict__ v_new,
    const int32_t* __restrict__ slots, TO* __restrict__ k_pool,
    TO* __restrict__ v_pool, int n, int hkv, int num_blocks, double k_rcp,
    double v_rcp) {
  constexpr int VPI = 16 / (int)sizeof(TI);  // values per input chunk
  constexpr int CPR = D / VPI;               // chunks per row and head
  constexpr int ITEMS = kGroup * CPR;        // K items (and V items)
  constexpr int NI = (2 * ITEMS + kAppendThreads - 1) / kAppendThreads;
  const int g = (int)(blockIdx.x % (unsigned)hkv);
  const int t0 = (int)(blockIdx.x / (unsigned)hkv) * kGroup;

  int tok[NI], col[NI], slot[NI];
  bool is_v[NI], live[NI];
  u32x4 raw[NI];
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    const int it = (int)threadIdx.x + r * kAppendThreads;
    is_v[r] = it >= ITEMS;
    const int j = is_v[r] ? it - ITEMS : it;
    const int tt = is_v[r] ? j % kGroup : j / CPR;
    col[r] = is_v[r] ? j / kGroup : j % CPR;
    tok[r] = t0 + tt;
    live[r] = it < 2 * ITEMS && tok[r] < n;
    const TI* src = is_v[r] ? v_new : k_new;
    const size_t at = ((size_t)tok[r] * hkv + g) * D + (size_t)col[r] * VPI;
    raw[r] = live[r] ? *reinterpret_cast<const u32x4*>(src + at) : u32x4{};
    slot[r] = live[r] ? slots[tok[r]] : -1;
  }
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    if (!live[r] || slot[r] < 0 || slot[r] >= num_blocks * kBlock) continue;
    const Chunk<TI, TO> ch(raw[r], is_v[r] ? v_rcp : k_rcp);
    const int off = slot[r] & (kBlock - 1);
    const size_t tile = ((size_t)(slot[r] >> 4) * hkv + g) * kBlock * D;
    const int e0 = col[r] * VPI;
    if (!is_v[r]) {
      TO* kp = k_pool + tile + (size_t)off * D + e0;
      if constexpr (sizeof(TI) != sizeof(TO))
        __builtin_nontemporal_store(ch.w, reinterpret_cast<u32x2*>(kp));
      else
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ch.v),
                                    reinterpret_cast<u32x4*>(kp));
    } else {
      TO* vp = v_pool + tile + (size_t)e0 * kBlock + off;
#pragma unroll
      for (int e = 0; e < VPI; ++e) vp[e * kBlock] = ch.elem(e);
    }
  }
}

template <typename TI, typename TO>
hipError_t launch_t(const void* k_new, const void* v_new, const int32_t* slots,
                    void* k_pool, void* v_pool, int n, int hkv, int d, int nb,
                    float k_scale, float v_scale, hipStream_t stream) {
  const dim3 grid((unsigned)append_workgroups(n, hkv));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kAppendThreads), 0, stream,
                       reinterpret_cast<const TI*>(k_new),
                       reinterpret_cast<const TI*>(v_new), slots,
                       reinterpret_cast<TO*>(k_pool),
                       reinterpret_cast<TO*>(v_pool), n, hkv, nb,
                       1.0 / (double)k_scale, 1.0 / (double)v_scale);
  };
  switch (d) {
    case 64: go(kv_append_kernel<TI, TO, 64>); break;
    case 128: go(kv_append_kernel<TI, TO, 128>); break;
    case 256: go(kv_append_kernel<TI, TO, 256>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t append_workgroups(int64_t num_tokens, int num_kv_heads) {
  return (num_tokens + kGroup - 1) / kGroup * num_kv_heads;
}

hipError_t launch_kv_append_quant(const void* k_new, const void* v_new,
                                  const int32_t* slots, void* k_pool,
                                  void* v_pool, int num_tokens,
                                  int num_kv_heads, int head_size,
                                  int num_blocks, float k_scale,
                                  float v_scale, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  return launch_t<uint16_t, uint8_t>(k_new, v_new, slots, k_pool, v_pool,
                                     num_tokens, num_kv_heads, head_size,
                                     num_blocks, k_scale, v_scale, stream);
}

hipError_t launch_kv_append(int elem_bytes, const void* k_new,
                            const void* v_new, const int32_t* slots,
                            void* k_pool, void* v_pool, int num_tokens,
                            int num_kv_heads, int head_size, int num_blocks,
                            hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  switch (elem_bytes) {
    case 1:
      return launch_t<uint8_t, uint8_t>(k_new, v_new, slots, k_pool, v_pool,
                                        num_tokens, num_kv_heads, head_size,
                                        num_blocks, 1.f, 1.f, stream);
    case 2:
      return launch_t<uint16_t, uint16_t>(k_new, v_new, slots, k_pool, v_pool,
                                          num_tokens, num_kv_heads, head_size,
                                          num_blocks, 1.f, 1.f, stream);
    case 4:
      return launch_t<uint32_t, uint32_t>(k_new, v_new, slots, k_pool, v_pool,
                                          num_tokens, num_kv_heads, head_size,
                                          num_blocks, 1.f, 1.f, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
