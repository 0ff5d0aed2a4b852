// KV append: each new token's K row goes to its slot's row of the K tile
// ([16][D] per block and KV head) and its V values to the slot's column of
// the V tile ([D][16]).  A pure byte copy.
//
// One thread per 16-byte chunk of a token's K row and one per 16-byte chunk
// of its V row; token i owns workgroups [i * wpt, (i + 1) * wpt).  The chunk
// loads do not depend on the slot, so a thread issues them together with the
// slot load and pays one memory round trip before its stores: a K chunk is one 16-byte store, a V chunk
// becomes 16 / sizeof(T) element stores one V-tile row (16 elements) apart.
#include "pa_launch.h"

namespace pa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int32_t* __restrict__ slots, T* __restrict__ k_pool,
    T* __restrict__ v_pool, int hkv, int d, int num_blocks, int wpt) {
  constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  const int i = blockIdx.x / wpt;
  const int chunks = hkv * d / E;  // chunks of one token's K (or V) row
  int c = (blockIdx.x - i * wpt) * kAppendThreads + threadIdx.x;
  const bool is_v = c >= chunks;
  if (is_v) c -= chunks;
  if (c >= chunks) return;
  const size_t row = (size_t)i * hkv * d + (size_t)c * E;
  const u32x4 val =
      *reinterpret_cast<const u32x4*>((is_v ? v_new : k_new) + row);
  const int slot = slots[i];
  if (slot < 0 || slot >= num_blocks * kBlock) return;
  const int phys = slot >> 4;
  const int off = slot & (kBlock - 1);
  const int g = c * E / d;
  const int e0 = c * E - g * d;
  const size_t tile = ((size_t)phys * hkv + g) * kBlock * d;
  if (!is_v) {
    *reinterpret_cast<u32x4*>(k_pool + tile + (size_t)off * d + e0) = val;
  } else {
    T el[E];
    __builtin_memcpy(el, &val, sizeof(val));
    T* vp = v_pool + tile + (size_t)e0 * kBlock + off;
#pragma unroll
    for (int e = 0; e < E; ++e) vp[e * kBlock] = el[e];
  }
}

// e4m3fn code of a float32 value: the nearest e4m3fn value, ties to the
// even code, magnitudes above 448 saturated to 448, NaN to 0x7F.  Every step
// is exact (power-of-two scalings) except the final round-to-nearest-even
// of rintf, so the code is fully determined by the float32 input.
__device__ __forceinline__ uint32_t e4m3fn_code(float v) {
  if (v != v) return 0x7Fu;
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fminf(fabsf(v), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    // subnormal range, steps of 2^-9; a result of 8 is the smallest normal
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
    const float mant = ldexpf(a, -e);  // in [1, 2)
    // a mantissa that rounds up to 8 carries into the exponent field
    code = ((uint32_t)(e + 7) << 3) + (uint32_t)rintf((mant - 1.f) * 8.f);
  }
  return code | sign;
}

// Quantising append: bf16 rows into an fp8 e4m3fn pool, each value divided
// (IEEE float32 division) by its tensor's scale.  One thread per 8 input
// values (16 bytes in, 8 bytes out), as in kv_append_kernel.
__global__ __launch_bounds__(kAppendThreads) void kv_append_quant_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, int hkv, int d, int num_blocks, int wpt,
    float k_scale, float v_scale) {
  constexpr int E = 8;
  const int i = blockIdx.x / wpt;
  const int chunks = hkv * d / E;
  int c = (blockIdx.x - i * wpt) * kAppendThreads + threadIdx.x;
  const bool is_v = c >= chunks;
  if (is_v) c -= chunks;
  if (c >= chunks) return;
  const size_t row = (size_t)i * hkv * d + (size_t)c * E;
  const u32x4 val =
      *reinterpret_cast<const u32x4*>((is_v ? v_new : k_new) + row);
  const int slot = slots[i];
  if (slot < 0 || slot >= num_blocks * kBlock) return;
  const float scale = is_v ? v_scale : k_scale;
  uint32_t q[E];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    q[2 * w] = e4m3fn_code(__uint_as_float(val[w] << 16) / scale);
    q[2 * w + 1] = e4m3fn_code(__uint_as_float(val[w] & 0xFFFF0000u) / scale);
  }
  const int phys = slot >> 4;
  const int off = slot & (kBlock - 1);
  const int g = c * E / d;
  const int e0 = c * E - g * d;
  const size_t tile = ((size_t)phys * hkv + g) * kBlock * d;
  if (!is_v) {
    uint2 packed;
    packed.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
    packed.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
    *reinterpret_cast<uint2*>(k_pool + tile + (size_t)off * d + e0) = packed;
  } else {
    uint8_t* vp = v_pool + tile + (size_t)e0 * kBlock + off;
#pragma unroll
    for (int e = 0; e < E; ++e) vp[e * kBlock] = (uint8_t)q[e];
  }
}

template <typename T>
void launch_t(const void* k_new, const void* v_new, const int32_t* slots,
              void* k_pool, void* v_pool, int n, int hkv, int d, int nb,
              hipStream_t stream) {
  const int wpt = append_workgroups_per_token((int)sizeof(T), hkv, d);
  hipLaunchKernelGGL(kv_append_kernel<T>, dim3((unsigned)(n * wpt)),
                     dim3(kAppendThreads), 0, stream,
                     reinterpret_cast<const T*>(k_new),
                     reinterpret_cast<const T*>(v_new), slots,
                     reinterpret_cast<T*>(k_pool),
                     reinterpret_cast<T*>(v_pool), hkv, d, nb, wpt);
}

}  // namespace

int append_workgroups_per_token(int elem_bytes, int num_kv_heads,
                                int head_size) {
  const int chunks = num_kv_heads * head_size * elem_bytes / 16;
  return (2 * chunks + kAppendThreads - 1) / kAppendThreads;
}

hipError_t launch_kv_append_quant(const void* k_new, const void* v_new,
                                  const int32_t* slots, void* k_pool,
                                  void* v_pool, int num_tokens,
                                  int num_kv_heads, int head_size,
                                  int num_blocks, float k_scale,
                                  float v_scale, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int wpt = append_workgroups_per_token(2, num_kv_heads, head_size);
  hipLaunchKernelGGL(kv_append_quant_kernel, dim3((unsigned)(num_tokens * wpt)),
                     dim3(kAppendThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(k_new),
                     reinterpret_cast<const uint16_t*>(v_new), slots,
                     reinterpret_cast<uint8_t*>(k_pool),
                     reinterpret_cast<uint8_t*>(v_pool), num_kv_heads,
                     head_size, num_blocks, wpt, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_append(int elem_bytes, const void* k_new,
                            const void* v_new, const int32_t* slots,
                            void* k_pool, void* v_pool, int num_tokens,
                            int num_kv_heads, int head_size, int num_blocks,
                            hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  switch (elem_bytes) {
    case 1:
      launch_t<uint8_t>(k_new, v_new, slots, k_pool, v_pool, num_tokens,
                        num_kv_heads, head_size, num_blocks, stream);
      break;
    case 2:
      launch_t<uint16_t>(k_new, v_new, slots, k_pool, v_pool, num_tokens,
                         num_kv_heads, head_size, num_blocks, stream);
      break;
    case 4:
      launch_t<uint32_t>(k_new, v_new, slots, k_pool, v_pool, num_tokens,
                         num_kv_heads, head_size, num_blocks, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
