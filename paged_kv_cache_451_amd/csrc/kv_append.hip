// KV append: each new token's K row goes to its slot's row of the K tile
// ([16][D] per block and KV head) and its V values to the slot's column of
// the V tile ([D][16]).  One workgroup per token; a pure byte copy.
#include "pa_launch.h"

namespace pa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int32_t* __restrict__ slots, T* __restrict__ k_pool,
    T* __restrict__ v_pool, int hkv, int d, int num_blocks) {
  const int i = blockIdx.x;
  const int slot = slots[i];
  if (slot < 0 || slot >= num_blocks * kBlock) return;
  const int phys = slot >> 4;
  const int off = slot & (kBlock - 1);
  const size_t row_elems = (size_t)hkv * d;
  const T* kn = k_new + (size_t)i * row_elems;
  const T* vn = v_new + (size_t)i * row_elems;
  const size_t blk = (size_t)phys * hkv * kBlock * d;

  // K: Hkv rows of D contiguous elements, 16 bytes at a time
  constexpr int kVec = 16 / (int)sizeof(T);
  const int vec_per_row = d / kVec;
  for (int c = threadIdx.x; c < hkv * vec_per_row; c += blockDim.x) {
    const int g = c / vec_per_row;
    const int e = (c % vec_per_row) * kVec;
    const u32x4 v = *reinterpret_cast<const u32x4*>(kn + (size_t)g * d + e);
    *reinterpret_cast<u32x4*>(k_pool + blk + ((size_t)g * kBlock + off) * d +
                              e) = v;
  }
  // V: one element per (head, d), stride 16 elements in the pool
  for (int c = threadIdx.x; c < hkv * d; c += blockDim.x) {
    const int g = c / d;
    const int e = c % d;
    v_pool[blk + ((size_t)g * d + e) * kBlock + off] = vn[c];
  }
}

template <typename T>
void launch_t(const void* k_new, const void* v_new, const int32_t* slots,
              void* k_pool, void* v_pool, int n, int hkv, int d, int nb,
              hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel<T>, dim3(n), dim3(256), 0, stream,
                     reinterpret_cast<const T*>(k_new),
                     reinterpret_cast<const T*>(v_new), slots,
                     reinterpret_cast<T*>(k_pool),
                     reinterpret_cast<T*>(v_pool), hkv, d, nb);
}

}  // namespace

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
