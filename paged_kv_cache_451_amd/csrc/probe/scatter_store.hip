// The store pattern of a KV append on its own: for each new token and KV
// head, the D isolated stores of its V column into the [D][16] tile of its
// slot's block (one element per 16-token row; the pages' block holds K and
// V for 16 tokens: "vLLM innenfra", KV-cache-manager paragraph), with no
// loads of the new rows and no K rows.  Threads map to (token, 8-element
// chunk of the column) with tokens fastest, 16 tokens and one KV head per
// workgroup, as the append does, so that the append's rate on scattered
// slots can be read against what its V stores alone cost.  Not part of the
// paged path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 16;  // tokens per workgroup
constexpr int kBlk = 16;  // tokens per block

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void scatter_v_kernel(
    T* __restrict__ v_pool, const int32_t* __restrict__ slots, int n, int hkv,
    int num_blocks) {
  constexpr int CPR = D / 8;  // 8-element chunks of a V column
  constexpr int ITEMS = kTok * CPR;
  const int g = (int)(blockIdx.x % (unsigned)hkv);
  const int t0 = (int)(blockIdx.x / (unsigned)hkv) * kTok;
  for (int it = (int)threadIdx.x; it < ITEMS; it += kThreads) {
    const int tok = t0 + it % kTok, col = it / kTok;
    if (tok >= n) continue;
    const int slot = slots[tok];
    if (slot < 0 || slot >= num_blocks * kBlk) continue;
    T* vp = v_pool + ((size_t)(slot >> 4) * hkv + g) * kBlk * D +
            (size_t)col * 8 * kBlk + (slot & (kBlk - 1));
#pragma unroll
    for (int e = 0; e < 8; ++e) vp[e * kBlk] = (T)(0x38 + e);
  }
}

template <typename T>
int launch(void* v_pool, const int32_t* slots, int n, int hkv, int d,
           int num_blocks, hipStream_t stream) {
  const dim3 grid((unsigned)(((int64_t)n + kTok - 1) / kTok * hkv));
  T* vp = static_cast<T*>(v_pool);
  switch (d) {
    case 64:
      hipLaunchKernelGGL((scatter_v_kernel<T, 64>), grid, dim3(kThreads), 0,
                         stream, vp, slots, n, hkv, num_blocks);
      break;
    case 128:
      hipLaunchKernelGGL((scatter_v_kernel<T, 128>), grid, dim3(kThreads), 0,
                         stream, vp, slots, n, hkv, num_blocks);
      break;
    default:
      hipLaunchKernelGGL((scatter_v_kernel<T, 256>), grid, dim3(kThreads), 0,
                         stream, vp, slots, n, hkv, num_blocks);
      break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace

extern "C" int pa_probe_scatter_v_store(void* v_pool, const int32_t* slots,
                                        int n, int num_kv_heads,
                                        int head_size, int num_blocks,
                                        int elem_bytes, void* stream) {
  if (!v_pool || !slots || n < 0 || num_kv_heads < 1 || num_blocks < 1)
    return -1;
  if (head_size != 64 && head_size != 128 && head_size != 256) return -2;
  if (elem_bytes != 1 && elem_bytes != 2) return -2;
  if ((int64_t)num_blocks * kBlk > INT32_MAX ||
      ((int64_t)n + kTok - 1) / kTok * num_kv_heads > INT32_MAX)
    return -1;
  if (n == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return elem_bytes == 2
             ? launch<uint16_t>(v_pool, slots, n, num_kv_heads, head_size,
                                num_blocks, s)
             : launch<uint8_t>(v_pool, slots, n, num_kv_heads, head_size,
                               num_blocks, s);
}
