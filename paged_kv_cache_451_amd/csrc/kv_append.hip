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

// e4m3fn codes of two float32 values (low byte: a): the nearest e4m3fn
// value, ties to the even code, magnitudes above 448 saturated to 448, NaN
// to 0x7F.  The magnitude is clamped to 448 first, so the hardware
// conversion (round to nearest even) never overflows.
__device__ __forceinline__ uint32_t e4m3fn_pair(float a, float b) {
  const float ca = fminf(fmaxf(a, -448.f), 448.f);
  const float cb = fminf(fmaxf(b, -448.f), 448.f);
  uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  if (a != a) c = (c & 0xFF00u) | 0x7Fu;
  if (b != b) c = (c & 0x00FFu) | 0x7F00u;
  return c & 0xFFFFu;
}

// Stored values of one 16-byte input chunk: a copy (TI = TO) or the
// e4m3fn codes of bf16 values divided by `scale` (IEEE float32 division).
template <typename TI, typename TO>
struct Chunk {
  static constexpr int N = 16 / (int)sizeof(TI);
  TO v[N];
  __device__ __forceinline__ Chunk(const u32x4& raw, float scale) {
    if constexpr (sizeof(TI) == sizeof(TO)) {
      (void)scale;
      __builtin_memcpy(v, &raw, sizeof(raw));
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t c = e4m3fn_pair(__uint_as_float(raw[w] << 16) / scale,
                                       __uint_as_float(raw[w] & 0xFFFF0000u) /
                                           scale);
        v[2 * w] = (TO)(c & 0xFFu);
        v[2 * w + 1] = (TO)(c >> 8);
      }
    }
  }
};

template <typename TI, typename TO, int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const TI* __restrict__ k_new, const TI* __restrict__ v_new,
    const int32_t* __restrict__ slots, TO* __restrict__ k_pool,
    TO* __restrict__ v_pool, int n, int hkv, int num_blocks, float k_scale,
    float v_scale) {
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
    const Chunk<TI, TO> ch(raw[r], is_v[r] ? v_scale : k_scale);
    const int off = slot[r] & (kBlock - 1);
    const size_t tile = ((size_t)(slot[r] >> 4) * hkv + g) * kBlock * D;
    const int e0 = col[r] * VPI;
    if (!is_v[r]) {
      TO* kp = k_pool + tile + (size_t)off * D + e0;
      if constexpr (VPI * sizeof(TO) == 16)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ch.v),
                                    reinterpret_cast<u32x4*>(kp));
      else
        __builtin_nontemporal_store(*reinterpret_cast<const u32x2*>(ch.v),
                                    reinterpret_cast<u32x2*>(kp));
    } else {
      TO* vp = v_pool + tile + (size_t)e0 * kBlock + off;
#pragma unroll
      for (int e = 0; e < VPI; ++e) vp[e * kBlock] = ch.v[e];
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
                       reinterpret_cast<TO*>(v_pool), n, hkv, nb, k_scale,
                       v_scale);
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
