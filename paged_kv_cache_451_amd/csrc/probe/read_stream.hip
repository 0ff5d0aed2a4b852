// Practical HBM read ceiling of the GPU: a plain nontemporal read stream
// over one contiguous buffer, with no indirection and no math.  It is the
// measuring stick the decode kernels' bandwidth is reported against, next
// to the published peak (decode attention is memory-bound: "vLLM
// innenfra", continuous-batching paragraph).  Not part of the paged path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLanes = 64;   // one wave per workgroup
constexpr int kUnroll = 16;  // 16-byte loads in flight per lane (16 KiB/wave)

// Workgroup w streams the contiguous chunk [w * chunk, (w + 1) * chunk) of
// 16-byte units: each iteration issues kUnroll loads per lane (lane l reads
// units i + 64u + l, so each load instruction covers 1 KiB of contiguous
// memory) before any is used.  The folded value is stored only if it equals
// a constant no real data is expected to produce, so the loads cannot be
// removed and nothing is written in practice.
__global__ __launch_bounds__(kLanes) void read_stream_kernel(
    const u32x4* __restrict__ p, size_t n16, size_t chunk,
    uint32_t* __restrict__ sink) {
  const size_t begin = (size_t)blockIdx.x * chunk;
  const size_t end = begin + chunk < n16 ? begin + chunk : n16;
  size_t i = begin + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * kLanes < end; i += kUnroll * kLanes) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_nontemporal_load(p + i + u * kLanes);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < end; i += kLanes) acc ^= __builtin_nontemporal_load(p + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

extern "C" int pa_probe_read_stream(const void* buf, size_t bytes,
                                    uint32_t* sink, int workgroups,
                                    void* stream) {
  if (!buf || !sink || workgroups < 1) return -1;
  if (((uintptr_t)buf & 15u) || (bytes & 15u)) return -4;
  const size_t n16 = bytes / 16;
  const size_t step = (size_t)kUnroll * kLanes;
  const size_t per = (n16 + workgroups - 1) / workgroups;
  const size_t chunk = (per + step - 1) / step * step;
  hipLaunchKernelGGL(read_stream_kernel, dim3(workgroups), dim3(kLanes), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), n16, chunk, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
