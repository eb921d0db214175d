// Measurement aid: the achievable HBM read ceiling for the decode kernels' access type.
// A grid-stride read of a device buffer with the same non-temporal 16-byte loads the decode
// kernels use for the KV cache, sixteen loads in flight per thread; the data is
// folded into a per-thread XOR that is stored only if it matches a value the input cannot be
// known to avoid, so the loads cannot be dropped.
#include <algorithm>

#include "pkv_device.h"
#include "pkv_probe.h"

namespace pkv {
namespace {

constexpr int kStreamUnroll = 16;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src,
                                                          int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    uint4 r[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) r[u] = kv_load<true>(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = kv_load<true>(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  // many short-lived workgroups (up to 32768, a few iterations each) measured fastest: fewer,
  // longer ones leave the memory system under-subscribed (2048: 6.25 vs 7.1 TB/s)
  const int64_t want = (n16 + 256 * kStreamUnroll - 1) / (256 * kStreamUnroll);
  const unsigned grid = (unsigned)std::min<int64_t>(std::max<int64_t>(want, 1), 32768);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace pkv
