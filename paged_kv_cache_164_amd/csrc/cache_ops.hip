// KV-cache maintenance kernels: the slot scatter of new tokens and the block copy.
//
// reshape_and_cache: the KV-cache write of the cybasar.com nano-vLLM article
// (section 5.2.3) in the block layout of the "Vllm" page ("CacheEngine"):
// slot -> (block = slot / block_size, offset = slot % block_size); a key row
// lands as 16-byte chunks key_cache[block][h][c][offset][0:x], a value row
// element by element in value_cache[block][h][d][offset].
//
// copy_blocks: CacheEngine "copy" -- whole key and value blocks, every layer,
// for each (src, dst) copy-on-write pair.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <typename E, bool VEC_KEY>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ key_cache,
    E* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping, int num_kv_heads,
    int head_size, int block_size, int64_t num_blocks, int64_t key_stride, int64_t value_stride) {
  constexpr int X = 16 / sizeof(E);
  const int64_t i = blockIdx.x;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_blocks * block_size) return;
  const int64_t blk = slot / block_size;
  const int off = static_cast<int>(slot % block_size);
  const int D = head_size;
  const int n = num_kv_heads * D;
  const int64_t tile = (int64_t)D * block_size;  // elements of one (block, head) tile
  E* kdst = key_cache + blk * num_kv_heads * tile;
  E* vdst = value_cache + blk * num_kv_heads * tile;
  const E* krow = key + i * key_stride;
  const E* vrow = value + i * value_stride;
  if constexpr (VEC_KEY) {
    const int chunks_per_head = D / X;
    for (int c = threadIdx.x; c < n / X; c += blockDim.x) {
      const int h = c / chunks_per_head, cc = c % chunks_per_head;
      *reinterpret_cast<uint4*>(kdst + h * tile + ((int64_t)cc * block_size + off) * X) =
          *reinterpret_cast<const uint4*>(krow + (int64_t)c * X);
    }
  } else {
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
      const int h = e / D, d = e % D;
      kdst[h * tile + ((int64_t)(d / X) * block_size + off) * X + d % X] = krow[e];
    }
  }
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int h = e / D, d = e % D;
    vdst[h * tile + (int64_t)d * block_size + off] = vrow[e];
  }
}

constexpr int kCopyThreads = 256;
constexpr int64_t kCopyChunk16 = kCopyThreads * 8;  // 16-byte words per workgroup (32 KiB)

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const uint64_t* __restrict__ key_ptrs, const uint64_t* __restrict__ value_ptrs,
    const int64_t* __restrict__ mapping, int64_t block_bytes, int64_t num_blocks,
    int chunks_per_block) {
  const int pair = blockIdx.x / chunks_per_block;
  const int chunk = blockIdx.x % chunks_per_block;
  const int layer = blockIdx.y;
  const int64_t src = mapping[2 * (int64_t)pair];
  const int64_t dst = mapping[2 * (int64_t)pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint64_t base = (blockIdx.z == 0 ? key_ptrs : value_ptrs)[layer];
  const int64_t n16 = block_bytes / 16;
  const int64_t lo = chunk * kCopyChunk16;
  const int64_t hi = min(n16, lo + kCopyChunk16);
  if ((base & 15u) == 0) {
    const uint4* s = reinterpret_cast<const uint4*>(base + src * block_bytes);
    uint4* d = reinterpret_cast<uint4*>(base + dst * block_bytes);
    for (int64_t k = lo + threadIdx.x; k < hi; k += kCopyThreads) d[k] = s[k];
  } else {
    const unsigned char* s = reinterpret_cast<const unsigned char*>(base + src * block_bytes);
    unsigned char* d = reinterpret_cast<unsigned char*>(base + dst * block_bytes);
    for (int64_t k = lo * 16 + threadIdx.x; k < hi * 16; k += kCopyThreads) d[k] = s[k];
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping, int num_tokens,
                                    int num_kv_heads, int head_size, int block_size,
                                    int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                                    int elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const bool vec = (reinterpret_cast<uintptr_t>(key) % 16 == 0) &&
                   ((key_stride * elem_bytes) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(key_cache) % 16 == 0);
  const dim3 grid(num_tokens), block(256);
#define PKV_RC(E, V)                                                                          \
  hipLaunchKernelGGL((reshape_and_cache_kernel<E, V>), grid, block, 0, stream,                \
                     static_cast<const E*>(key), static_cast<const E*>(value),                \
                     static_cast<E*>(key_cache), static_cast<E*>(value_cache), slot_mapping, \
                     num_kv_heads, head_size, block_size, num_blocks, key_stride, value_stride)
  if (elem_bytes == 2) {
    if (vec) PKV_RC(uint16_t, true); else PKV_RC(uint16_t, false);
  } else {
    if (vec) PKV_RC(uint32_t, true); else PKV_RC(uint32_t, false);
  }
#undef PKV_RC
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const uint64_t* key_ptrs, const uint64_t* value_ptrs, int num_layers,
                              const int64_t* mapping, int num_pairs, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream) {
  if (num_pairs == 0 || num_layers == 0) return hipSuccess;
  const int64_t chunks = (block_bytes / 16 + kCopyChunk16 - 1) / kCopyChunk16;
  const dim3 grid((unsigned)(num_pairs * chunks), (unsigned)num_layers, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, key_ptrs, value_ptrs,
                     mapping, block_bytes, num_blocks, (int)chunks);
  return hipGetLastError();
}

}  // namespace pkv
