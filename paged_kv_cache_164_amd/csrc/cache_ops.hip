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
#include "pkv_cache_write.h"
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_kv8.h"
#include "pkv_kv8_host.h"
#include "pkv_swap.h"

namespace pkv {
namespace {

// One workgroup per new token: cache_write_token (pkv_cache_write.h).
template <typename E, bool VEC>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ key_cache,
    E* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping, int num_kv_heads,
    int head_size, int block_size, int64_t num_blocks, int64_t key_stride, int64_t value_stride) {
  cache_write_token<E, VEC>(blockIdx.x, key, value, key_cache, value_cache, slot_mapping,
                            num_kv_heads, head_size, block_size, num_blocks, key_stride,
                            value_stride);
}

// The same scatter for many tokens (a prefill chunk), 16-bit elements: one workgroup per run
// of 16 consecutive tokens.  A thread holds one (head, dim) value element of 8 tokens, and 8
// tokens whose slots are consecutive, 8-aligned and inside one block -- the usual case for a
// chunk, whose tokens fill blocks in order -- land as one 16-byte store of the value row
// instead of eight 2-byte ones.  Other runs fall back to element stores.  With 16-byte aligned
// value rows (VEC_VAL) the run's values come in through LDS with 16-byte loads and are read
// back transposed; otherwise each thread loads its 8 elements one by one.  Keys are 16-byte
// chunks either way (token index fastest across threads, so a block's consecutive tokens are
// written as one contiguous run).
constexpr int kRunTokens = 16;
constexpr int kRunMinTokens = 512;  // below it, one workgroup per token spreads the work wider

// Values of a run staged through LDS: kValChunk elements of the 16 token rows at a time, read
// with 16-byte loads (rows padded by 8 elements, so that rows 8 apart sit in other banks).
constexpr int kValChunk = 512;
constexpr int kValPitch = kValChunk + 8;

template <bool VEC_KEY, bool VEC_VAL>
__global__ __launch_bounds__(256) void reshape_and_cache_runs_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint16_t* __restrict__ key_cache, uint16_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads, int head_size,
    int block_size, int64_t num_blocks, int64_t key_stride, int64_t value_stride) {
  constexpr int X = 8;  // elements per 16-byte key chunk
  __shared__ int64_t s_slot[kRunTokens];
  __shared__ int s_vec[2];
  const int64_t i0 = (int64_t)blockIdx.x * kRunTokens;
  const int ntok = (int)min<int64_t>(kRunTokens, num_tokens - i0);
  const int tid = threadIdx.x;
  if (tid < kRunTokens) {
    int64_t sl = (tid < ntok) ? slot_mapping[i0 + tid] : -1;
    s_slot[tid] = (sl < 0 || sl >= num_blocks * block_size) ? -1 : sl;  // skipped: -1
  }
  __syncthreads();
  if (tid < 2) {
    const int64_t a = s_slot[8 * tid];
    // the vector store needs every value row 8-element aligned: block_size a multiple of 8
    bool ok = block_size % 8 == 0 && a >= 0 && a % 8 == 0 &&
              slot_offset(a, block_size) + 8 <= block_size;
    for (int k = 1; k < 8; ++k) ok = ok && s_slot[8 * tid + k] == a + k;
    s_vec[tid] = ok;
  }
  __syncthreads();
  const int D = head_size;
  const int n = num_kv_heads * D;
  const int64_t tile = (int64_t)D * block_size;
  for (int t = tid; t < kRunTokens * (n / X); t += blockDim.x) {
    const int j = t % kRunTokens, c = t / kRunTokens;
    const int64_t sl = s_slot[j];
    if (sl < 0) continue;
    const int h = c / (D / X), cc = c % (D / X);
    uint16_t* dst = key_cache + (slot_block(sl, block_size) * num_kv_heads + h) * tile +
                    ((int64_t)cc * block_size + slot_offset(sl, block_size)) * X;
    const uint16_t* src = key + (i0 + j) * key_stride + (int64_t)c * X;
    if constexpr (VEC_KEY) {
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    } else {
      for (int k = 0; k < X; ++k) dst[k] = src[k];
    }
  }
  // values: a thread takes one (head, dim) row and 8 tokens (half = t % 2), so consecutive
  // threads write consecutive 16-byte pieces: a wave's stores cover whole value rows
  auto store_values = [&](int e, int half, const uint32_t (&v)[4]) {
    const int h = e / D, d = e % D;
    const int kb = 8 * half;
    if (s_vec[half]) {
      const int64_t sl = s_slot[kb];
      uint16_t* dst = value_cache + (slot_block(sl, block_size) * num_kv_heads + h) * tile +
                      (int64_t)d * block_size + slot_offset(sl, block_size);
      *reinterpret_cast<uint4*>(dst) = make_uint4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t sl = s_slot[kb + k];
        if (sl < 0) continue;
        value_cache[(slot_block(sl, block_size) * num_kv_heads + h) * tile + (int64_t)d * block_size +
                    slot_offset(sl, block_size)] = uint16_t(v[k / 2] >> (16 * (k & 1)));
      }
    }
  };
  if constexpr (VEC_VAL) {
    __shared__ __align__(16) uint16_t s_val[kRunTokens * kValPitch];
    for (int c0 = 0; c0 < n; c0 += kValChunk) {
      const int pieces = min(kValChunk, n - c0) / 8;
      for (int t = tid; t < kRunTokens * pieces; t += blockDim.x) {
        const int j = t / pieces, q = t % pieces;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (j < ntok) v = *reinterpret_cast<const uint4*>(value + (i0 + j) * value_stride + c0 + q * 8);
        *reinterpret_cast<uint4*>(&s_val[j * kValPitch + q * 8]) = v;
      }
      __syncthreads();
      for (int t = tid; t < 16 * pieces; t += blockDim.x) {
        const int el = t >> 1, half = t & 1;
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          v[k] = uint32_t(s_val[(8 * half + 2 * k) * kValPitch + el]) |
                 (uint32_t(s_val[(8 * half + 2 * k + 1) * kValPitch + el]) << 16);
        store_values(c0 + el, half, v);
      }
      __syncthreads();
    }
  } else {
    for (int t = tid; t < 2 * n; t += blockDim.x) {
      const int e = t >> 1, half = t & 1;
      const int kb = 8 * half;
      uint32_t v[4];
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        const uint32_t lo = (kb + k < ntok) ? value[(i0 + kb + k) * value_stride + e] : 0u;
        const uint32_t hi = (kb + k + 1 < ntok) ? value[(i0 + kb + k + 1) * value_stride + e] : 0u;
        v[k / 2] = lo | (hi << 16);
      }
      store_values(e, half, v);
    }
  }
}

// One workgroup per new token: cache_write_token_kv8 (pkv_cache_write.h).
template <class IN, int CODE>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int num_kv_heads, int head_size, int block_size,
    int64_t num_blocks, int64_t key_stride, int64_t value_stride, float k_scale, float v_scale) {
  cache_write_token_kv8<IN, CODE>(blockIdx.x, key, value, key_cache, value_cache, slot_mapping,
                                  num_kv_heads, head_size, block_size, num_blocks, key_stride,
                                  value_stride, k_scale, v_scale);
}

// The 8-bit write for many tokens: 16 tokens per workgroup, as reshape_and_cache_runs_kernel.
// A run of 8 consecutive tokens landing in 8 consecutive, 8-aligned slots of one block writes
// its codes of a value row as one 8-byte store; other runs fall back to byte stores.  Keys are
// 16-byte chunks (16 codes) either way.  With 16-byte aligned key and value rows (VEC) the new
// elements come in with 16-byte loads (values through LDS, as in the 16-bit run kernel).
// VEC: key and value rows 16-byte aligned (16-byte loads of the new elements).
template <class IN, int CODE, bool VEC>
__global__ __launch_bounds__(256) void reshape_and_cache_kv8_runs_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads, int head_size,
    int block_size, int64_t num_blocks, int64_t key_stride, int64_t value_stride, float k_scale,
    float v_scale) {
  __shared__ int64_t s_slot[kRunTokens];
  __shared__ int s_vec[2];
  const int64_t i0 = (int64_t)blockIdx.x * kRunTokens;
  const int ntok = (int)min<int64_t>(kRunTokens, num_tokens - i0);
  const int tid = threadIdx.x;
  if (tid < kRunTokens) {
    int64_t sl = (tid < ntok) ? slot_mapping[i0 + tid] : -1;
    s_slot[tid] = (sl < 0 || sl >= num_blocks * block_size) ? -1 : sl;  // skipped: -1
  }
  __syncthreads();
  if (tid < 2) {
    const int64_t a = s_slot[8 * tid];
    // the vector store needs every value row 8-element aligned: block_size a multiple of 8
    bool ok = block_size % 8 == 0 && a >= 0 && a % 8 == 0 &&
              slot_offset(a, block_size) + 8 <= block_size;
    for (int k = 1; k < 8; ++k) ok = ok && s_slot[8 * tid + k] == a + k;
    s_vec[tid] = ok;
  }
  __syncthreads();
  const int D = head_size;
  const int n = num_kv_heads * D;
  const int64_t tile = (int64_t)D * block_size;  // bytes of one (block, head) tile
  // keys: one 16-byte chunk (16 dims) of one token per thread, token index fastest; with
  // aligned rows the 16 elements come in as two 16-byte loads
  for (int t = tid; t < kRunTokens * (n / 16); t += blockDim.x) {
    const int j = t % kRunTokens, c = t / kRunTokens;
    const int64_t sl = s_slot[j];
    if (sl < 0) continue;
    const int h = c / (D / 16), cc = c % (D / 16);
    const uint16_t* e = key + (i0 + j) * key_stride + (int64_t)c * 16;
    uint16_t el[16];
    if constexpr (VEC) {
      const uint4 a = reinterpret_cast<const uint4*>(e)[0], b = reinterpret_cast<const uint4*>(e)[1];
      const uint32_t wds[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        el[2 * k] = uint16_t(wds[k] & 0xffffu);
        el[2 * k + 1] = uint16_t(wds[k] >> 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) el[k] = e[k];
    }
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = quant2<CODE>(widen16(IN(), el[4 * k]), widen16(IN(), el[4 * k + 1]), k_scale) |
             (quant2<CODE>(widen16(IN(), el[4 * k + 2]), widen16(IN(), el[4 * k + 3]), k_scale) << 16);
    *reinterpret_cast<uint4*>(key_cache + (slot_block(sl, block_size) * num_kv_heads + h) * tile +
                              ((int64_t)cc * block_size + slot_offset(sl, block_size)) * 16) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
  // values: a thread takes one (head, dim) row and 8 tokens (half = t % 2); x holds the 8
  // elements of the row, tokens past the run 0
  auto store_values = [&](int e, int half, const float (&x)[8]) {
    const int h = e / D, d = e % D;
    const int kb = 8 * half;
    uint32_t v[2];
#pragma unroll
    for (int k = 0; k < 8; k += 4)
      v[k / 4] = quant2<CODE>(x[k], x[k + 1], v_scale) | (quant2<CODE>(x[k + 2], x[k + 3], v_scale) << 16);
    if (s_vec[half]) {
      const int64_t sl = s_slot[kb];
      *reinterpret_cast<uint2*>(value_cache + (slot_block(sl, block_size) * num_kv_heads + h) * tile +
                                (int64_t)d * block_size + slot_offset(sl, block_size)) = make_uint2(v[0], v[1]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t sl = s_slot[kb + k];
        if (sl < 0) continue;
        value_cache[(slot_block(sl, block_size) * num_kv_heads + h) * tile + (int64_t)d * block_size +
                    slot_offset(sl, block_size)] = uint8_t(v[k / 4] >> (8 * (k & 3)));
      }
    }
  };
  if constexpr (VEC) {
    __shared__ __align__(16) uint16_t s_val[kRunTokens * kValPitch];
    for (int c0 = 0; c0 < n; c0 += kValChunk) {
      const int pieces = min(kValChunk, n - c0) / 8;
      for (int t = tid; t < kRunTokens * pieces; t += blockDim.x) {
        const int j = t / pieces, q = t % pieces;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (j < ntok) v = *reinterpret_cast<const uint4*>(value + (i0 + j) * value_stride + c0 + q * 8);
        *reinterpret_cast<uint4*>(&s_val[j * kValPitch + q * 8]) = v;
      }
      __syncthreads();
      for (int t = tid; t < 16 * pieces; t += blockDim.x) {
        const int el = t >> 1, half = t & 1;
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = widen16(IN(), s_val[(8 * half + k) * kValPitch + el]);
        store_values(c0 + el, half, x);
      }
      __syncthreads();
    }
  } else {
    for (int t = tid; t < 2 * n; t += blockDim.x) {
      const int e = t >> 1, half = t & 1;
      const int kb = 8 * half;
      float x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        x[k] = (kb + k < ntok) ? widen16(IN(), value[(i0 + kb + k) * value_stride + e]) : 0.f;
      store_values(e, half, x);
    }
  }
}

constexpr int kCopyThreads = 256;
constexpr int64_t kCopyChunk16 = kCopyThreads * 8;  // 16-byte words per workgroup (32 KiB)
constexpr int64_t kSwapChunk8 = kCopyThreads * 16;  // 8-byte words per workgroup (32 KiB)

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

// swap_blocks: whole blocks between the device cache and page-locked host memory that the device
// addresses directly (CacheEngine swap_in / swap_out).  One launch moves up to kSwapPairs blocks;
// the pair list travels in the kernel arguments, so nothing is allocated.  The host side is read
// and written with system-scope relaxed 8-byte atomics (coherent with the host whatever the
// allocation's coherence flag); the lanes of a wave touch 512 contiguous bytes per access, whole
// lines, on both sides.
template <bool TO_HOST>
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    unsigned char* __restrict__ dst, const unsigned char* __restrict__ src, SwapList list,
    int64_t block_bytes, int chunks_per_block) {
  const int pair = blockIdx.x / chunks_per_block;
  const int chunk = blockIdx.x % chunks_per_block;
  const int64_t n8 = block_bytes / 8;
  const int64_t lo = chunk * kSwapChunk8;
  const int64_t hi = min(n8, lo + kSwapChunk8);
  const uint64_t* s = reinterpret_cast<const uint64_t*>(src + list.src[pair] * block_bytes);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst + list.dst[pair] * block_bytes);
  constexpr int U = 8;  // 8-byte words in flight per thread
  for (int64_t k0 = lo + threadIdx.x; k0 < hi; k0 += U * kCopyThreads) {
    uint64_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u * kCopyThreads;
      if (k < hi) {
        if constexpr (TO_HOST) w[u] = s[k];
        else w[u] = __hip_atomic_load(s + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u * kCopyThreads;
      if (k < hi) {
        if constexpr (TO_HOST) __hip_atomic_store(d + k, w[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        else d[k] = w[u];
      }
    }
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
  // many 16-bit tokens: the run kernel (its 16-byte value stores need an aligned cache)
  if (elem_bytes == 2 && num_tokens >= kRunMinTokens &&
      reinterpret_cast<uintptr_t>(value_cache) % 16 == 0) {
    const dim3 rgrid((unsigned)((num_tokens + kRunTokens - 1) / kRunTokens));
    const bool vec_val = (reinterpret_cast<uintptr_t>(value) % 16 == 0) && (value_stride % 8 == 0);
#define PKV_RUNS(V, W)                                                                          \
  hipLaunchKernelGGL((reshape_and_cache_runs_kernel<V, W>), rgrid, dim3(256), 0, stream,        \
                     static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),    \
                     static_cast<uint16_t*>(key_cache), static_cast<uint16_t*>(value_cache),    \
                     slot_mapping, num_tokens, num_kv_heads, head_size, block_size, num_blocks, \
                     key_stride, value_stride)
    if (vec) {
      if (vec_val) PKV_RUNS(true, true); else PKV_RUNS(true, false);
    } else {
      if (vec_val) PKV_RUNS(false, true); else PKV_RUNS(false, false);
    }
#undef PKV_RUNS
    return hipGetLastError();
  }
  const bool vec_both = vec && (reinterpret_cast<uintptr_t>(value) % 16 == 0) &&
                        ((value_stride * elem_bytes) % 16 == 0);
  const dim3 grid(num_tokens), block(256);
#define PKV_RC(E, V)                                                                          \
  hipLaunchKernelGGL((reshape_and_cache_kernel<E, V>), grid, block, 0, stream,                \
                     static_cast<const E*>(key), static_cast<const E*>(value),                \
                     static_cast<E*>(key_cache), static_cast<E*>(value_cache), slot_mapping, \
                     num_kv_heads, head_size, block_size, num_blocks, key_stride, value_stride)
  if (elem_bytes == 2) {
    if (vec_both) PKV_RC(uint16_t, true); else PKV_RC(uint16_t, false);
  } else {
    if (vec_both) PKV_RC(uint32_t, true); else PKV_RC(uint32_t, false);
  }
#undef PKV_RC
  return hipGetLastError();
}

template <int CODE>
hipError_t launch_rc8(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int num_tokens, int num_kv_heads, int head_size,
                      int block_size, int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                      int dtype, float k_scale, float v_scale, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  // many tokens: the run kernel (its 8-byte value stores need an 8-byte aligned cache)
  if (num_tokens >= kRunMinTokens && reinterpret_cast<uintptr_t>(value_cache) % 8 == 0) {
    const dim3 rgrid((unsigned)((num_tokens + kRunTokens - 1) / kRunTokens));
    const bool vec_rows = (reinterpret_cast<uintptr_t>(value) % 16 == 0) && (value_stride % 8 == 0) &&
                          (reinterpret_cast<uintptr_t>(key) % 16 == 0) && (key_stride % 8 == 0);
#define PKV_RUNS8(IN, W)                                                                        \
  hipLaunchKernelGGL((reshape_and_cache_kv8_runs_kernel<IN, CODE, W>), rgrid, dim3(256), 0,     \
                     stream, static_cast<const uint16_t*>(key),                                 \
                     static_cast<const uint16_t*>(value), static_cast<uint8_t*>(key_cache),     \
                     static_cast<uint8_t*>(value_cache), slot_mapping, num_tokens,              \
                     num_kv_heads, head_size, block_size, num_blocks, key_stride,               \
                     value_stride, k_scale, v_scale)
    if (vec_rows) {
      if (dtype == 1) PKV_RUNS8(F16, true); else PKV_RUNS8(BF16, true);
    } else {
      if (dtype == 1) PKV_RUNS8(F16, false); else PKV_RUNS8(BF16, false);
    }
#undef PKV_RUNS8
    return hipGetLastError();
  }
  const dim3 grid(num_tokens), block(256);
#define PKV_RC8(IN)                                                                             \
  hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<IN, CODE>), grid, block, 0, stream,          \
                     static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),    \
                     static_cast<uint8_t*>(key_cache), static_cast<uint8_t*>(value_cache),      \
                     slot_mapping, num_kv_heads, head_size, block_size, num_blocks, key_stride, \
                     value_stride, k_scale, v_scale)
  if (dtype == 1) PKV_RC8(F16); else PKV_RC8(BF16);
#undef PKV_RC8
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                        void* value_cache, const int64_t* slot_mapping,
                                        int num_tokens, int num_kv_heads, int head_size,
                                        int block_size, int64_t num_blocks, int64_t key_stride,
                                        int64_t value_stride, int dtype, float k_scale,
                                        float v_scale, hipStream_t stream) {
  return launch_rc8<kCodeE4M3>(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                               num_kv_heads, head_size, block_size, num_blocks, key_stride,
                               value_stride, dtype, k_scale, v_scale, stream);
}

hipError_t launch_reshape_and_cache_i8(const void* key, const void* value, void* key_cache,
                                       void* value_cache, const int64_t* slot_mapping,
                                       int num_tokens, int num_kv_heads, int head_size,
                                       int block_size, int64_t num_blocks, int64_t key_stride,
                                       int64_t value_stride, int dtype, float k_scale,
                                       float v_scale, hipStream_t stream) {
  return launch_rc8<kCodeI8>(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                             num_kv_heads, head_size, block_size, num_blocks, key_stride,
                             value_stride, dtype, k_scale, v_scale, stream);
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

hipError_t launch_swap_blocks(void* dst, const void* src, const SwapList& list, int num_pairs,
                              int64_t block_bytes, bool to_host, hipStream_t stream) {
  if (num_pairs <= 0) return hipSuccess;
  const int64_t chunks = (block_bytes / 8 + kSwapChunk8 - 1) / kSwapChunk8;
  const dim3 grid((unsigned)(num_pairs * chunks));
  auto* d = static_cast<unsigned char*>(dst);
  auto* s = static_cast<const unsigned char*>(src);
  if (to_host)
    hipLaunchKernelGGL(swap_blocks_kernel<true>, grid, dim3(kCopyThreads), 0, stream, d, s, list,
                       block_bytes, (int)chunks);
  else
    hipLaunchKernelGGL(swap_blocks_kernel<false>, grid, dim3(kCopyThreads), 0, stream, d, s, list,
                       block_bytes, (int)chunks);
  return hipGetLastError();
}

}  // namespace pkv
