// The per-token KV-cache writes of reshape_and_cache and its 8-bit forms (cache_ops.hip), as
// device functions that a kernel runs in one of its workgroups: the slot scatter of the
// cybasar.com nano-vLLM article (section 5.2.3) in the block layout of the "Vllm" page
// ("CacheEngine").
#pragma once

#include "pkv_device.h"
#include "pkv_kv8_host.h"

namespace pkv {

// A valid (non-negative) slot's block and offset: shift and mask for a power-of-two block size
// (every size the attention kernels take), a 64-bit division otherwise.
__device__ inline int64_t slot_block(int64_t slot, int block_size) {
  if ((block_size & (block_size - 1)) == 0)
    return slot >> __builtin_ctz(static_cast<unsigned>(block_size));
  return slot / block_size;
}
__device__ inline int slot_offset(int64_t slot, int block_size) {
  if ((block_size & (block_size - 1)) == 0) return static_cast<int>(slot & (block_size - 1));
  return static_cast<int>(slot % block_size);
}

// Token i's key and value rows, written by one workgroup.  VEC (16-byte aligned rows and key
// cache): a thread takes 16-byte chunks of the key row and of the value row, all its loads in
// flight together; a key chunk is one 16-byte store, a value chunk X element stores down the
// value rows.  Otherwise element by element.
template <typename E, bool VEC>
__device__ __forceinline__ void cache_write_token(
    int64_t i, const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ key_cache,
    E* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping, int num_kv_heads,
    int head_size, int block_size, int64_t num_blocks, int64_t key_stride, int64_t value_stride) {
  constexpr int X = 16 / sizeof(E);
  const int D = head_size;
  const int n = num_kv_heads * D;
  const int64_t tile = (int64_t)D * block_size;  // elements of one (block, head) tile
  const E* krow = key + i * key_stride;
  const E* vrow = value + i * value_stride;
  if constexpr (VEC) {
    const int nc = n / X, cph = D / X;
    const uint4* k4 = reinterpret_cast<const uint4*>(krow);
    const uint4* v4 = reinterpret_cast<const uint4*>(vrow);
    // the first two chunks per thread (a whole row of up to 2 blockDim.x chunks) without a
    // branch: indices past the row are clamped to its last chunk and their values dropped
    const int c0 = threadIdx.x, c1 = c0 + blockDim.x;
    const int l0 = min(c0, nc - 1), l1 = min(c1, nc - 1);
    const uint4 ka = k4[l0], va = v4[l0], kb = k4[l1], vb = v4[l1];
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * block_size) return;
    const int64_t blk = slot_block(slot, block_size);
    const int off = slot_offset(slot, block_size);
    E* kdst = key_cache + blk * num_kv_heads * tile;
    E* vdst = value_cache + blk * num_kv_heads * tile;
    auto put = [&](int c, const uint4& kq, const uint4& vq) {
      const int h = c / cph, cc = c % cph;
      *reinterpret_cast<uint4*>(kdst + h * tile + ((int64_t)cc * block_size + off) * X) = kq;
      const E* ve = reinterpret_cast<const E*>(&vq);
      E* vd = vdst + h * tile + (int64_t)(cc * X) * block_size + off;
#pragma unroll
      for (int e = 0; e < X; ++e) vd[(int64_t)e * block_size] = ve[e];
    };
    if (c0 < nc) put(c0, ka, va);
    if (c1 < nc) put(c1, kb, vb);
    for (int c = c0 + 2 * blockDim.x; c < nc; c += blockDim.x) put(c, k4[c], v4[c]);
  } else {
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * block_size) return;
    const int64_t blk = slot_block(slot, block_size);
    const int off = slot_offset(slot, block_size);
    E* kdst = key_cache + blk * num_kv_heads * tile;
    E* vdst = value_cache + blk * num_kv_heads * tile;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
      const int h = e / D, d = e % D;
      kdst[h * tile + ((int64_t)(d / X) * block_size + off) * X + d % X] = krow[e];
    }
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
      const int h = e / D, d = e % D;
      vdst[h * tile + (int64_t)d * block_size + off] = vrow[e];
    }
  }
}

// The same scatter into an 8-bit cache (x = 16): each new element of the model's 16-bit type is
// quantised with its cache's scale, the division x / scale rounded to float32, then
//   E4M3: code = E4M3(clamp(x / scale, -448, 448)), to nearest, ties to even (NaN stays NaN);
//   INT8: code = clamp(x / scale, -127, 127) rounded to the nearest integer, ties to even
//         (NaN gives 0).
__device__ __forceinline__ float widen16(F16, uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ float widen16(BF16, uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float to_e4m3_range(float x, float scale) {
  const float y = __fdiv_rn(x, scale);
  return (y != y) ? y : fminf(fmaxf(y, -448.f), 448.f);
}
__device__ __forceinline__ uint32_t to_i8(float x, float scale) {
  const float y = __fdiv_rn(x, scale);
  if (y != y) return 0u;
  return uint32_t(static_cast<int>(rintf(fminf(fmaxf(y, -127.f), 127.f)))) & 0xffu;
}
// two codes, in the low 16 bits (byte 0 = first)
template <int CODE>
__device__ __forceinline__ uint32_t quant2(float x0, float x1, float scale) {
  if constexpr (CODE == kCodeE4M3)
    return __builtin_amdgcn_cvt_pk_fp8_f32(to_e4m3_range(x0, scale), to_e4m3_range(x1, scale), 0,
                                           false) & 0xffffu;
  else
    return to_i8(x0, scale) | (to_i8(x1, scale) << 8);
}

// Token i's key and value rows into an 8-bit cache, written by one workgroup.
template <class IN, int CODE>
__device__ __forceinline__ void cache_write_token_kv8(
    int64_t i, const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int num_kv_heads, int head_size, int block_size,
    int64_t num_blocks, int64_t key_stride, int64_t value_stride, float k_scale, float v_scale) {
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_blocks * block_size) return;
  const int64_t blk = slot_block(slot, block_size);
  const int off = slot_offset(slot, block_size);
  const int D = head_size;
  const int n = num_kv_heads * D;
  const int64_t tile = (int64_t)D * block_size;  // bytes of one (block, head) tile
  uint8_t* kdst = key_cache + blk * num_kv_heads * tile;
  uint8_t* vdst = value_cache + blk * num_kv_heads * tile;
  const uint16_t* krow = key + i * key_stride;
  const uint16_t* vrow = value + i * value_stride;
  // keys: one 16-byte chunk (16 dims) per thread
  const int chunks_per_head = D / 16;
  for (int c = threadIdx.x; c < n / 16; c += blockDim.x) {
    const int h = c / chunks_per_head, cc = c % chunks_per_head;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t* e = krow + (int64_t)c * 16 + 4 * k;
      w[k] = quant2<CODE>(widen16(IN(), e[0]), widen16(IN(), e[1]), k_scale) |
             (quant2<CODE>(widen16(IN(), e[2]), widen16(IN(), e[3]), k_scale) << 16);
    }
    *reinterpret_cast<uint4*>(kdst + h * tile + ((int64_t)cc * block_size + off) * 16) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
  // values: one byte per element, two elements per conversion
  for (int e = 2 * threadIdx.x; e < n; e += 2 * blockDim.x) {
    const uint32_t q = quant2<CODE>(widen16(IN(), vrow[e]), widen16(IN(), vrow[e + 1]), v_scale);
    const int h = e / D, d = e % D;
    vdst[h * tile + (int64_t)d * block_size + off] = uint8_t(q & 0xff);
    vdst[h * tile + (int64_t)(d + 1) * block_size + off] = uint8_t(q >> 8);
  }
}

}  // namespace pkv
