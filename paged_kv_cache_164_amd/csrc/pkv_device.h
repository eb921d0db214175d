// Device-side helpers shared by the pkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Element-type tags.  X = elements per 16-byte chunk (16 / sizeof).
struct F32 {
  static constexpr int X = 4;
  static constexpr int kBytes = 4;
};
struct F16 {
  static constexpr int X = 8;
  static constexpr int kBytes = 2;
};
struct BF16 {
  static constexpr int X = 8;
  static constexpr int kBytes = 2;
};

// Unpack one 16-byte chunk into X floats (exact widening).
__device__ __forceinline__ void unpack(F32, const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack2_f16(uint32_t u, float* f) {
  half2_t h = __builtin_bit_cast(half2_t, u);
  f[0] = static_cast<float>(h[0]);
  f[1] = static_cast<float>(h[1]);
}
__device__ __forceinline__ void unpack(F16, const uint4& v, float* f) {
  unpack2_f16(v.x, f + 0);
  unpack2_f16(v.y, f + 2);
  unpack2_f16(v.z, f + 4);
  unpack2_f16(v.w, f + 6);
}
// bf16 is the upper half of an IEEE binary32: shifting it into place is exact.
__device__ __forceinline__ void unpack2_bf16(uint32_t u, float* f) {
  f[0] = __uint_as_float(u << 16);
  f[1] = __uint_as_float(u & 0xffff0000u);
}
__device__ __forceinline__ void unpack(BF16, const uint4& v, float* f) {
  unpack2_bf16(v.x, f + 0);
  unpack2_bf16(v.y, f + 2);
  unpack2_bf16(v.z, f + 4);
  unpack2_bf16(v.w, f + 6);
}

// Two floats to two packed 16-bit elements, round to nearest even (one v_cvt_pk_* on gfx950).
typedef float pkv_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pkv_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 pkv_f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(BF16, float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((pkv_f32x2{x, y}), pkv_bf16x2));
}
__device__ __forceinline__ uint32_t pack2(F16, float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((pkv_f32x2{x, y}), pkv_f16x2));
}
// Two packed ones of the element type (an all-ones MFMA operand turns a product into row sums).
__device__ __forceinline__ uint32_t one_bits(BF16) { return 0x3f803f80u; }
__device__ __forceinline__ uint32_t one_bits(F16) { return 0x3c003c00u; }

// Online softmax with a lazy maximum (log2 units): a column's running maximum moves, and its
// accumulators are rescaled, only when a tile's maximum exceeds it by more than this margin, so
// weights stay below 2^8 and most tiles skip the rescale.
constexpr float kLazyRescale = 8.f;

// Round-to-nearest-even narrowing stores.
__device__ __forceinline__ void store_elem(F32, void* base, int64_t i, float v) {
  static_cast<float*>(base)[i] = v;
}
__device__ __forceinline__ void store_elem(F16, void* base, int64_t i, float v) {
  static_cast<_Float16*>(base)[i] = static_cast<_Float16>(v);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ void store_elem(BF16, void* base, int64_t i, float v) {
  static_cast<uint16_t*>(base)[i] = f32_to_bf16_rne(v);
}

// Butterfly reductions across lanes whose ids differ in the bits of [lo, 64).
template <int LO>
__device__ __forceinline__ float xor_sum_from(float v) {
#pragma unroll
  for (int m = LO; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
template <int HI>
__device__ __forceinline__ float xor_sum_below(float v) {
#pragma unroll
  for (int m = 1; m < HI; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Loads of KV-cache data.  Each context token's keys and values are read once per decode
// call, so STREAM = true issues them non-temporal: they then do not displace the small, reused
// data (work list, block tables, queries) from the caches, and the dependent loads that start a
// work item keep hitting in L2 instead of queueing behind the stream at HBM.
template <bool STREAM>
__device__ __forceinline__ uint4 kv_load(const uint4* p) {
  if constexpr (STREAM) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *p;
  }
}
template <bool STREAM>
__device__ __forceinline__ uint2 kv_load(const uint2* p) {
  if constexpr (STREAM) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v[0], v[1]);
  } else {
    return *p;
  }
}

}  // namespace pkv
