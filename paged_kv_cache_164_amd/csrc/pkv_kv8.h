// Widening of the 8-bit KV cache's codes to the model's 16-bit type, exactly: every E4M3 value
// and every integer code -128 .. 127 is representable in fp16 and bf16.
//   E4M3: gfx950's v_cvt_pk_f32_fp8 decodes two codes to fp32; bf16 keeps the upper halves
//         (one v_perm), fp16 packs with v_cvt_pkrtz (exact here).
//   INT8 (two's-complement bytes): bf16 via fp32 (sign-extended byte, convert, upper half);
//         fp16 by placing the biased byte b = code + 128 in the mantissa of 1024 (fp16 0x6400
//         | b is 1024 + b) and subtracting 1152 in one packed fp16 add.
#pragma once

#include "pkv_device.h"
#include "pkv_kv8_host.h"

namespace pkv {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two codes (byte pair HI of w) as two 16-bit values of the query's type, packed.
template <int CODE, bool HI>
__device__ __forceinline__ uint32_t widen2(BF16, uint32_t w) {
  if constexpr (CODE == kCodeE4M3) {
    const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    // exact values: the upper halves of the two floats are their bf16 encodings
    return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
  } else {
    const float f0 = static_cast<float>(static_cast<int8_t>(w >> (HI ? 16 : 0)));
    const float f1 = static_cast<float>(static_cast<int8_t>(w >> (HI ? 24 : 8)));
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
}
template <int CODE, bool HI>
__device__ __forceinline__ uint32_t widen2(F16, uint32_t w) {
  if constexpr (CODE == kCodeE4M3) {
    const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[0], f[1]));  // exact
  } else {
    // [b0 | 0x64, b1 | 0x64] of the biased bytes, i.e. fp16 (1024 + b0, 1024 + b1)
    const uint32_t biased = w ^ 0x80808080u;
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, biased, HI ? 0x04030402u : 0x04010400u);
    const f16x2_t v = __builtin_bit_cast(f16x2_t, h) - f16x2_t{(_Float16)1152.f, (_Float16)1152.f};
    return __builtin_bit_cast(uint32_t, v);
  }
}
// Eight codes (8 bytes) as eight 16-bit values: one MFMA operand.
template <class DT, int CODE = kCodeE4M3>
__device__ __forceinline__ uint4 widen8(uint32_t lo, uint32_t hi) {
  return make_uint4(widen2<CODE, false>(DT(), lo), widen2<CODE, true>(DT(), lo),
                    widen2<CODE, false>(DT(), hi), widen2<CODE, true>(DT(), hi));
}

}  // namespace pkv
