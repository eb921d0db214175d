// Widening of OCP FP8 E4M3 codes (the 8-bit KV cache) to the model's 16-bit type, exactly: every
// E4M3 value is representable in fp16 and bf16.  gfx950's v_cvt_pk_f32_fp8 decodes two codes to
// fp32; bf16 keeps the upper halves (one v_perm), fp16 packs with v_cvt_pkrtz (exact here).
#pragma once

#include "pkv_device.h"

namespace pkv {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two E4M3 codes (byte pair HI of w) as two 16-bit values of the query's type, packed.
template <bool HI>
__device__ __forceinline__ uint32_t widen2(BF16, uint32_t w) {
  const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  // exact values: the upper halves of the two floats are their bf16 encodings
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}
template <bool HI>
__device__ __forceinline__ uint32_t widen2(F16, uint32_t w) {
  const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[0], f[1]));  // exact
}
// Eight codes (8 bytes) as eight 16-bit values: one MFMA operand.
template <class DT>
__device__ __forceinline__ uint4 widen8(uint32_t lo, uint32_t hi) {
  return make_uint4(widen2<false>(DT(), lo), widen2<true>(DT(), lo), widen2<false>(DT(), hi),
                    widen2<true>(DT(), hi));
}

}  // namespace pkv
