// Host-side launchers of the INT8 form of the 8-bit KV cache (the E4M3 forms are declared with
// the other kernels).  Shapes and scales are validated by the caller.
#pragma once

#include "pkv_internal.h"

namespace pkv {

// Code formats of an 8-bit cache (0 stands for a 16-bit cache).
constexpr int kCodeE4M3 = 1;  // OCP FP8 E4M3
constexpr int kCodeI8 = 2;    // signed integers -127 .. 127 (two's-complement bytes)

// Decode over INT8 codes; arguments as for launch_decode_fp8.
hipError_t launch_decode_i8(const DecodeArgs& a, int dtype, int head_size, int block_size,
                            int group, hipStream_t stream);
// Cache write quantising to INT8 codes; arguments as for launch_reshape_and_cache_fp8.
hipError_t launch_reshape_and_cache_i8(const void* key, const void* value, void* key_cache,
                                       void* value_cache, const int64_t* slot_mapping,
                                       int num_tokens, int num_kv_heads, int head_size,
                                       int block_size, int64_t num_blocks, int64_t key_stride,
                                       int64_t value_stride, int dtype, float k_scale,
                                       float v_scale, hipStream_t stream);

}  // namespace pkv
