// Measurement aid, kept apart from the attention path's declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
// Non-temporal 16-byte streaming read of `bytes` (probe_stream.hip).
hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream);
}  // namespace pkv
