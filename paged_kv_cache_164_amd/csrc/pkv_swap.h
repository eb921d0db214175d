// swap_blocks' kernel path (host-side declarations): whole blocks between the device cache and
// page-locked host memory that the device addresses at the host pointer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

// (src, dst) block ids of one swap_blocks launch, passed by value in the kernel arguments.
constexpr int kSwapPairs = 112;
struct SwapList {
  int64_t src[kSwapPairs];
  int64_t dst[kSwapPairs];
};
// Moves list's first num_pairs blocks of block_bytes (a multiple of 8; both bases 8-byte
// aligned).  The host side must be page-locked memory the device addresses at this pointer.
hipError_t launch_swap_blocks(void* dst, const void* src, const SwapList& list, int num_pairs,
                              int64_t block_bytes, bool to_host, hipStream_t stream);

}  // namespace pkv
