// Work plan of the decode kernels: the list of (sequence, partition) pairs that hold tokens.
//
// The grid of a paged decode over B sequences with up to NP_max partitions each has
// B * NP_max slots, most of them empty when context lengths are skewed; launching the empty
// ones costs dispatcher time that the real ones wait for.  Instead, one workgroup lists the
// non-empty pairs and persistent workers pull them from a queue.  Order of the list: every
// full partition first (sequence-major), then each sequence's partial last partition, so the
// shortest items run last and the end of the kernel drains quickly.  A sequence of length 0
// gets one (empty) partial item: its worker writes the zero output.
//
// Layout in the caller's workspace (see workspace_layout): header[0] = queue counter (reset
// here), header[1] = number of pairs; pairs[i] = b * kMaxPartitions + p.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kPlanThreads = 1024;

// Exclusive prefix sum of one value per thread over the workgroup; returns the total in *total.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(incl, d, 64);
    if (lane >= d) incl += n;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = (lane < kPlanThreads / 64) ? s_wave[lane] : 0;
    int wi = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int n = __shfl_up(wi, d, 64);
      if (lane >= d) wi += n;
    }
    if (lane < kPlanThreads / 64) s_wave[lane] = wi - w;  // exclusive wave offsets
    if (lane == kPlanThreads / 64 - 1) s_wave[kPlanThreads / 64] = wi;
  }
  __syncthreads();
  const int r = s_wave[wave] + incl - v;
  *total = s_wave[kPlanThreads / 64];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ context_lens,
                                                            int num_seqs, int len_limit, int P,
                                                            uint32_t* __restrict__ header,
                                                            uint32_t* __restrict__ pairs) {
  __shared__ int s_wave[kPlanThreads / 64 + 1];
  // each thread owns a contiguous run of sequences
  const int per = (num_seqs + kPlanThreads - 1) / kPlanThreads;
  const int b0 = threadIdx.x * per, b1 = min(num_seqs, b0 + per);
  int nfull = 0, npart = 0;
  for (int b = b0; b < b1; ++b) {
    const int L = min(max(context_lens[b], 0), len_limit);
    nfull += L / P;
    npart += (L % P != 0 || L == 0) ? 1 : 0;
  }
  int total_full, total_part;
  int fo = block_exclusive_scan(nfull, s_wave, &total_full);
  int po = total_full + block_exclusive_scan(npart, s_wave, &total_part);
  for (int b = b0; b < b1; ++b) {
    const int L = min(max(context_lens[b], 0), len_limit);
    const int F = L / P;
    for (int p = 0; p < F; ++p) pairs[fo++] = uint32_t(b) * kMaxPartitions + p;
    if (L % P != 0 || L == 0) pairs[po++] = uint32_t(b) * kMaxPartitions + F;
  }
  if (threadIdx.x == 0) {
    header[0] = 0;  // queue counter
    header[1] = uint32_t(total_full + total_part);
  }
}

}  // namespace

hipError_t launch_plan(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.context_lens,
                     a.num_seqs, a.len_limit, a.partition_size, a.queue, a.pairs);
  return hipGetLastError();
}

}  // namespace pkv
