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

// Shared-prefix decode.  Group g holds the sequences [s0, s1) = [starts[g], starts[g+1]) whose
// first `pre` tokens sit in the same physical blocks (beams or samples of one prompt).  Its
// prefix is cut into partitions [p P, min((p + 1) P, pre)), each read once for up to
// `per_item` members at a time (their query rows become the columns of one item); each member
// then gets its own items over [pre + j P, min(pre + (j + 1) P, L)).  A member's partial slots
// are its prefix partitions first, then its own: np_of[b] of them in all.
// pre = min(prefix_lens[g], every member's length), rounded down to a multiple of the block size;
// a one-member group has pre = 0.  The group bounds are clamped into [0, num_seqs], and no more
// than `capacity` items are written, so a malformed group list cannot address out of bounds.
struct GroupSpan {
  int s0, s1, pre;
};

__device__ __forceinline__ GroupSpan group_span(const DecodeArgs& a, int g, int bs) {
  GroupSpan r;
  r.s0 = min(max(a.group_starts[g], 0), a.num_seqs);
  r.s1 = min(max(a.group_starts[g + 1], r.s0), a.num_seqs);
  r.pre = 0;
  if (r.s1 - r.s0 >= 2) {
    int pre = min(max(a.prefix_lens[g], 0), a.len_limit);
    for (int b = r.s0; b < r.s1; ++b) pre = min(pre, max(a.context_lens[b], 0));
    r.pre = pre - pre % bs;
  }
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void plan_shared_kernel(DecodeArgs a, int bs,
                                                                   int per_item,
                                                                   int64_t capacity) {
  __shared__ int s_wave[kPlanThreads / 64 + 1];
  const int P = a.partition_size;
  for (int b = threadIdx.x; b < a.num_seqs; b += kPlanThreads) a.np_of[b] = 0;
  __syncthreads();
  // each thread owns a contiguous run of groups
  const int per = (a.num_groups + kPlanThreads - 1) / kPlanThreads;
  const int g0 = threadIdx.x * per, g1 = min(a.num_groups, g0 + per);
  auto len_of = [&](int b) { return min(max(a.context_lens[b], 0), a.len_limit); };
  int nfull = 0, npart = 0;
  for (int g = g0; g < g1; ++g) {
    const GroupSpan sp = group_span(a, g, bs);
    const int chunks = (sp.s1 - sp.s0 + per_item - 1) / per_item;
    nfull += chunks * (sp.pre / P);
    npart += chunks * (sp.pre % P != 0 ? 1 : 0);
    for (int b = sp.s0; b < sp.s1; ++b) {
      const int L = len_of(b), r = L - sp.pre;
      nfull += r / P;
      npart += (r % P != 0 || L == 0) ? 1 : 0;
    }
  }
  int total_full, total_part;
  int64_t fo = block_exclusive_scan(nfull, s_wave, &total_full);
  int64_t po = total_full + block_exclusive_scan(npart, s_wave, &total_part);
  auto put = [&](int64_t& pos, int b0, int nseq, int slot, int begin, int end) {
    if (pos < capacity)
      a.items[pos] = make_uint4(uint32_t(b0), uint32_t(nseq) | (uint32_t(slot) << 8),
                                uint32_t(begin), uint32_t(end));
    ++pos;
  };
  for (int g = g0; g < g1; ++g) {
    const GroupSpan sp = group_span(a, g, bs);
    const int npre = (sp.pre + P - 1) / P;
    for (int c0 = sp.s0; c0 < sp.s1; c0 += per_item) {
      const int n = min(per_item, sp.s1 - c0);
      for (int p = 0; p < npre; ++p) {
        const int begin = p * P, end = min(begin + P, sp.pre);
        put(end - begin == P ? fo : po, c0, n, p, begin, end);
      }
    }
    for (int b = sp.s0; b < sp.s1; ++b) {
      const int L = len_of(b);
      const int npriv = (L - sp.pre + P - 1) / P;
      for (int j = 0; j < npriv; ++j) {
        const int begin = sp.pre + j * P, end = min(begin + P, L);
        put(end - begin == P ? fo : po, b, 1, npre + j, begin, end);
      }
      if (L == 0) put(po, b, 1, 0, 0, 0);  // its item writes the zero output
      a.np_of[b] = max(npre + npriv, 1);
    }
  }
  if (threadIdx.x == 0) {
    a.queue[0] = 0;
    a.queue[1] = uint32_t(min<int64_t>(int64_t(total_full) + total_part, capacity));
  }
}

}  // namespace

hipError_t launch_plan_shared(const DecodeArgs& a, int block_size, int seqs_per_item,
                              hipStream_t stream) {
  const int64_t capacity = (int64_t)a.num_seqs * a.max_partitions;
  hipLaunchKernelGGL(plan_shared_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, block_size,
                     seqs_per_item, capacity);
  return hipGetLastError();
}

hipError_t launch_plan(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.context_lens,
                     a.num_seqs, a.len_limit, a.partition_size, a.queue, a.pairs);
  return hipGetLastError();
}

}  // namespace pkv
