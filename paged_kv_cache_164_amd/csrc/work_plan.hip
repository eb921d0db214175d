// Work plan of the decode kernels: the list of work items, one per (token range, sequences).
//
// A dense grid of B * partitions slots would be mostly empty when context lengths are skewed,
// and launching the empty slots costs dispatcher time that the real ones wait for.  Instead,
// one workgroup lists the non-empty items and the attention grid takes them in list order
// (workgroup t: item t / num_kv_heads).  Each range of tokens [s, e) is cut into whole
// partitions of P tokens, and what remains after the last whole partition into chunks of at
// most Q = P / 2 tokens (whole blocks).  The list holds every whole partition first, then the
// chunks from the longest to the shortest (eight size classes): the last items to start are
// the shortest, so the end of the kernel drains quickly (longest-processing-time-first order).
//
// Shared prefixes (optional): group g holds the sequences [s0, s1) = [starts[g], starts[g+1])
// whose first `pre` tokens sit in the same physical blocks (beams or samples of one prompt,
// PagedAttention's block sharing).  The prefix range [0, pre) gets items that carry up to
// `per_item` members at once (their query rows become the columns of one item), so each shared
// block is read once per item rather than once per member; each member's own range [pre, L)
// gets items of its own.  pre = min(prefix_lens[g], every member's length), rounded down to a
// multiple of the block size; a one-member group has pre = 0.  Without groups every sequence is
// a group of its own.
//
// A sequence's partial-result slots are numbered in token order: its prefix items, then its own.
// np_of[b] counts them; a sequence with one item (np_of <= 1) gets its output directly, and a
// sequence of length 0 gets one empty item, which writes the zero output.  Group bounds are
// clamped into [0, num_seqs], and at most `capacity` items are written, so a malformed group
// list cannot make the call address out of bounds.
//
// Layout in the caller's workspace (see workspace_layout): header[1] = number of items;
// items[i] = (b0, nseq | slot << 8, begin, end).
#include "pkv_cache_write.h"
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_tile_addr.h"

#include <algorithm>

namespace pkv {
namespace {

constexpr int kPlanThreads = 1024;

constexpr int kWavesPerPlan = kPlanThreads / 64;
constexpr int kClasses = 1 + 8;  // whole partitions, then eight chunk size classes

// Exclusive prefix sums over the workgroup of N values per thread, all at once.  On return
// v[k] holds the sum of v[k] over the lower threads, plus the totals of all classes j < k
// (the lists of the classes follow one another), and *total the sum of everything.
// s_wave: [waves][N] shared scratch; s_base: [N + 1].
template <int N>
__device__ void block_exclusive_scan_classes(int (&v)[N], int (*s_wave)[N], int* s_base,
                                             int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int incl[N];
#pragma unroll
  for (int k = 0; k < N; ++k) incl[k] = v[k];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int n = __shfl_up(incl[k], d, 64);
      if (lane >= d) incl[k] += n;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < N; ++k) s_wave[wave][k] = incl[k];
  }
  __syncthreads();
  // Wave 0: lane k (< N) turns class k's wave totals into exclusive wave offsets and finds the
  // class total; a scan over lanes then lays the classes one after another.
  if (wave == 0) {
    int tot = 0;
    if (lane < N) {
      int c[kWavesPerPlan];
#pragma unroll
      for (int w = 0; w < kWavesPerPlan; ++w) c[w] = (w < nwaves) ? s_wave[w][lane] : 0;
#pragma unroll
      for (int w = 0; w < kWavesPerPlan; ++w) {
        if (w < nwaves) s_wave[w][lane] = tot;
        tot += c[w];
      }
    }
    int cls = tot;  // inclusive scan of the class totals over lanes 0..N-1
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int n = __shfl_up(cls, d, 64);
      if (lane >= d) cls += n;
    }
    if (lane < N) s_base[lane] = cls - tot;
    if (lane == N - 1) s_base[N] = cls;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = s_base[k] + s_wave[wave][k] + incl[k] - v[k];
  *total = s_base[N];
}

struct GroupSpan {
  int s0, s1, pre;
};

__device__ __forceinline__ GroupSpan group_span(const DecodeArgs& a, int g, int bs) {
  GroupSpan r;
  if (a.group_starts == nullptr) {
    r.s0 = g;
    r.s1 = g + 1;
    r.pre = 0;
    return r;
  }
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

// Items of a token range: whole partitions, then remainder chunks of at most Q
// (whole_parts, chunk_end, chunk_class: pkv_tile_addr.h).

// Per-thread counters (or next positions) of the item classes.  Classes are selected with
// unrolled compare-and-add, never by a run-time array index, so the counters stay in registers.
struct ClassCounters {
  int v[kClasses];
  __device__ void clear() {
#pragma unroll
    for (int k = 0; k < kClasses; ++k) v[k] = 0;
  }
  __device__ void add(int cls, int n) {
#pragma unroll
    for (int k = 0; k < kClasses; ++k) v[k] += (k == cls) ? n : 0;
  }
  // returns the current value of class cls and advances it
  __device__ int take(int cls) {
    int r = 0;
#pragma unroll
    for (int k = 0; k < kClasses; ++k) {
      r = (k == cls) ? v[k] : r;
      v[k] += (k == cls) ? 1 : 0;
    }
    return r;
  }
};

__device__ __forceinline__ void plan_body(const DecodeArgs& a, int bs, int per_item,
                                          int64_t capacity) {
  __shared__ int s_wave[kWavesPerPlan][kClasses];
  __shared__ int s_base[kClasses + 1];
  const int P = a.partition_size, Q = a.tail_chunk;
  const int ngroups = a.group_starts ? a.num_groups : a.num_seqs;
  if (a.group_starts) {  // sequences outside every group keep a count of 0 (the reduce skips them)
    for (int b = threadIdx.x; b < a.num_seqs; b += blockDim.x) a.np_of[b] = 0;
    __syncthreads();
  }
  // each thread owns a contiguous run of groups
  const int per = (ngroups + blockDim.x - 1) / blockDim.x;
  const int g0 = threadIdx.x * per, g1 = min(ngroups, g0 + per);
  auto len_of = [&](int b) { return min(max(a.context_lens[b], 0), a.len_limit); };

  // pass 1: items per class.  A range [s, e) has (e - s) / P whole partitions and at most two
  // chunks; `mult` copies of it (one per member chunk of a shared prefix).
  ClassCounters c;
  c.clear();
  auto count_range = [&](int s, int e, int mult) {
    const int F = whole_parts(e - s, P);
    c.add(0, F * mult);
    for (int t0 = s + F * P; t0 < e; t0 += Q) c.add(chunk_class(chunk_end(t0, e, Q) - t0, Q), mult);
  };
  for (int g = g0; g < g1; ++g) {
    const GroupSpan sp = group_span(a, g, bs);
    count_range(0, sp.pre, (sp.s1 - sp.s0 + per_item - 1) / per_item);
    for (int b = sp.s0; b < sp.s1; ++b) {
      const int L = len_of(b);
      count_range(sp.pre, L, 1);
      if (L == 0) c.add(kClasses - 1, 1);
    }
  }
  int total;
  block_exclusive_scan_classes(c.v, s_wave, s_base, &total);

  // pass 2: the same items, each at its class's next position, slots in token order
  auto put = [&](int cls, int b0, int nseq, int slot, int begin, int end) {
    const int64_t pos = c.take(cls);
    if (pos < capacity)
      a.items[pos] = make_uint4(uint32_t(b0), uint32_t(nseq) | (uint32_t(slot) << 8),
                                uint32_t(begin), uint32_t(end));
  };
  // Whole partitions take consecutive places of class 0.  A thread writes up to kOwnWhole of
  // them itself; longer runs are queued to its wave, which writes them with all lanes below.
  constexpr int kOwnWhole = 8;
  int q_b0 = 0, q_nseq = 0, q_s = 0, q_slot = 0, q_count = 0;
  int64_t q_pos = 0;
  auto put_range = [&](int b0, int nseq, int s, int e, int slot) {
    const int F = whole_parts(e - s, P);
    const int64_t w0 = c.v[0];
    c.v[0] += F;
    if (F > kOwnWhole && q_count == 0) {  // one queued run per thread (see below)
      q_b0 = b0, q_nseq = nseq, q_s = s, q_slot = slot, q_count = F, q_pos = w0;
      slot += F;
    } else {
      for (int j = 0; j < F; ++j, ++slot) {
        if (w0 + j < capacity)
          a.items[w0 + j] = make_uint4(uint32_t(b0), uint32_t(nseq) | (uint32_t(slot) << 8),
                                       uint32_t(s + j * P), uint32_t(s + (j + 1) * P));
      }
    }
    for (int t0 = s + F * P; t0 < e; t0 += Q, ++slot) {
      const int t1 = chunk_end(t0, e, Q);
      put(chunk_class(t1 - t0, Q), b0, nseq, slot, t0, t1);
    }
    return slot;
  };
  for (int g = g0; g < g1; ++g) {
    const GroupSpan sp = group_span(a, g, bs);
    int npre = 0;
    for (int c0 = sp.s0; c0 < sp.s1; c0 += per_item)
      npre = put_range(c0, min(per_item, sp.s1 - c0), 0, sp.pre, 0);
    for (int b = sp.s0; b < sp.s1; ++b) {
      const int L = len_of(b);
      const int n = put_range(b, 1, sp.pre, L, npre);
      if (L == 0) put(kClasses - 1, b, 1, 0, 0, 0);  // its item writes the zero output
      a.np_of[b] = max(n, 1);
    }
  }
  // the queued runs of whole partitions, one lane's run at a time, 64 items per step
  unsigned long long pending = __ballot(q_count > 0);
  while (pending) {
    const int l = __ffsll(pending) - 1;
    pending &= pending - 1;
    const int b0 = __shfl(q_b0, l, 64), nseq = __shfl(q_nseq, l, 64), s0 = __shfl(q_s, l, 64);
    const int slot0 = __shfl(q_slot, l, 64), F = __shfl(q_count, l, 64);
    const int64_t w0 = __shfl(q_pos, l, 64);
    for (int j = threadIdx.x & 63; j < F; j += 64) {
      if (w0 + j < capacity)
        a.items[w0 + j] = make_uint4(uint32_t(b0), uint32_t(nseq) | (uint32_t(slot0 + j) << 8),
                                     uint32_t(s0 + j * P), uint32_t(s0 + (j + 1) * P));
    }
  }
  if (threadIdx.x == 0) {
    a.queue[0] = 0;
    a.queue[1] = uint32_t(min<int64_t>(total, capacity));
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DecodeArgs a, int bs, int per_item,
                                                            int64_t capacity) {
  plan_body(a, bs, per_item, capacity);
}

// The plan and a decode step's cache write in one launch: workgroup 0 lists the work items,
// workgroup 1 + i writes new token i (cache_write_token).  The two are independent -- the plan
// reads block tables and lengths, the write reads new keys and values and slots -- so the short
// write no longer waits behind the plan, and one launch gap is saved.
template <typename E, bool VEC>
__global__ __launch_bounds__(kPlanThreads) void plan_and_cache_kernel(DecodeArgs a, int bs,
                                                                      int per_item,
                                                                      int64_t capacity,
                                                                      CacheWriteArgs w) {
  if (blockIdx.x == 0) {
    plan_body(a, bs, per_item, capacity);
  } else {
    cache_write_token<E, VEC>(blockIdx.x - 1, static_cast<const E*>(w.key),
                              static_cast<const E*>(w.value), static_cast<E*>(w.key_cache),
                              static_cast<E*>(w.value_cache), w.slot_mapping, w.num_kv_heads,
                              w.head_size, w.block_size, w.num_blocks, w.key_stride,
                              w.value_stride);
  }
}

// The same with the write into an 8-bit cache (cache_write_token_kv8): the new fp16 / bf16 keys
// and values quantised with the cache's scales.
template <class IN, int CODE>
__global__ __launch_bounds__(kPlanThreads) void plan_and_cache_kv8_kernel(
    DecodeArgs a, int bs, int per_item, int64_t capacity, CacheWriteArgs w, float k_scale,
    float v_scale) {
  if (blockIdx.x == 0) {
    plan_body(a, bs, per_item, capacity);
  } else {
    cache_write_token_kv8<IN, CODE>(blockIdx.x - 1, static_cast<const uint16_t*>(w.key),
                                    static_cast<const uint16_t*>(w.value),
                                    static_cast<uint8_t*>(w.key_cache),
                                    static_cast<uint8_t*>(w.value_cache), w.slot_mapping,
                                    w.num_kv_heads, w.head_size, w.block_size, w.num_blocks,
                                    w.key_stride, w.value_stride, k_scale, v_scale);
  }
}

int plan_threads(const DecodeArgs& a) {
  // one thread per group up to 1024 threads, in whole waves
  const int groups = a.group_starts ? a.num_groups : a.num_seqs;
  return (int)std::min<int64_t>(kPlanThreads, std::max<int64_t>(64, (groups + 63) / 64 * 64));
}

}  // namespace

hipError_t launch_plan(const DecodeArgs& a, int block_size, int seqs_per_item, hipStream_t stream) {
  const int64_t capacity = (int64_t)a.num_seqs * a.slots;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(plan_threads(a)), 0, stream, a, block_size,
                     seqs_per_item, capacity);
  return hipGetLastError();
}

hipError_t launch_plan_and_cache(const DecodeArgs& a, int block_size, int seqs_per_item,
                                 const CacheWriteArgs& w, int elem_bytes, hipStream_t stream) {
  const int64_t capacity = (int64_t)a.num_seqs * a.slots;
  const bool vec = (reinterpret_cast<uintptr_t>(w.key) % 16 == 0) &&
                   ((w.key_stride * elem_bytes) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(w.key_cache) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(w.value) % 16 == 0) &&
                   ((w.value_stride * elem_bytes) % 16 == 0);
  const dim3 grid((unsigned)(1 + w.num_tokens)), block(plan_threads(a));
#define PKV_PC(E, V)                                                                           \
  hipLaunchKernelGGL((plan_and_cache_kernel<E, V>), grid, block, 0, stream, a, block_size,     \
                     seqs_per_item, capacity, w)
  if (elem_bytes == 2) {
    if (vec) PKV_PC(uint16_t, true); else PKV_PC(uint16_t, false);
  } else {
    if (vec) PKV_PC(uint32_t, true); else PKV_PC(uint32_t, false);
  }
#undef PKV_PC
  return hipGetLastError();
}

hipError_t launch_plan_and_cache_kv8(const DecodeArgs& a, int block_size, int seqs_per_item,
                                     const CacheWriteArgs& w, int dtype, int code, float k_scale,
                                     float v_scale, hipStream_t stream) {
  const int64_t capacity = (int64_t)a.num_seqs * a.slots;
  const dim3 grid((unsigned)(1 + w.num_tokens)), block(plan_threads(a));
#define PKV_PC8(IN, CODE)                                                                      \
  hipLaunchKernelGGL((plan_and_cache_kv8_kernel<IN, CODE>), grid, block, 0, stream, a,         \
                     block_size, seqs_per_item, capacity, w, k_scale, v_scale)
  if (code == kCodeE4M3) {
    if (dtype == 1) PKV_PC8(F16, kCodeE4M3); else PKV_PC8(BF16, kCodeE4M3);
  } else {
    if (dtype == 1) PKV_PC8(F16, kCodeI8); else PKV_PC8(BF16, kCodeI8);
  }
#undef PKV_PC8
  return hipGetLastError();
}

}  // namespace pkv
