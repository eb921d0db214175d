// Host-side declarations shared by the pkv translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kDefaultPartition = 1024;  // partition_size 0 ("auto")
constexpr int kMaxPartitions = 8192;      // per sequence; a work item packs b * kMaxPartitions + p
constexpr int kMaxPlanSeqs = 1 << 19;     // sequences addressable by a packed work item
constexpr int kMaxPartition = 1024;
constexpr int kThreads = 256;  // every attention workgroup: 4 wave64s
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;  // logits are kept in base-2 units

// Everything the attention kernels need, resolved on the host.
struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint32_t* queue;  // [2]: (reserved, number of work items), written by the plan kernel
  uint32_t* pairs;  // [num_seqs * max_partitions] work items b * kMaxPartitions + p
  const char* prefetch_pad;  // kPrefetchPad bytes read by prefetches past a work item's end
  // Shared-prefix decode only (null / 0 otherwise):
  const int32_t* group_starts;  // [num_groups + 1] sequences of group g: [starts[g], starts[g+1])
  const int32_t* prefix_lens;   // [num_groups] tokens shared by the members of a group
  int num_groups;
  uint4* items;    // [num_seqs * max_partitions] work items (b0, nseq | slot << 8, begin, end)
  int32_t* np_of;  // [num_seqs] partial results of each sequence (<= 1: written directly)
  float* part_m;    // [num_seqs, num_heads, max_partitions] running max (log2 units)
  float* part_l;    // [num_seqs, num_heads, max_partitions] sum of exp2(s - m)
  float* part_acc;  // [num_seqs, num_heads, max_partitions, head_size] unnormalised output
  float scale_log2;  // scale * log2(e): logits are kept in base-2 units
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int max_blocks;       // block_tables row length
  int len_limit;        // min(max_context_len, max_blocks * block_size)
  int partition_size;
  int max_partitions;   // partial slots per (sequence, head): ceil(max_context_len / partition_size)
                        // (+1 for shared-prefix decode, whose prefix may end inside a partition)
};

// Workspace: [queue header | prefetch pad | work items | split-K partials (several partitions)].
constexpr size_t kPrefetchPad = 8192;  // >= the bytes of one (block, head) tile: D * bs * 2
struct WorkspaceLayout {
  size_t pad_off, pairs_off, m_off, l_off, acc_off, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(int num_seqs, int num_heads, int head_size,
                                        int max_partitions) {
  WorkspaceLayout w{};
  const int parts = max_partitions > 0 ? max_partitions : 1;
  w.pad_off = 256;
  w.pairs_off = w.pad_off + kPrefetchPad;
  w.m_off = w.pairs_off + align256(size_t(num_seqs) * parts * sizeof(uint32_t));
  if (parts == 1) {
    w.l_off = w.acc_off = w.total = w.m_off;
    return w;
  }
  const size_t stats = size_t(num_seqs) * num_heads * parts * sizeof(float);
  w.l_off = w.m_off + align256(stats);
  w.acc_off = w.l_off + align256(stats);
  w.total = w.acc_off + align256(stats * head_size);
  return w;
}

// Workspace of the shared-prefix decode: [queue header | prefetch pad | per-sequence partial
// counts | work items (16 B) | partials], with `slots` partial slots per (sequence, head).
struct SharedWorkspaceLayout {
  size_t pad_off, np_off, items_off, m_off, l_off, acc_off, total;
};

inline SharedWorkspaceLayout shared_workspace_layout(int num_seqs, int num_heads, int head_size,
                                                     int slots) {
  SharedWorkspaceLayout w{};
  w.pad_off = 256;
  w.np_off = w.pad_off + kPrefetchPad;
  w.items_off = w.np_off + align256(size_t(num_seqs) * sizeof(int32_t));
  w.m_off = w.items_off + align256(size_t(num_seqs) * slots * 16);
  const size_t stats = size_t(num_seqs) * num_heads * slots * sizeof(float);
  w.l_off = w.m_off + align256(stats);
  w.acc_off = w.l_off + align256(stats);
  w.total = w.acc_off + align256(stats * head_size);
  return w;
}

// Dynamic LDS of the phase-1 kernels (must stay within the 64 KiB a launch gets by default).
inline size_t valu_lds_bytes(int group, int head_size, int partition_size) {
  return sizeof(float) * (size_t(group) * partition_size + kWaves * group * head_size + 2 * group);
}
constexpr size_t kMaxDynamicLds = 65536;

// Kernel launchers: return hipSuccess or the launch error.  Shapes are validated by the caller.
hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_size, int block_size,
                              int group, hipStream_t stream);
bool valu_supported(int dtype, int head_size, int block_size, int group);
bool gqa_supported(int dtype, int head_size, int block_size, int group);
hipError_t launch_decode_gqa(const DecodeArgs& a, int dtype, int head_size, int block_size,
                               int group, hipStream_t stream);
hipError_t launch_plan(const DecodeArgs& a, hipStream_t stream);
// Shared-prefix decode: the plan kernel over groups, then the matrix-core kernel over its items.
bool shared_supported(int dtype, int head_size, int block_size, int group);
hipError_t launch_plan_shared(const DecodeArgs& a, int block_size, int seqs_per_item,
                              hipStream_t stream);
hipError_t launch_decode_shared(const DecodeArgs& a, int dtype, int head_size, int block_size,
                                int group, hipStream_t stream);
hipError_t launch_reduce(const DecodeArgs& a, int dtype, int head_size, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping, int num_tokens,
                                    int num_kv_heads, int head_size, int block_size,
                                    int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                                    int elem_bytes, hipStream_t stream);
hipError_t launch_copy_blocks(const uint64_t* key_ptrs, const uint64_t* value_ptrs, int num_layers,
                              const int64_t* mapping, int num_pairs, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream);

}  // namespace pkv
