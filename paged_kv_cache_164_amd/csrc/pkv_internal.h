// Host-side declarations shared by the pkv translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace pkv {

constexpr int kMaxPartition = 4096;       // partition_size limit
constexpr int kMaxItemBlocks = 128;       // block ids an item holds in lane registers (16-bit)
constexpr int kMaxItemBlocks8 = 256;      // ... in the 8-bit cache kernel
constexpr int kMaxPartitions = 8192;      // per sequence (bounds the workspace and the grid)
constexpr int kTailChunks = 2;            // a remainder is cut into at most this many chunks
constexpr int kThreads = 256;  // VALU workgroup: 4 wave64s
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;  // logits are kept in base-2 units

// partition_size 0 ("auto"): on the matrix cores, 2048 tokens when an item's block ids fit its
// lane registers (block_size >= 16 for a 16-bit cache, >= 8 for an 8-bit one), else 1024; and
// for very long contexts (max_context_len >= kLongContext) 4096 where the ids fit (block_size
// 32 for a 16-bit cache, >= 16 for an 8-bit one): fewer, longer items halve the per-item
// overhead and the partials to merge (8 x 131072 tokens, block 32: 703 vs 717 us for the
// 16-bit kernel, 389 vs 403 us for the 8-bit one), while for many mixed lengths of a few
// thousand tokens 4096-token items were slower (8-bit, block 16: 285 vs 269 us).
constexpr int kLongContext = 32768;
inline int auto_partition(bool mfma, bool kv8, int block_size, int max_context_len) {
  const int max_blocks = kv8 ? kMaxItemBlocks8 : kMaxItemBlocks;
  if (!mfma) return 1024;
  if (max_context_len >= kLongContext && block_size * max_blocks >= 4096) return 4096;
  return block_size * max_blocks >= 2048 ? 2048 : 1024;
}
// Remainders (the tokens after a range's last whole partition) are cut into chunks of at most
// ceil(P / 2) rounded up to whole blocks, so the last items of a call are short.
inline int tail_chunk(int P, int block_size) {
  const int q = (P + kTailChunks - 1) / kTailChunks;
  return (q + block_size - 1) / block_size * block_size;
}
// Partial-result slots per (sequence, head) that the workspace provides.  A sequence's items
// are at most floor(L / P) whole partitions plus kTailChunks chunks for each of its (at most
// two: shared prefix, own tokens) ranges.  For partition_size 0 the layout is sized with
// P = 1024, the smaller auto choice, so it does not depend on the block size or kernel.
inline int64_t layout_slots(int max_context_len, int partition_size) {
  const int64_t P = partition_size > 0 ? partition_size : 1024;
  return (max_context_len + P - 1) / P + 2 * kTailChunks;
}

// Everything the attention kernels need, resolved on the host.
struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint32_t* queue;           // [2]: (reserved, number of work items), written by the plan kernel
  const char* prefetch_pad;  // kPrefetchPad bytes read by prefetches past a work item's end
  // Prefix groups (shared-prefix decode); null: every sequence is a group of its own.
  const int32_t* group_starts;  // [num_groups + 1] sequences of group g: [starts[g], starts[g+1])
  const int32_t* prefix_lens;   // [num_groups] tokens shared by the members of a group
  int num_groups;
  uint4* items;    // [num_seqs * slots] work items (b0, nseq | slot << 8, begin, end)
  int32_t* np_of;  // [num_seqs] partial results of each sequence (<= 1: written directly)
  float* part_m;    // [num_seqs, num_heads, slots] running max (log2 units)
  float* part_l;    // [num_seqs, num_heads, slots] sum of exp2(s - m)
  float* part_acc;  // [num_seqs, num_heads, slots, head_size] unnormalised output
  float scale_log2;  // scale * log2(e) (* key scale for an 8-bit cache): base-2 logit units
  float v_scale;     // 8-bit cache: value scale, applied to the output (1 otherwise)
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int max_blocks;       // block_tables row length
  int len_limit;        // min(max_context_len, max_blocks * block_size)
  int partition_size;   // P: tokens of a whole partition
  int tail_chunk;       // Q: tokens of a remainder chunk
  int slots;            // partial slots per (sequence, head); also items per sequence
  int plan_mode;        // 0: plan, then attention; 1: plan only; 2: attention on the plan
                        // already in the workspace
};

// A work item as the attention kernels read it from the list, which may come from an earlier
// call (plan_mode 2): an item whose sequences, partial slot or token range do not fit this
// call's shapes is skipped, a guard against lists planned for other shapes.
__host__ __device__ inline bool item_fits(const DecodeArgs& a, uint4 it) {
  const uint32_t b0 = it.x, nseq = it.y & 255u, slot = it.y >> 8;
  return nseq >= 1u && b0 < uint32_t(a.num_seqs) && nseq <= uint32_t(a.num_seqs) - b0 &&
         slot < uint32_t(a.slots) && it.z <= it.w && it.w <= uint32_t(a.len_limit);
}

// Workspace: [queue header | prefetch pad | per-sequence partial counts | work items (16 B) |
// split-K partials], each region 256-byte aligned.
constexpr size_t kPrefetchPad = 8192;  // >= the bytes of one (block, head) tile: D * bs * 2
struct WorkspaceLayout {
  size_t pad_off, np_off, items_off, m_off, l_off, acc_off, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(int num_seqs, int num_heads, int head_size, int64_t slots) {
  WorkspaceLayout w{};
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
// The plan kernel lists the work items; the attention kernels run one workgroup per (item,
// KV head); the reduce kernel merges each sequence's partial results.
hipError_t launch_plan(const DecodeArgs& a, int block_size, int seqs_per_item, hipStream_t stream);
// A decode step's new tokens, written by reshape_and_cache's per-token scatter.
struct CacheWriteArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const int64_t* slot_mapping;
  int num_tokens;
  int num_kv_heads;
  int head_size;
  int block_size;
  int64_t num_blocks;
  int64_t key_stride;  // elements between token rows
  int64_t value_stride;
};
// The plan kernel and the cache write of w in one launch (16- and 32-bit caches).
hipError_t launch_plan_and_cache(const DecodeArgs& a, int block_size, int seqs_per_item,
                                 const CacheWriteArgs& w, int elem_bytes, hipStream_t stream);
// The same with the write into an 8-bit cache (code kCodeE4M3 / kCodeI8; dtype 1 / 2 = fp16 /
// bf16 new keys and values).
hipError_t launch_plan_and_cache_kv8(const DecodeArgs& a, int block_size, int seqs_per_item,
                                     const CacheWriteArgs& w, int dtype, int code, float k_scale,
                                     float v_scale, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_size, int block_size,
                              int group, hipStream_t stream);
bool valu_supported(int dtype, int head_size, int block_size, int group);
bool gqa_supported(int dtype, int head_size, int block_size, int group);
hipError_t launch_decode_gqa(const DecodeArgs& a, int dtype, int head_size, int block_size,
                             int group, hipStream_t stream);
hipError_t launch_reduce(const DecodeArgs& a, int dtype, int head_size, hipStream_t stream);
// 8-bit (FP8 E4M3) caches, fp16 / bf16 queries (dtype 1 / 2); shapes as for launch_decode_gqa.
hipError_t launch_decode_fp8(const DecodeArgs& a, int dtype, int head_size, int block_size,
                             int group, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping, int num_tokens,
                                    int num_kv_heads, int head_size, int block_size,
                                    int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                                    int elem_bytes, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                        void* value_cache, const int64_t* slot_mapping,
                                        int num_tokens, int num_kv_heads, int head_size,
                                        int block_size, int64_t num_blocks, int64_t key_stride,
                                        int64_t value_stride, int dtype, float k_scale,
                                        float v_scale, hipStream_t stream);
// Device address of the static scratch of the allocation-free decode on the current device
// (PKV_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned); PKV_OK or an error code.
int noalloc_scratch_address(void** out);
// Records msg as the calling thread's pkv_last_error() and returns code (host code).
int record_error(int code, const char* msg);
inline int record_error(int code, const std::string& msg) { return record_error(code, msg.c_str()); }

hipError_t launch_copy_blocks(const uint64_t* key_ptrs, const uint64_t* value_ptrs, int num_layers,
                              const int64_t* mapping, int num_pairs, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream);

}  // namespace pkv
