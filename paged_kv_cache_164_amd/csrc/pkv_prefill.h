// Host-side declarations of the multi-query attention path (chunked prefill, mixed batches).
#pragma once

#include "pkv_internal.h"

namespace pkv {

// ---- multi-query attention (chunked prefill, mixed batches) ----
// A workgroup handles kPrefillColumns (query token, query head) columns of one request and one
// KV head: q_tile = kPrefillColumns / G query tokens.  A tile's keys are cut at multiples of the
// partition size (auto: kPrefillAutoPartition); pieces start at multiples of 32 tokens.
constexpr int kPrefillColumns = 256;
constexpr int kPrefillAutoPartition = 8192;
constexpr int kPrefillMaxPartition = 8192;
constexpr int kPrefillMaxIds = 1088;  // >= (P + q_tile + 62) / 8 + 1 block ids of one item

struct PrefillArgs {
  void* out;                       // [T, Hq, D]
  const void* query;               // [T, Hq, D]
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;     // [B]
  const int32_t* query_start_loc;  // [B + 1]
  uint32_t* queue;                 // [2]: (reserved, number of work items)
  uint4* items;                    // (request, tile, first key, end key)
  int32_t* np_of;                  // [T] pieces of each query row (read by the reduce)
  float* part_m;                   // [T, Hq, slots]
  float* part_l;
  float* part_acc;                 // [T, Hq, slots, D]
  float scale_log2;                // scale * log2(e) (* key scale for an 8-bit cache)
  float v_scale;                   // 8-bit cache: value scale, applied to the output (else 1)
  int num_seqs, num_tokens, num_heads, num_kv_heads, max_blocks, max_context_len;
  int group, q_tile, partition_size, slots;
  int64_t capacity;                // items the workspace holds
};

// Items a call can produce: every tile of every request, each cut into at most
// ceil(max_context_len / P) pieces.
inline int64_t prefill_capacity(int num_seqs, int num_tokens, int q_tile, int max_context_len,
                                int partition_size) {
  const int64_t tiles = num_tokens / q_tile + num_seqs;
  const int64_t pieces = max_context_len > 0 ? (max_context_len + partition_size - 1) / partition_size : 1;
  return tiles * pieces;
}
struct PrefillLayout {
  size_t items_off, np_off, m_off, l_off, acc_off, total;
  int64_t capacity, slots;
};
inline PrefillLayout prefill_layout(int num_seqs, int num_tokens, int num_heads, int num_kv_heads,
                                    int head_size, int max_context_len, int partition_size) {
  PrefillLayout w{};
  const int group = num_kv_heads > 0 ? num_heads / num_kv_heads : 1;
  const int q_tile = kPrefillColumns / (group > 0 ? group : 1);
  w.capacity = prefill_capacity(num_seqs, num_tokens, q_tile, max_context_len, partition_size);
  w.slots = max_context_len > 0 ? (max_context_len + partition_size - 1) / partition_size : 1;
  w.items_off = 256;
  w.np_off = w.items_off + align256(size_t(w.capacity) * 16);
  w.m_off = w.np_off + align256(size_t(num_tokens) * sizeof(int32_t));
  if (w.slots <= 1) {  // no split: nothing but the work list
    w.l_off = w.acc_off = w.total = w.m_off;
    return w;
  }
  const size_t stats = size_t(num_tokens) * num_heads * w.slots * sizeof(float);
  w.l_off = w.m_off + align256(stats);
  w.acc_off = w.l_off + align256(stats);
  w.total = w.acc_off + align256(stats * head_size);
  return w;
}
bool prefill_supported(int dtype, int head_size, int block_size, int group);
// plan + attention kernel (+ the split-K reduce, given as `red`, when a.slots > 1); kv_code: 0
// for a 16-bit cache, else the caches hold 8-bit codes (1: E4M3, 2: INT8) and queries and output
// stay 16-bit (dtype)
hipError_t launch_prefill(const PrefillArgs& a, const DecodeArgs& red, int dtype, int head_size,
                          int block_size, int kv_code, hipStream_t stream);

}  // namespace pkv
