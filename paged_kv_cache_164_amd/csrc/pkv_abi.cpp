// C ABI of libpkv: argument validation, workspace layout and kernel dispatch.
// The contracts are stated in include/pkv.h.
#include "pkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <string>
#include <vector>

#include "pkv_internal.h"
#include "pkv_kv8_host.h"
#include "pkv_prefill.h"
#include "pkv_probe.h"
#include "pkv_swap.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return PKV_ERR_HIP;
}

int elem_bytes(int dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
  }
  return 0;
}


struct Resolved {
  pkv::DecodeArgs args;
  size_t ws_needed;
  int group;
  int block_size;
  bool use_mfma;
  int kv_code;  // 0: 16/32-bit cache, else pkv::kCodeE4M3 or pkv::kCodeI8
};

// Code format and scales of an 8-bit cache; null for 16/32-bit caches.
struct Kv8 {
  float k_scale, v_scale;
  int code;  // pkv::kCodeE4M3 or pkv::kCodeI8
};

// Prefix groups of the shared-prefix decode (null for the plain decode).
struct Groups {
  const int32_t* starts;
  const int32_t* prefix_lens;
  int32_t count;
};

// Bytes of workspace for the given sizes (0 if invalid); shared by the size query, the decode
// entry points and the reduce entry point, which must agree on the layout.
size_t workspace_bytes_for(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                           int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_size <= 0 || max_context_len < 0) return 0;
  if (partition_size < 0 || partition_size > pkv::kMaxPartition) return 0;
  const int64_t slots = pkv::layout_slots(max_context_len, partition_size);
  if (slots > pkv::kMaxPartitions + 2 * pkv::kTailChunks) return 0;
  return pkv::workspace_layout(num_seqs, num_heads, head_size, slots).total;
}

// Shared validation of the decode entry points.
int resolve_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                   const int32_t* block_tables, const int32_t* context_lens, float scale,
                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                   int32_t block_size, int32_t max_num_blocks_per_seq, int32_t max_context_len,
                   int32_t dtype, int32_t partition_size, void* workspace, size_t workspace_bytes,
                   Resolved* r, const Groups* groups = nullptr, const Kv8* kv8 = nullptr) {
  if (elem_bytes(dtype) == 0) return fail(PKV_ERR_INVALID_ARG, "dtype must be PKV_F32, PKV_F16 or PKV_BF16");
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      max_num_blocks_per_seq < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative or zero size");
  if (num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_heads must be a multiple of num_kv_heads");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
  const int group = num_heads / num_kv_heads;
  if (head_size != 64 && head_size != 128) return fail(PKV_ERR_UNSUPPORTED, "head_size must be 64 or 128");
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size must be 8, 16 or 32");
  // 16-bit caches run on the matrix-core kernel (any group size up to 16), fp32 on the VALU one;
  // 8-bit caches on their matrix-core kernel, with fp16 / bf16 queries.
  const bool shared = groups != nullptr;
  if (kv8 && dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "an 8-bit cache needs PKV_F16 or PKV_BF16 queries");
  if (kv8 && !(std::isfinite(kv8->k_scale) && kv8->k_scale > 0.f && std::isfinite(kv8->v_scale) &&
               kv8->v_scale > 0.f))
    return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  const bool use_mfma = dtype != PKV_F32 && pkv::gqa_supported(dtype, head_size, block_size, group);
  if (shared && !use_mfma)
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode needs PKV_F16 or PKV_BF16 and a group size <= 16");
  if (!use_mfma && !pkv::valu_supported(dtype, head_size, block_size, group))
    return fail(PKV_ERR_UNSUPPORTED, "unsupported group size num_heads/num_kv_heads");
  if (partition_size < 0 || partition_size > pkv::kMaxPartition ||
      (partition_size > 0 && (partition_size < block_size || partition_size % block_size != 0)))
    return fail(PKV_ERR_INVALID_ARG, "partition_size must be 0 or a multiple of block_size in [block_size, 4096]");
  const int P = partition_size > 0 ? partition_size
                                   : pkv::auto_partition(use_mfma, kv8 != nullptr, block_size,
                                                         max_context_len);
  if (kv8 && P > pkv::kMaxItemBlocks8 * block_size)
    return fail(PKV_ERR_INVALID_ARG, "partition_size may span at most 256 blocks (8-bit cache)");
  if (use_mfma && !kv8 && P > pkv::kMaxItemBlocks * block_size)
    return fail(PKV_ERR_INVALID_ARG, "partition_size may span at most 128 blocks");
  const size_t lds = use_mfma ? 0 : pkv::valu_lds_bytes(group, head_size, P);
  if (lds > pkv::kMaxDynamicLds)
    return fail(PKV_ERR_UNSUPPORTED, "group size x partition_size needs more than 64 KiB of LDS");
  const int64_t slots = pkv::layout_slots(max_context_len, partition_size);
  if (slots > pkv::kMaxPartitions + 2 * pkv::kTailChunks)
    return fail(PKV_ERR_UNSUPPORTED, "max_context_len / partition_size exceeds 8192 partitions");
  const int64_t grid = (int64_t)num_seqs * num_kv_heads * slots;
  if (grid >= (int64_t(1) << 31)) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  if (num_seqs > 0 && (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens))
    return fail(PKV_ERR_NULL_POINTER, "null tensor pointer");
  if (shared && num_seqs > 0) {
    if (!groups->starts || !groups->prefix_lens) return fail(PKV_ERR_NULL_POINTER, "null group array");
    if (groups->count < 1 || groups->count > num_seqs)
      return fail(PKV_ERR_INVALID_ARG, "num_groups must be in [1, num_seqs]");
  }
  const pkv::WorkspaceLayout w = pkv::workspace_layout(num_seqs, num_heads, head_size, slots);
  const size_t need = num_seqs > 0 ? w.total : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace missing or too small: need " + std::to_string(need) + " bytes");
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  pkv::DecodeArgs& a = r->args;
  a = pkv::DecodeArgs{};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.group_starts = shared ? groups->starts : nullptr;
  a.prefix_lens = shared ? groups->prefix_lens : nullptr;
  a.num_groups = shared ? groups->count : 0;
  if (need > 0) {
    char* ws = static_cast<char*>(workspace);
    a.queue = reinterpret_cast<uint32_t*>(ws);
    a.prefetch_pad = ws + w.pad_off;
    a.np_of = reinterpret_cast<int32_t*>(ws + w.np_off);
    a.items = reinterpret_cast<uint4*>(ws + w.items_off);
    a.part_m = reinterpret_cast<float*>(ws + w.m_off);
    a.part_l = reinterpret_cast<float*>(ws + w.l_off);
    a.part_acc = reinterpret_cast<float*>(ws + w.acc_off);
  }
  a.scale_log2 = scale * pkv::kLog2e * (kv8 ? kv8->k_scale : 1.f);
  a.v_scale = kv8 ? kv8->v_scale : 1.f;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_num_blocks_per_seq;
  a.len_limit = (int)std::min<int64_t>(max_context_len, (int64_t)max_num_blocks_per_seq * block_size);
  a.partition_size = P;
  a.tail_chunk = pkv::tail_chunk(P, block_size);
  a.slots = (int)slots;
  r->ws_needed = need;
  r->group = group;
  r->block_size = block_size;
  r->use_mfma = use_mfma;
  r->kv_code = kv8 ? kv8->code : 0;
  return PKV_OK;
}

int launch_phase1(const Resolved& r, int dtype, int head_size, int block_size, hipStream_t s) {
  if (r.args.num_seqs == 0) return PKV_OK;
  hipError_t e = r.kv_code == pkv::kCodeE4M3
      ? pkv::launch_decode_fp8(r.args, dtype, head_size, block_size, r.group, s)
      : r.kv_code == pkv::kCodeI8
      ? pkv::launch_decode_i8(r.args, dtype, head_size, block_size, r.group, s)
      : r.use_mfma
      ? pkv::launch_decode_gqa(r.args, dtype, head_size, block_size, r.group, s)
      : pkv::launch_decode_valu(r.args, dtype, head_size, block_size, r.group, s);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attention kernel launch");
}

// The reduce kernel reads each sequence's partial count from the workspace and returns at once
// for sequences with a single item, so it is launched whatever the lengths turned out to be.
int launch_phase2(const Resolved& r, int dtype, int head_size, hipStream_t s) {
  if (r.args.num_seqs == 0) return PKV_OK;
  hipError_t e = pkv::launch_reduce(r.args, dtype, head_size, s);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "reduce kernel launch");
}

// Partition size of the multi-query path (0: auto), or -1 if invalid.
int prefill_partition(int32_t partition_size) {
  if (partition_size == 0) return pkv::kPrefillAutoPartition;
  if (partition_size < 32 || partition_size > pkv::kPrefillMaxPartition || partition_size % 32 != 0)
    return -1;
  return partition_size;
}

// Shapes of the multi-query path that the layout depends on (0 bytes if invalid).
size_t prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size, int32_t max_context_len,
                               int32_t partition_size) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      max_context_len < 0 || num_heads % num_kv_heads != 0 || num_heads / num_kv_heads > 16)
    return 0;
  const int P = prefill_partition(partition_size);
  if (P < 0) return 0;
  if (num_seqs == 0 || num_tokens == 0) return 0;
  return pkv::prefill_layout(num_seqs, num_tokens, num_heads, num_kv_heads, head_size,
                             max_context_len, P).total;
}

}  // namespace

namespace pkv {
int record_error(int code, const char* msg) { return fail(code, msg); }
}  // namespace pkv

static int prefill_call(void* out, const void* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_tables,
                        const int32_t* context_lens, const int32_t* query_start_loc, float scale,
                        const Kv8* kv8, int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                        int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
                        int32_t partition_size, void* workspace, size_t workspace_bytes,
                        void* stream) {
  try {
    if (dtype != PKV_F16 && dtype != PKV_BF16)
      return fail(dtype == PKV_F32 ? PKV_ERR_UNSUPPORTED : PKV_ERR_INVALID_ARG,
                  "multi-query attention runs on the matrix cores: dtype must be PKV_F16 or PKV_BF16");
    if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        max_context_len < 0 || max_num_blocks_per_seq < 0)
      return fail(PKV_ERR_INVALID_ARG, "negative or zero size");
    if (num_heads % num_kv_heads != 0)
      return fail(PKV_ERR_INVALID_ARG, "num_heads must be a multiple of num_kv_heads");
    if (!(std::isfinite(scale) && scale > 0.f))
      return fail(PKV_ERR_INVALID_ARG, "scale must be finite and positive");
    if (kv8 && !(std::isfinite(kv8->k_scale) && kv8->k_scale > 0.f && std::isfinite(kv8->v_scale) &&
                 kv8->v_scale > 0.f))
      return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
    const int group = num_heads / num_kv_heads;
    if (!pkv::prefill_supported(dtype, head_size, block_size, group))
      return fail(PKV_ERR_UNSUPPORTED,
                  "head_size must be 64 or 128, block_size 8, 16 or 32, num_heads/num_kv_heads <= 16");
    if ((int64_t)head_size * block_size * 2 * num_kv_heads >= (int64_t(1) << 32))
      return fail(PKV_ERR_UNSUPPORTED, "a cache block (all KV heads) must be below 4 GiB");
    const int P = prefill_partition(partition_size);
    if (P < 0)
      return fail(PKV_ERR_INVALID_ARG, "partition_size must be 0 or a multiple of 32 in [32, 8192]");
    if ((int64_t)max_num_blocks_per_seq * block_size < max_context_len)
      return fail(PKV_ERR_INVALID_ARG, "block table rows are shorter than max_context_len");
    if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
        !query_start_loc)
      return fail(PKV_ERR_NULL_POINTER, "null tensor pointer");
    const pkv::PrefillLayout w = pkv::prefill_layout(num_seqs, num_tokens, num_heads, num_kv_heads,
                                                     head_size, max_context_len, P);
    if (w.capacity * num_kv_heads >= (int64_t(1) << 31))
      return fail(PKV_ERR_UNSUPPORTED, "grid too large");
    if (workspace == nullptr || workspace_bytes < w.total)
      return fail(PKV_ERR_WORKSPACE, "workspace missing or too small: need " + std::to_string(w.total) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    char* ws = static_cast<char*>(workspace);
    pkv::PrefillArgs a{};
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start_loc = query_start_loc;
    a.queue = reinterpret_cast<uint32_t*>(ws);
    a.items = reinterpret_cast<uint4*>(ws + w.items_off);
    a.np_of = reinterpret_cast<int32_t*>(ws + w.np_off);
    a.part_m = reinterpret_cast<float*>(ws + w.m_off);
    a.part_l = reinterpret_cast<float*>(ws + w.l_off);
    a.part_acc = reinterpret_cast<float*>(ws + w.acc_off);
    a.scale_log2 = scale * pkv::kLog2e * (kv8 ? kv8->k_scale : 1.f);
    a.v_scale = kv8 ? kv8->v_scale : 1.f;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks = max_num_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.group = group;
    a.q_tile = pkv::kPrefillColumns / group;
    a.partition_size = P;
    a.slots = (int)w.slots;
    a.capacity = w.capacity;
    // the split-K reduce of the decode path, with one "sequence" per query row
    pkv::DecodeArgs red{};
    red.out = out;
    red.np_of = a.np_of;
    red.part_m = a.part_m;
    red.part_l = a.part_l;
    red.part_acc = a.part_acc;
    red.num_seqs = num_tokens;
    red.num_heads = num_heads;
    red.num_kv_heads = num_kv_heads;
    red.slots = a.slots;
    const hipError_t e = pkv::launch_prefill(a, red, dtype, head_size, block_size,
                                             kv8 ? kv8->code : 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : hip_fail(e, "multi-query attention launch");
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}


extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

size_t pkv_paged_attention_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                          int32_t max_context_len, int32_t partition_size) {
  return workspace_bytes_for(num_seqs, num_heads, head_size, max_context_len, partition_size);
}

#define PKV_DECODE_PARAMS                                                                     \
  void *out, const void *query, const void *key_cache, const void *value_cache,               \
      const int32_t *block_tables, const int32_t *context_lens, float scale, int32_t num_seqs, \
      int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,         \
      int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,                 \
      int32_t partition_size, void *workspace, size_t workspace_bytes, void *stream
#define PKV_DECODE_ARGS                                                                        \
  out, query, key_cache, value_cache, block_tables, context_lens, scale, num_seqs, num_heads, \
      num_kv_heads, head_size, block_size, max_num_blocks_per_seq, max_context_len, dtype,    \
      partition_size, workspace, workspace_bytes

int pkv_paged_attention_decode(PKV_DECODE_PARAMS) {
  try {
    Resolved r;
    int rc = resolve_decode(PKV_DECODE_ARGS, &r);
    if (rc != PKV_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = launch_phase1(r, dtype, head_size, block_size, s);
    if (rc != PKV_OK) return rc;
    return launch_phase2(r, dtype, head_size, s);
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

size_t pkv_paged_attention_noalloc_scratch_bytes(void) { return PKV_NOALLOC_SCRATCH_BYTES; }

// The decode with the library's static scratch as its workspace (no allocation in the call).
int pkv_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                       int32_t block_size, int32_t max_num_blocks_per_seq,
                                       int32_t max_context_len, int32_t dtype,
                                       int32_t partition_size, void* stream) {
  try {
    const size_t need = workspace_bytes_for(num_seqs, num_heads, head_size, max_context_len,
                                            partition_size);
    if (need > PKV_NOALLOC_SCRATCH_BYTES)
      return fail(PKV_ERR_WORKSPACE, "these sizes need " + std::to_string(need) +
                                         " bytes of scratch; the allocation-free decode holds " +
                                         std::to_string(PKV_NOALLOC_SCRATCH_BYTES));
    // Every argument is checked before the scratch's address is looked up: a stand-in address
    // (256-byte aligned, never dereferenced) takes its place for that check.
    Resolved r;
    void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
    int rc = resolve_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            num_seqs, num_heads, num_kv_heads, head_size, block_size,
                            max_num_blocks_per_seq, max_context_len, dtype, partition_size,
                            stand_in, PKV_NOALLOC_SCRATCH_BYTES, &r);
    if (rc != PKV_OK || r.ws_needed == 0) return rc;
    void* ws = nullptr;
    rc = pkv::noalloc_scratch_address(&ws);
    if (rc != PKV_OK) return rc;
    return pkv_paged_attention_decode(out, query, key_cache, value_cache, block_tables,
                                      context_lens, scale, num_seqs, num_heads, num_kv_heads,
                                      head_size, block_size, max_num_blocks_per_seq,
                                      max_context_len, dtype, partition_size, ws,
                                      PKV_NOALLOC_SCRATCH_BYTES, stream);
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

#define PKV_SHARED_PARAMS_NO_STREAM                                                           \
  void *out, const void *query, const void *key_cache, const void *value_cache,               \
      const int32_t *block_tables, const int32_t *context_lens, const int32_t *group_starts,  \
      const int32_t *prefix_lens, int32_t num_groups, float scale, int32_t num_seqs,          \
      int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,         \
      int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,                 \
      int32_t partition_size, void *workspace, size_t workspace_bytes
#define PKV_SHARED_PARAMS PKV_SHARED_PARAMS_NO_STREAM, void *stream

// The shared-prefix decode, whole (mode 0: plan, attention kernel, reduce), the plan alone
// (mode 1) or the attention kernel on the plan already in the workspace (mode 2).
static int decode_shared_mode(PKV_SHARED_PARAMS, int mode) {
  try {
    Resolved r;
    const Groups groups{group_starts, prefix_lens, num_groups};
    int rc = resolve_decode(PKV_DECODE_ARGS, &r, &groups);
    if (rc != PKV_OK) return rc;
    if (num_seqs == 0) return PKV_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    r.args.plan_mode = mode;
    rc = launch_phase1(r, dtype, head_size, block_size, s);
    if (rc != PKV_OK || mode != 0) return rc;
    return launch_phase2(r, dtype, head_size, s);
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

#define PKV_SHARED_ARGS                                                                       \
  out, query, key_cache, value_cache, block_tables, context_lens, group_starts, prefix_lens,  \
      num_groups, scale, num_seqs, num_heads, num_kv_heads, head_size, block_size,            \
      max_num_blocks_per_seq, max_context_len, dtype, partition_size, workspace,              \
      workspace_bytes, stream

int pkv_paged_attention_decode_shared(PKV_SHARED_PARAMS) {
  return decode_shared_mode(PKV_SHARED_ARGS, 0);
}

int pkv_paged_attention_plan_shared(PKV_SHARED_PARAMS) {
  return decode_shared_mode(PKV_SHARED_ARGS, 1);
}

int pkv_paged_attention_partitions_planned_shared(PKV_SHARED_PARAMS) {
  return decode_shared_mode(PKV_SHARED_ARGS, 2);
}

// The 8-bit decode, whole (mode 0), the plan alone (mode 1) or the attention kernel on the plan
// already in the workspace (mode 2).
static int decode_kv8(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      const Kv8& kv8, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_size, int32_t block_size, int32_t max_num_blocks_per_seq,
                      int32_t max_context_len, int32_t dtype, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, void* stream, int mode) {
  try {
    Resolved r;
    int rc = resolve_decode(PKV_DECODE_ARGS, &r, nullptr, &kv8);
    if (rc != PKV_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    r.args.plan_mode = mode;
    rc = launch_phase1(r, dtype, head_size, block_size, s);
    if (rc != PKV_OK || mode != 0) return rc;
    return launch_phase2(r, dtype, head_size, s);
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

#define PKV_DECODE_KV8_PARAMS                                                                   \
  void *out, const void *query, const void *key_cache, const void *value_cache,                 \
      const int32_t *block_tables, const int32_t *context_lens, float scale, float k_scale,     \
      float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,                 \
      int32_t head_size, int32_t block_size, int32_t max_num_blocks_per_seq,                    \
      int32_t max_context_len, int32_t dtype, int32_t partition_size, void *workspace,          \
      size_t workspace_bytes, void *stream
#define PKV_DECODE_KV8_CALL(CODE, MODE)                                                         \
  decode_kv8(out, query, key_cache, value_cache, block_tables, context_lens, scale,             \
             Kv8{k_scale, v_scale, CODE}, num_seqs, num_heads, num_kv_heads, head_size,         \
             block_size, max_num_blocks_per_seq, max_context_len, dtype, partition_size,        \
             workspace, workspace_bytes, stream, MODE)

int pkv_paged_attention_decode_fp8(PKV_DECODE_KV8_PARAMS) {
  return PKV_DECODE_KV8_CALL(pkv::kCodeE4M3, 0);
}

int pkv_paged_attention_decode_int8(PKV_DECODE_KV8_PARAMS) {
  return PKV_DECODE_KV8_CALL(pkv::kCodeI8, 0);
}

int pkv_paged_attention_plan_fp8(PKV_DECODE_KV8_PARAMS) {
  return PKV_DECODE_KV8_CALL(pkv::kCodeE4M3, 1);
}

int pkv_paged_attention_partitions_planned_fp8(PKV_DECODE_KV8_PARAMS) {
  return PKV_DECODE_KV8_CALL(pkv::kCodeE4M3, 2);
}

int pkv_paged_attention_plan_int8(PKV_DECODE_KV8_PARAMS) {
  return PKV_DECODE_KV8_CALL(pkv::kCodeI8, 1);
}

int pkv_paged_attention_partitions_planned_int8(PKV_DECODE_KV8_PARAMS) {
  return PKV_DECODE_KV8_CALL(pkv::kCodeI8, 2);
}

int pkv_paged_attention_partitions(PKV_DECODE_PARAMS) {
  try {
    Resolved r;
    int rc = resolve_decode(PKV_DECODE_ARGS, &r);
    if (rc != PKV_OK) return rc;
    return launch_phase1(r, dtype, head_size, block_size, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

// Phase 1 split in two: the plan kernel alone (plan_mode 1), and the attention kernel on the
// plan already in the workspace (plan_mode 2).
static int phase1_mode(PKV_DECODE_PARAMS, int mode) {
  try {
    Resolved r;
    int rc = resolve_decode(PKV_DECODE_ARGS, &r);
    if (rc != PKV_OK) return rc;
    r.args.plan_mode = mode;
    return launch_phase1(r, dtype, head_size, block_size, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

int pkv_paged_attention_plan(PKV_DECODE_PARAMS) { return phase1_mode(PKV_DECODE_ARGS, stream, 1); }

int pkv_paged_attention_partitions_planned(PKV_DECODE_PARAMS) {
  return phase1_mode(PKV_DECODE_ARGS, stream, 2);
}

// The plan and the new tokens' cache write (16- and 32-bit caches) in one launch; groups: the
// shared-prefix plan, or null for the plain one.
static int plan_and_cache_16(void* out, const void* query, const void* key_cache,
                             const void* value_cache, const int32_t* block_tables,
                             const int32_t* context_lens, float scale, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                             int32_t block_size, int32_t max_num_blocks_per_seq,
                             int32_t max_context_len, int32_t dtype, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, const Groups* groups,
                             const void* key, const void* value, const int64_t* slot_mapping,
                             int32_t num_tokens, int64_t num_blocks, int64_t key_stride,
                             int64_t value_stride, void* stream) {
  try {
    Resolved r;
    int rc = resolve_decode(PKV_DECODE_ARGS, &r, groups);
    if (rc != PKV_OK) return rc;
    const int eb = elem_bytes(dtype);
    if (num_tokens < 0 || num_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
    if (key_stride < (int64_t)num_kv_heads * head_size || value_stride < (int64_t)num_kv_heads * head_size)
      return fail(PKV_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_size");
    if (num_tokens > 0 && (!key || !value || !slot_mapping || !key_cache || !value_cache))
      return fail(PKV_ERR_NULL_POINTER, "null tensor pointer");
    if ((int64_t)num_tokens + 1 >= (int64_t(1) << 31)) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const pkv::CacheWriteArgs w{key, value, const_cast<void*>(key_cache),
                                const_cast<void*>(value_cache), slot_mapping, num_tokens,
                                num_kv_heads, head_size, block_size, num_blocks, key_stride,
                                value_stride};
    hipError_t e;
    if (num_seqs == 0)  // no plan: the write alone
      e = pkv::launch_reshape_and_cache(key, value, w.key_cache, w.value_cache, slot_mapping,
                                        num_tokens, num_kv_heads, head_size, block_size,
                                        num_blocks, key_stride, value_stride, eb, s);
    else
      e = pkv::launch_plan_and_cache(r.args, block_size, r.use_mfma ? 16 / r.group : 1, w, eb, s);
    return e == hipSuccess ? PKV_OK : hip_fail(e, "plan and cache write launch");
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

int pkv_paged_attention_plan_and_cache(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                       int32_t block_size, int32_t max_num_blocks_per_seq,
                                       int32_t max_context_len, int32_t dtype,
                                       int32_t partition_size, void* workspace,
                                       size_t workspace_bytes, const void* key, const void* value,
                                       const int64_t* slot_mapping, int32_t num_tokens,
                                       int64_t num_blocks, int64_t key_stride,
                                       int64_t value_stride, void* stream) {
  return plan_and_cache_16(PKV_DECODE_ARGS, nullptr, key, value, slot_mapping, num_tokens,
                           num_blocks, key_stride, value_stride, stream);
}

int pkv_paged_attention_plan_and_cache_shared(PKV_SHARED_PARAMS_NO_STREAM, const void* key,
                                              const void* value, const int64_t* slot_mapping,
                                              int32_t num_tokens, int64_t num_blocks,
                                              int64_t key_stride, int64_t value_stride,
                                              void* stream) {
  const Groups groups{group_starts, prefix_lens, num_groups};
  return plan_and_cache_16(PKV_DECODE_ARGS, &groups, key, value, slot_mapping, num_tokens,
                           num_blocks, key_stride, value_stride, stream);
}

// The plan and the write of the new tokens into an 8-bit cache, in one launch.
static int plan_and_cache_kv8(void* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, const Kv8& kv8,
                              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_size, int32_t block_size,
                              int32_t max_num_blocks_per_seq, int32_t max_context_len,
                              int32_t dtype, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, const void* key, const void* value,
                              const int64_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
                              int64_t key_stride, int64_t value_stride, void* stream) {
  try {
    Resolved r;
    int rc = resolve_decode(PKV_DECODE_ARGS, &r, nullptr, &kv8);
    if (rc != PKV_OK) return rc;
    if (num_tokens < 0 || num_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
    if (key_stride < (int64_t)num_kv_heads * head_size || value_stride < (int64_t)num_kv_heads * head_size)
      return fail(PKV_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_size");
    if (num_tokens > 0 && (!key || !value || !slot_mapping || !key_cache || !value_cache))
      return fail(PKV_ERR_NULL_POINTER, "null tensor pointer");
    if (num_tokens > 0 && reinterpret_cast<uintptr_t>(key_cache) % 16 != 0)
      return fail(PKV_ERR_INVALID_ARG, "key_cache must be 16-byte aligned");
    if ((int64_t)num_tokens + 1 >= (int64_t(1) << 31)) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* kc = const_cast<void*>(key_cache);
    void* vc = const_cast<void*>(value_cache);
    hipError_t e;
    if (num_seqs == 0) {  // no plan: the write alone
      if (num_tokens == 0) return PKV_OK;
      auto* launch = kv8.code == pkv::kCodeE4M3 ? pkv::launch_reshape_and_cache_fp8
                                                : pkv::launch_reshape_and_cache_i8;
      e = launch(key, value, kc, vc, slot_mapping, num_tokens, num_kv_heads, head_size, block_size,
                 num_blocks, key_stride, value_stride, dtype, kv8.k_scale, kv8.v_scale, s);
    } else {
      const pkv::CacheWriteArgs w{key, value, kc, vc, slot_mapping, num_tokens, num_kv_heads,
                                  head_size, block_size, num_blocks, key_stride, value_stride};
      e = pkv::launch_plan_and_cache_kv8(r.args, block_size, 16 / r.group, w, dtype, kv8.code,
                                         kv8.k_scale, kv8.v_scale, s);
    }
    return e == hipSuccess ? PKV_OK : hip_fail(e, "plan and 8-bit cache write launch");
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

#define PKV_PLAN_AND_CACHE_KV8_PARAMS                                                            \
  void *out, const void *query, const void *key_cache, const void *value_cache,                 \
      const int32_t *block_tables, const int32_t *context_lens, float scale, float k_scale,     \
      float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,                 \
      int32_t head_size, int32_t block_size, int32_t max_num_blocks_per_seq,                    \
      int32_t max_context_len, int32_t dtype, int32_t partition_size, void *workspace,          \
      size_t workspace_bytes, const void *key, const void *value, const int64_t *slot_mapping,  \
      int32_t num_tokens, int64_t num_blocks, int64_t key_stride, int64_t value_stride,         \
      void *stream
#define PKV_PLAN_AND_CACHE_KV8_CALL(CODE)                                                        \
  plan_and_cache_kv8(out, query, key_cache, value_cache, block_tables, context_lens, scale,      \
                     Kv8{k_scale, v_scale, CODE}, num_seqs, num_heads, num_kv_heads, head_size, \
                     block_size, max_num_blocks_per_seq, max_context_len, dtype, partition_size, \
                     workspace, workspace_bytes, key, value, slot_mapping, num_tokens,           \
                     num_blocks, key_stride, value_stride, stream)

int pkv_paged_attention_plan_and_cache_fp8(PKV_PLAN_AND_CACHE_KV8_PARAMS) {
  return PKV_PLAN_AND_CACHE_KV8_CALL(pkv::kCodeE4M3);
}

int pkv_paged_attention_plan_and_cache_int8(PKV_PLAN_AND_CACHE_KV8_PARAMS) {
  return PKV_PLAN_AND_CACHE_KV8_CALL(pkv::kCodeI8);
}

int pkv_paged_attention_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t head_size, int32_t max_context_len,
                               int32_t dtype, int32_t partition_size, const void* workspace,
                               size_t workspace_bytes, void* stream) {
  try {
    if (elem_bytes(dtype) == 0) return fail(PKV_ERR_INVALID_ARG, "bad dtype");
    if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0)
      return fail(PKV_ERR_INVALID_ARG, "negative or zero size");
    if (head_size != 64 && head_size != 128) return fail(PKV_ERR_UNSUPPORTED, "head_size must be 64 or 128");
    if (partition_size < 0 || partition_size > pkv::kMaxPartition)
      return fail(PKV_ERR_INVALID_ARG, "bad partition_size");
    if (num_seqs == 0) return PKV_OK;
    if (!out || !context_lens) return fail(PKV_ERR_NULL_POINTER, "null tensor pointer");
    const int64_t slots = pkv::layout_slots(max_context_len, partition_size);
    if (slots > pkv::kMaxPartitions + 2 * pkv::kTailChunks)
      return fail(PKV_ERR_UNSUPPORTED, "too many partitions");
    const pkv::WorkspaceLayout w = pkv::workspace_layout(num_seqs, num_heads, head_size, slots);
    if (!workspace || workspace_bytes < w.total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return fail(PKV_ERR_WORKSPACE, "workspace missing, misaligned or too small");
    Resolved r{};
    pkv::DecodeArgs& a = r.args;
    char* ws = const_cast<char*>(static_cast<const char*>(workspace));
    a.out = out;
    a.context_lens = context_lens;
    a.np_of = reinterpret_cast<int32_t*>(ws + w.np_off);
    a.part_m = reinterpret_cast<float*>(ws + w.m_off);
    a.part_l = reinterpret_cast<float*>(ws + w.l_off);
    a.part_acc = reinterpret_cast<float*>(ws + w.acc_off);
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.len_limit = max_context_len;
    a.slots = (int)slots;
    return launch_phase2(r, dtype, head_size, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

size_t pkv_paged_attention_prefill_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                                  int32_t num_heads, int32_t num_kv_heads,
                                                  int32_t head_size, int32_t max_context_len,
                                                  int32_t partition_size) {
  return prefill_workspace_bytes(num_seqs, num_tokens, num_heads, num_kv_heads, head_size,
                                 max_context_len, partition_size);
}

int pkv_paged_attention_prefill(void* out, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                float scale, int32_t num_seqs, int32_t num_tokens,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                int32_t block_size, int32_t max_num_blocks_per_seq,
                                int32_t max_context_len, int32_t dtype, int32_t partition_size,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_call(out, query, key_cache, value_cache, block_tables, context_lens,
                      query_start_loc, scale, nullptr, num_seqs, num_tokens, num_heads,
                      num_kv_heads, head_size, block_size, max_num_blocks_per_seq,
                      max_context_len, dtype, partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attention_prefill_fp8(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* query_start_loc,
                                    float scale, float k_scale, float v_scale, int32_t num_seqs,
                                    int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t block_size,
                                    int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                    int32_t dtype, int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const Kv8 kv8{k_scale, v_scale, pkv::kCodeE4M3};
  return prefill_call(out, query, key_cache, value_cache, block_tables, context_lens,
                      query_start_loc, scale, &kv8, num_seqs, num_tokens, num_heads,
                      num_kv_heads, head_size, block_size, max_num_blocks_per_seq,
                      max_context_len, dtype, partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attention_prefill_int8(void* out, const void* query, const void* key_cache,
                                     const void* value_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* query_start_loc,
                                     float scale, float k_scale, float v_scale, int32_t num_seqs,
                                     int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_size, int32_t block_size,
                                     int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                     int32_t dtype, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const Kv8 kv8{k_scale, v_scale, pkv::kCodeI8};
  return prefill_call(out, query, key_cache, value_cache, block_tables, context_lens,
                      query_start_loc, scale, &kv8, num_seqs, num_tokens, num_heads,
                      num_kv_heads, head_size, block_size, max_num_blocks_per_seq,
                      max_context_len, dtype, partition_size, workspace, workspace_bytes, stream);
}

int pkv_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  try {
    if (bytes == 0) return PKV_OK;
    if (!src || !sink) return fail(PKV_ERR_NULL_POINTER, "null pointer");
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (bytes & 15u))
      return fail(PKV_ERR_INVALID_ARG, "src and bytes must be multiples of 16");
    const hipError_t e = pkv::launch_stream_read(src, (int64_t)bytes, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : hip_fail(e, "stream read launch");
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

int pkv_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_size, int32_t block_size, int64_t num_blocks,
                          int64_t key_stride, int64_t value_stride, int32_t dtype, void* stream) {
  try {
    const int eb = elem_bytes(dtype);
    if (eb == 0) return fail(PKV_ERR_INVALID_ARG, "bad dtype");
    if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
      return fail(PKV_ERR_INVALID_ARG, "negative or zero size");
    const int x = 16 / eb;
    if (head_size % x != 0) return fail(PKV_ERR_INVALID_ARG, "head_size must be a multiple of x = 16/sizeof");
    if (key_stride < (int64_t)num_kv_heads * head_size || value_stride < (int64_t)num_kv_heads * head_size)
      return fail(PKV_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_size");
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
      return fail(PKV_ERR_NULL_POINTER, "null tensor pointer");
    hipError_t e = pkv::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
                                                 num_tokens, num_kv_heads, head_size, block_size,
                                                 num_blocks, key_stride, value_stride, eb,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : hip_fail(e, "reshape_and_cache launch");
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

static int reshape_and_cache_kv8(const void* key, const void* value, void* key_cache,
                                 void* value_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                                 int32_t block_size, int64_t num_blocks, int64_t key_stride,
                                 int64_t value_stride, int32_t dtype, float k_scale, float v_scale,
                                 int code, void* stream) {
  try {
    if (dtype != PKV_F16 && dtype != PKV_BF16)
      return fail(PKV_ERR_INVALID_ARG, "key and value must be PKV_F16 or PKV_BF16");
    if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
      return fail(PKV_ERR_INVALID_ARG, "negative or zero size");
    if (head_size % 16 != 0) return fail(PKV_ERR_INVALID_ARG, "head_size must be a multiple of x = 16");
    if (key_stride < (int64_t)num_kv_heads * head_size || value_stride < (int64_t)num_kv_heads * head_size)
      return fail(PKV_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_size");
    if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
      return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
      return fail(PKV_ERR_NULL_POINTER, "null tensor pointer");
    if (reinterpret_cast<uintptr_t>(key_cache) % 16 != 0)
      return fail(PKV_ERR_INVALID_ARG, "key_cache must be 16-byte aligned");
    auto* launch = code == pkv::kCodeE4M3 ? pkv::launch_reshape_and_cache_fp8
                                          : pkv::launch_reshape_and_cache_i8;
    hipError_t e = launch(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                          num_kv_heads, head_size, block_size, num_blocks, key_stride,
                          value_stride, dtype, k_scale, v_scale, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : hip_fail(e, "8-bit reshape_and_cache launch");
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

int pkv_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                              void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                              int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                              int32_t dtype, float k_scale, float v_scale, void* stream) {
  return reshape_and_cache_kv8(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                               num_kv_heads, head_size, block_size, num_blocks, key_stride,
                               value_stride, dtype, k_scale, v_scale, pkv::kCodeE4M3, stream);
}

int pkv_reshape_and_cache_int8(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                               int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                               int32_t dtype, float k_scale, float v_scale, void* stream) {
  return reshape_and_cache_kv8(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                               num_kv_heads, head_size, block_size, num_blocks, key_stride,
                               value_stride, dtype, k_scale, v_scale, pkv::kCodeI8, stream);
}

int pkv_copy_blocks(const uint64_t* key_cache_ptrs, const uint64_t* value_cache_ptrs,
                    int32_t num_layers, const int64_t* block_mapping, int32_t num_pairs,
                    int64_t block_bytes, int64_t num_blocks, void* stream) {
  try {
    if (num_layers < 0 || num_pairs < 0 || block_bytes <= 0 || num_blocks < 0)
      return fail(PKV_ERR_INVALID_ARG, "negative or zero size");
    if (block_bytes % 16 != 0) return fail(PKV_ERR_INVALID_ARG, "block_bytes must be a multiple of 16");
    if (num_layers > 65535) return fail(PKV_ERR_UNSUPPORTED, "more than 65535 layers");
    if (num_layers == 0 || num_pairs == 0) return PKV_OK;
    if (!key_cache_ptrs || !value_cache_ptrs || !block_mapping)
      return fail(PKV_ERR_NULL_POINTER, "null pointer");
    const int64_t chunks = (block_bytes / 16 + 2047) / 2048;
    if ((int64_t)num_pairs * chunks >= (int64_t(1) << 31)) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
    hipError_t e = pkv::launch_copy_blocks(key_cache_ptrs, value_cache_ptrs, num_layers, block_mapping,
                                           num_pairs, block_bytes, num_blocks,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : hip_fail(e, "copy_blocks launch");
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

int pkv_swap_blocks(void* dst, const void* src, const int64_t* block_mapping, int32_t num_pairs,
                    int64_t block_bytes, int64_t src_num_blocks, int64_t dst_num_blocks,
                    int32_t direction, void* stream) {
  try {
    if (num_pairs < 0 || block_bytes <= 0 || src_num_blocks < 0 || dst_num_blocks < 0)
      return fail(PKV_ERR_INVALID_ARG, "negative or zero size");
    if (direction != PKV_SWAP_IN && direction != PKV_SWAP_OUT)
      return fail(PKV_ERR_INVALID_ARG, "direction must be PKV_SWAP_IN or PKV_SWAP_OUT");
    if (num_pairs == 0) return PKV_OK;
    if (!dst || !src || !block_mapping) return fail(PKV_ERR_NULL_POINTER, "null pointer");
    const void* host = direction == PKV_SWAP_IN ? src : dst;
    const void* dev = direction == PKV_SWAP_IN ? dst : src;
    hipPointerAttribute_t hattr{}, attr{};
    hipError_t e = hipPointerGetAttributes(&hattr, host);
    if (e != hipSuccess || hattr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();  // clear the sticky error of an unregistered pointer
      return fail(PKV_ERR_NOT_PINNED, "host side of swap_blocks is not page-locked host memory");
    }
    e = hipPointerGetAttributes(&attr, dev);
    if (e != hipSuccess || attr.type != hipMemoryTypeDevice) {
      (void)hipGetLastError();
      return fail(PKV_ERR_INVALID_ARG, "device side of swap_blocks is not device memory");
    }
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int64_t s = block_mapping[2 * i], d = block_mapping[2 * i + 1];
      if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks)
        return fail(PKV_ERR_INVALID_ARG, "block id out of range at pair " + std::to_string(i));
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The device reaches the pinned memory at the host pointer itself (mapped host memory under
    // unified addressing): one kernel per kSwapPairs blocks, all blocks' bytes in flight at once.
    if (hattr.devicePointer == host && block_bytes % 8 == 0 &&
        reinterpret_cast<uintptr_t>(dst) % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 8 == 0) {
      pkv::SwapList list;
      for (int32_t i0 = 0; i0 < num_pairs; i0 += pkv::kSwapPairs) {
        const int32_t n = std::min<int32_t>(pkv::kSwapPairs, num_pairs - i0);
        for (int32_t j = 0; j < n; ++j) {
          list.src[j] = block_mapping[2 * (i0 + j)];
          list.dst[j] = block_mapping[2 * (i0 + j) + 1];
        }
        e = pkv::launch_swap_blocks(dst, src, list, n, block_bytes, direction == PKV_SWAP_OUT, st);
        if (e != hipSuccess) return hip_fail(e, "swap_blocks launch");
      }
      return PKV_OK;
    }
    // Otherwise the copy engines, runs of consecutive ids as one asynchronous copy each.
    const hipMemcpyKind kind = direction == PKV_SWAP_IN ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
    int32_t i = 0;
    while (i < num_pairs) {
      const int64_t s0 = block_mapping[2 * i], d0 = block_mapping[2 * i + 1];
      int32_t n = 1;
      while (i + n < num_pairs && block_mapping[2 * (i + n)] == s0 + n &&
             block_mapping[2 * (i + n) + 1] == d0 + n)
        ++n;
      e = hipMemcpyAsync(static_cast<char*>(dst) + d0 * block_bytes,
                         static_cast<const char*>(src) + s0 * block_bytes, (size_t)n * block_bytes,
                         kind, st);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
      i += n;
    }
    return PKV_OK;
  } catch (...) {
    return fail(PKV_ERR_HIP, "unexpected C++ exception");
  }
}

}  // extern "C"
