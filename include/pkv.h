/*
 * pkv -- paged KV-cache decode attention and cache maintenance for MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no C++ or framework types cross it.
 *
 * Storage layout of the KV cache (the "Vllm" page of the yang20150702 agent
 * guide, section "CacheEngine"): with x = 16 / sizeof(element),
 *   key block   [num_kv_heads, head_size / x, block_size, x]
 *   value block [num_kv_heads, head_size, block_size]
 * and the pool of physical blocks is the outermost dimension:
 *   key_cache   [num_blocks, num_kv_heads, head_size / x, block_size, x]
 *   value_cache [num_blocks, num_kv_heads, head_size, block_size]
 * Token t of sequence b is at physical block block_tables[b][t / block_size],
 * offset t % block_size (the mlqm.cn vLLM explainer, "PagedAttention"
 * block-table description).  A slot is block * block_size + offset (the
 * tiemojia.cn vLLM 0.10 article, section 3.3 "KV Manager").
 *
 * Common rules for every call:
 *  - Every pointer named "device" must be device memory of the current HIP
 *    device; the caller owns all buffers.  The library allocates and frees
 *    nothing during a call and keeps no device state between calls.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work on it and return; nothing waits for the GPU, except that
 *    pkv_swap_blocks reads its host-side block list before returning.
 *  - Return value: PKV_OK (0) or a negative PKV_ERR_* code; then nothing was
 *    enqueued and pkv_last_error() gives a message for the calling thread.
 *  - No exception crosses the ABI.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types; x = 16 / sizeof: 4 for PKV_F32, 8 for PKV_F16 and PKV_BF16 */
enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 };

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,   /* a size or id out of range, or inconsistent */
  PKV_ERR_UNSUPPORTED = -2,   /* valid but not built: head_size, block_size, group size */
  PKV_ERR_NULL_POINTER = -3,
  PKV_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required */
  PKV_ERR_HIP = -5,           /* a HIP runtime call failed (message has the HIP error) */
  PKV_ERR_NOT_PINNED = -6     /* swap_blocks host side is not page-locked host memory */
};

enum pkv_swap_direction { PKV_SWAP_IN = 0 /* host -> device */, PKV_SWAP_OUT = 1 /* device -> host */ };

/*
 * Single-query decode attention over the paged cache (PagedAttention).
 *
 * Computes, for every sequence b and query head h (the "Vllm" page, section
 * "transformer": softmax(Q K^T / sqrt(d_k)) V, one query row per sequence at
 * decode time):
 *   g = h / (num_heads / num_kv_heads)           (grouped-query head map)
 *   s_t = scale * sum_d query[b][h][d] * K_b[t][g][d],  t < context_lens[b]
 *   out[b][h][:] = sum_t softmax(s)_t * V_b[t][g][:]
 * where K_b, V_b are the sequence's tokens reached through block_tables.
 * Accumulation is fp32; out is rounded to the element type (round to nearest
 * even).  context_lens[b] == 0 gives out[b] = 0.
 *
 * Long contexts are split (split-K decoding, the "Vllm" page, "Prefill vs
 * decoding" item 5 on FlashDecoding): each sequence into whole partitions of P
 * = partition_size tokens, and the tokens after its last whole partition into
 * chunks of at most Q = ceil(P / 2) tokens rounded up to whole blocks (short work
 * items for the end of the call).  Each piece is handled by its own
 * workgroup per KV head; a sequence with several pieces gets its output from
 * a second kernel that merges them in token order with the log-sum-exp rule.
 * The call is bit-identical to pkv_paged_attention_partitions followed by
 * pkv_paged_attention_reduce.
 *
 * Arguments (device unless stated):
 *   out          [num_seqs, num_heads, head_size] element type, written
 *   query        [num_seqs, num_heads, head_size] element type
 *   key_cache    [num_blocks, num_kv_heads, head_size/x, block_size, x]
 *   value_cache  [num_blocks, num_kv_heads, head_size, block_size]
 *   block_tables int32 [num_seqs, max_num_blocks_per_seq]; entries past
 *                ceil(context_lens[b] / block_size) are never used as block ids
 *                (they may be read, inside the row)
 *   context_lens int32 [num_seqs]; each must be <= max_context_len and
 *                <= max_num_blocks_per_seq * block_size (larger values are
 *                clamped to those bounds: no fault, but the result is then
 *                that of the clamped length)
 *   scale        host float, usually 1/sqrt(head_size)
 *   head_size    64 or 128;  block_size 8, 16 or 32
 *   num_heads    a multiple of num_kv_heads; group size num_heads/num_kv_heads
 *                in {1, 2, 4, 8} for PKV_F32, 1..16 for PKV_F16/PKV_BF16
 *   max_context_len  host upper bound of context_lens (sizes the grid)
 *   partition_size   0 = auto: 2048 for PKV_F16/PKV_BF16 with block_size >= 16,
 *                4096 instead with block_size 32 when max_context_len >= 32768,
 *                else 1024; otherwise a multiple of block_size in
 *                [block_size, 4096], at most 128 blocks for PKV_F16/PKV_BF16;
 *                at most 8192 partitions per sequence
 *   workspace    device scratch of at least
 *                pkv_paged_attention_workspace_size(...) bytes, 256-byte
 *                aligned, no initial contents required (it holds the list of
 *                work items built by the call, and the split-K partials);
 *                one call at a time per workspace
 * Physical block ids in block_tables must be valid pool indices: they are
 * not checked on the device.
 */
int pkv_paged_attention_decode(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, float scale, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                               int32_t block_size, int32_t max_num_blocks_per_seq,
                               int32_t max_context_len, int32_t dtype, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch needed by the decode calls (pkv_paged_attention_decode,
 * _partitions + _reduce, _decode_shared): a 256-byte header, an 8 KiB prefetch
 * pad, one int32 per sequence, and per sequence S work items of 16 bytes and,
 * per (sequence, query head), S fp32 running maxima, S fp32 running sums and
 * S * head_size fp32 partial outputs, where S = ceil(max_context_len / P') + 4
 * with P' = partition_size, or 1024 for partition_size 0.  Returns 0 for
 * num_seqs == 0 and for invalid arguments. */
size_t pkv_paged_attention_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                          int32_t max_context_len, int32_t partition_size);

/*
 * pkv_paged_attention_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It takes no workspace: the work list and the split-K partials
 * live in a static device array of PKV_NOALLOC_SCRATCH_BYTES (64 MiB) that the
 * library holds on every device it runs on until the process ends.  The call
 * itself allocates and frees nothing.
 *
 * Arguments, result and error codes as for pkv_paged_attention_decode (the same
 * kernels run; the output is bit-identical to it), without workspace and
 * workspace_bytes.  Sizes whose pkv_paged_attention_workspace_size exceeds
 * PKV_NOALLOC_SCRATCH_BYTES are refused with PKV_ERR_WORKSPACE before anything
 * is enqueued.  The first call on a device looks the array's device address up
 * (hipGetSymbolAddress; a failure returns PKV_ERR_HIP).  Every call on one
 * device shares that device's array: calls that can overlap on one device (on
 * different streams, or from several threads) race and must be serialised by
 * the caller.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pkv_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                       int32_t block_size, int32_t max_num_blocks_per_seq,
                                       int32_t max_context_len, int32_t dtype,
                                       int32_t partition_size, void* stream);

/* Bytes of the static scratch of pkv_paged_attention_decode_noalloc
 * (PKV_NOALLOC_SCRATCH_BYTES). */
size_t pkv_paged_attention_noalloc_scratch_bytes(void);

/* The first phase of pkv_paged_attention_decode, alone: the work-list kernel
 * and then one workgroup per (work item, KV head).  Sequences handled by one
 * item get their final output in `out`; the others leave per-item partial
 * results (and their count) in `workspace` for pkv_paged_attention_reduce.
 * Same arguments and rules as pkv_paged_attention_decode. */
int pkv_paged_attention_partitions(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                   int32_t block_size, int32_t max_num_blocks_per_seq,
                                   int32_t max_context_len, int32_t dtype,
                                   int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* pkv_paged_attention_partitions split once more, so that one work list can serve several
 * calls: a decode step's block tables and lengths are the same for every layer of the model,
 * so the list can be built once per step and each layer's attention run on it.
 *   pkv_paged_attention_plan: the work-list kernel alone; it writes the list (and each
 *     sequence's item count) into `workspace`.
 *   pkv_paged_attention_partitions_planned: the attention kernel alone, on the list in
 *     `workspace`; with pkv_paged_attention_reduce after it, bit-identical to
 *     pkv_paged_attention_decode.
 * Both take the arguments and rules of pkv_paged_attention_decode (16- and 32-bit caches).
 * A planned call must use the block_tables, context_lens, num_seqs, num_kv_heads, head_size,
 * block_size, max_num_blocks_per_seq, max_context_len, dtype and partition_size of the plan
 * (query, caches and out may change), unchanged on the device since the plan ran; otherwise
 * the behaviour is undefined.  (The kernel skips list entries that do not fit the call's
 * sequence count, partial slots and length limit, but an entry made for longer contexts would
 * reach block-table entries past a sequence's blocks.)  A workspace no plan has written since
 * it was zeroed holds an empty list: the call then writes nothing. */
int pkv_paged_attention_plan(void* out, const void* query, const void* key_cache,
                             const void* value_cache, const int32_t* block_tables,
                             const int32_t* context_lens, float scale, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                             int32_t block_size, int32_t max_num_blocks_per_seq,
                             int32_t max_context_len, int32_t dtype, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attention_partitions_planned(void* out, const void* query, const void* key_cache,
                                           const void* value_cache, const int32_t* block_tables,
                                           const int32_t* context_lens, float scale,
                                           int32_t num_seqs, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_size,
                                           int32_t block_size, int32_t max_num_blocks_per_seq,
                                           int32_t max_context_len, int32_t dtype,
                                           int32_t partition_size, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* The first calls of a decode step in one launch: pkv_reshape_and_cache of the
 * step's new tokens and pkv_paged_attention_plan.  The two are independent (the
 * plan reads block_tables and context_lens only; the write reads key, value and
 * slot_mapping and writes the caches), so one launch runs the plan in one
 * workgroup and the write in the others, and the short write no longer waits
 * behind the plan (the "Vllm" page, "transformer" decoding paragraph: the new
 * token's K/V are appended, then attended to).  The caches and the workspace
 * end exactly as after pkv_reshape_and_cache followed by
 * pkv_paged_attention_plan; pkv_paged_attention_partitions_planned and
 * pkv_paged_attention_reduce complete the step.
 *   arguments up to workspace_bytes: as for pkv_paged_attention_plan (16- and
 *     32-bit caches; out and query are not read)
 *   key, value, slot_mapping, num_tokens, num_blocks, key_stride, value_stride:
 *     as for pkv_reshape_and_cache, into the same key_cache and value_cache, with
 *     the decode's dtype, num_kv_heads, head_size and block_size
 * Errors as for those two calls; nothing is enqueued when any argument fails. */
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
                                       int64_t value_stride, void* stream);

/* The second kernel alone: for each sequence with more than one work item,
 * out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p with M = max_p m_p,
 * over its items p in token order.  Sequences with one item are left
 * untouched.  Must follow pkv_paged_attention_partitions on the same stream
 * with the same sizes (the workspace holds the counts it reads). */
int pkv_paged_attention_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t head_size, int32_t max_context_len,
                               int32_t dtype, int32_t partition_size, const void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Decode attention for sequences that share a prompt prefix (beam search,
 * parallel sampling): the same result as pkv_paged_attention_decode, but each
 * shared block is read from memory once per group instead of once per
 * sequence.  Sharing is what the block tables express: the members of a group
 * point to the same physical blocks for their first tokens (PagedAttention's
 * memory sharing with reference counts and copy-on-write, the mlqm.cn vLLM
 * explainer, "PagedAttention" and its copy-on-write example; the AIGC
 * interview book section 23, fork / append_slots).  The prefix is cut like a
 * context (whole partitions, then chunks) into items that carry up to
 * 16 / (num_heads / num_kv_heads) members' query rows at once; every member's
 * own tokens follow in items of their own; all partial results of a sequence
 * are merged in token order with the log-sum-exp rule.
 *
 * Arguments as for pkv_paged_attention_decode, plus (device):
 *   group_starts int32 [num_groups + 1]: group g holds sequences
 *                [group_starts[g], group_starts[g + 1]); the groups must cover
 *                0 .. num_seqs - 1 once, in order (group_starts[0] = 0,
 *                non-decreasing, group_starts[num_groups] = num_seqs); a
 *                sequence sharing nothing is a group of one
 *   prefix_lens  int32 [num_groups]: tokens at the start of every member that
 *                lie in the same physical blocks (table entries equal for
 *                tokens below it).  Used as min(prefix_lens[g], each member's
 *                context length) rounded down to a multiple of block_size;
 *                ignored for a group of one.
 *   num_groups   in [1, num_seqs] (any value when num_seqs == 0)
 *   workspace    at least pkv_paged_attention_workspace_size(...) bytes,
 *                256-byte aligned, no initial contents required
 * PKV_F16 and PKV_BF16 only; any group size num_heads/num_kv_heads in 1..16.
 * Group arrays that break the rules above cannot make the call read or write
 * outside its buffers, but the output of a sequence that is not covered
 * exactly once is then unspecified.  Results agree with
 * pkv_paged_attention_decode within rounding; for PKV_F16/PKV_BF16 they are
 * bit-identical to it when every prefix is a multiple of the partition size
 * in use (both calls then cut every sequence at the same tokens and run the
 * same kernel).
 */
int pkv_paged_attention_decode_shared(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const int32_t* group_starts,
                                      const int32_t* prefix_lens, int32_t num_groups, float scale,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_size, int32_t block_size,
                                      int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                      int32_t dtype, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* The shared-prefix decode in two stages, as pkv_paged_attention_plan and
 * pkv_paged_attention_partitions_planned are for the plain one (the groups,
 * tables and lengths of a decode step serve every layer, so one plan serves all
 * of them):
 *   pkv_paged_attention_plan_shared: the work-list kernel alone (prefix items
 *     carry a group's query rows), written into `workspace`;
 *   pkv_paged_attention_partitions_planned_shared: the attention kernel alone on
 *     that list; with pkv_paged_attention_reduce after it (same num_seqs,
 *     num_heads, head_size, max_context_len, dtype, partition_size, workspace),
 *     bit-identical to pkv_paged_attention_decode_shared.
 * Arguments and rules as for pkv_paged_attention_decode_shared.  A planned call
 * must use the plan's group_starts, prefix_lens, num_groups, block_tables,
 * context_lens and sizes, unchanged on the device since the plan ran (query,
 * caches and out may change); otherwise the behaviour is undefined.  A
 * workspace no plan has written since it was zeroed holds an empty list: the
 * call then writes nothing. */
int pkv_paged_attention_plan_shared(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* group_starts,
                                    const int32_t* prefix_lens, int32_t num_groups, float scale,
                                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t block_size,
                                    int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                    int32_t dtype, int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream);
int pkv_paged_attention_partitions_planned_shared(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_starts,
    const int32_t* prefix_lens, int32_t num_groups, float scale, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/* pkv_paged_attention_plan_and_cache for the shared-prefix decode: the write of
 * the step's new tokens (pkv_reshape_and_cache) and pkv_paged_attention_plan_shared
 * in one launch.  The caches and the workspace end exactly as after those two
 * calls; pkv_paged_attention_partitions_planned_shared and
 * pkv_paged_attention_reduce complete the step.  A beam step's copy-on-write
 * (pkv_copy_blocks) must be ordered before this call when a new token lands in
 * a copied block.
 *   arguments up to workspace_bytes: as for pkv_paged_attention_plan_shared
 *   key, value, slot_mapping, num_tokens, num_blocks, key_stride, value_stride:
 *     as for pkv_reshape_and_cache, into the same key_cache and value_cache
 * Errors as for those two calls; nothing is enqueued when any argument fails. */
int pkv_paged_attention_plan_and_cache_shared(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_starts,
    const int32_t* prefix_lens, int32_t num_groups, float scale, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, const void* key,
    const void* value, const int64_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
    int64_t key_stride, int64_t value_stride, void* stream);

/*
 * Decode attention over an 8-bit KV cache: keys and values stored as OCP FP8
 * E4M3 codes with one float scale per cache (key = code * k_scale, value =
 * code * v_scale), the 8-bit KV-cache quantisation the AIGC interview book
 * names for TurboMind (LMDeploy section).  The E4M3 format: sign, 4 exponent
 * bits (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, largest
 * value 448.  Computes the attention of pkv_paged_attention_decode on the
 * dequantised keys and values, with fp32 accumulation.
 *   key_cache    uint8 [num_blocks, num_kv_heads, head_size/16, block_size, 16]
 *                (x = 16 / sizeof = 16)
 *   value_cache  uint8 [num_blocks, num_kv_heads, head_size, block_size]
 *   query, out   PKV_F16 or PKV_BF16 (`dtype`), as for the 16-bit call
 *   k_scale, v_scale  host floats, finite and > 0
 * All other arguments, the partitioning, the workspace
 * (pkv_paged_attention_workspace_size) and the error codes as for
 * pkv_paged_attention_decode, except the partition size: auto is 2048 for
 * every block size (4096 with block_size 16 or 32 when max_context_len >=
 * 32768), and a partition may span up to 256 blocks.  Group sizes
 * 1..16.
 */
int pkv_paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, float k_scale,
                                   float v_scale, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                   int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                   int32_t dtype, int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * The same decode over an 8-bit integer KV cache: keys and values stored as
 * signed integer codes -127 .. 127 (two's-complement bytes; the byte 0x80
 * reads as -128) with one float scale per cache (key = code * k_scale, value
 * = code * v_scale): the symmetric linear reading of the 8-bit KV-cache
 * quantisation the AIGC interview book names for TurboMind and LMDeploy.
 * Layouts, arguments, partitioning, workspace and errors exactly as for
 * pkv_paged_attention_decode_fp8.
 */
int pkv_paged_attention_decode_int8(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, float scale, float k_scale,
                                    float v_scale, int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                    int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                    int32_t dtype, int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* The 8-bit decode in two stages, as pkv_paged_attention_plan and
 * pkv_paged_attention_partitions_planned are for the 16-bit one: the work-list
 * kernel alone (pkv_paged_attention_plan_fp8 / _int8), then the attention
 * kernel alone on that list (pkv_paged_attention_partitions_planned_fp8 /
 * _int8), then pkv_paged_attention_reduce (same num_seqs, num_heads, head_size,
 * max_context_len, dtype, partition_size, workspace): bit-identical to
 * pkv_paged_attention_decode_fp8 / _int8.  Arguments and rules as for those
 * calls; a planned call must use the tables, lengths and sizes of its plan,
 * unchanged on the device since the plan ran (query, caches, scales and out may
 * change), otherwise the behaviour is undefined.  A workspace no plan has
 * written since it was zeroed holds an empty list: the call then writes
 * nothing. */
int pkv_paged_attention_plan_fp8(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, float scale, float k_scale,
    float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attention_partitions_planned_fp8(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, float scale, float k_scale,
    float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attention_plan_int8(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, float scale, float k_scale,
    float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attention_partitions_planned_int8(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, float scale, float k_scale,
    float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/* pkv_paged_attention_plan_and_cache over an 8-bit cache: the write of the
 * step's new tokens (pkv_reshape_and_cache_fp8 / _int8, with the cache's k_scale
 * and v_scale) and pkv_paged_attention_plan_fp8 / _int8 in one launch.  The
 * caches and the workspace end exactly as after those two calls in that order;
 * pkv_paged_attention_partitions_planned_fp8 / _int8 and
 * pkv_paged_attention_reduce complete the step.
 *   arguments up to workspace_bytes: as for pkv_paged_attention_plan_fp8
 *   key, value, slot_mapping, num_tokens, num_blocks, key_stride, value_stride:
 *     as for pkv_reshape_and_cache_fp8, into the same key_cache and value_cache,
 *     fp16 / bf16 keys and values of the decode's dtype, num_kv_heads, head_size
 *     and block_size
 * Errors as for those two calls; nothing is enqueued when any argument fails. */
int pkv_paged_attention_plan_and_cache_fp8(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, float scale, float k_scale,
    float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, const void* key,
    const void* value, const int64_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
    int64_t key_stride, int64_t value_stride, void* stream);
int pkv_paged_attention_plan_and_cache_int8(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, float scale, float k_scale,
    float v_scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t max_context_len, int32_t dtype,
    int32_t partition_size, void* workspace, size_t workspace_bytes, const void* key,
    const void* value, const int64_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
    int64_t key_stride, int64_t value_stride, void* stream);

/*
 * Multi-query paged attention: chunked prefill and mixed prefill / decode
 * batches.  The query rows of num_seqs requests are flattened; request b owns
 * rows [query_start_loc[b], query_start_loc[b + 1]) (the attention metadata of
 * the tiemojia.cn vLLM run-flow article, section 3.5).  Its n rows are the
 * last n positions of its context of L = context_lens[b] tokens (the chunk
 * chunked prefill adds, the AIGC interview book's scheduler note; a decode
 * token is n = 1), so row i (0-based) sits at position p = L - n + i and
 *   out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_t) V_t
 * over the request's own keys and values (block table row b, GQA head map
 * h / (num_heads / num_kv_heads), layouts as for the decode).  The chunk's
 * own keys and values must already be in the cache (pkv_reshape_and_cache).
 *   query, out        device [num_tokens, num_heads, head_size], PKV_F16 or
 *                     PKV_BF16 (`dtype`); fp32 accumulation, weights rounded
 *                     once to dtype, output rounded to nearest even
 *   query_start_loc   device int32 [num_seqs + 1], 0 = first, last = num_tokens
 *   context_lens      device int32 [num_seqs], each <= max_context_len
 *   block_tables      device int32 [num_seqs, max_num_blocks_per_seq],
 *                     max_num_blocks_per_seq * block_size >= max_context_len
 *   scale             finite and > 0
 *   partition_size    0 (auto: 8192) or a multiple of 32 in [32, 8192]: the
 *                     keys of a query tile are cut at multiples of it and the
 *                     pieces merged by a split-K reduce
 *   workspace         device, 256-byte aligned, at least
 *                     pkv_paged_attention_prefill_workspace_size(...) bytes
 * head_size 64 or 128, block_size 8, 16 or 32, group size 1..16.  A request
 * whose metadata is inconsistent on the device (decreasing offsets, rows past
 * num_tokens, n > L, L > max_context_len) is skipped: its rows are left as
 * they were.  Rows of an n = 0 request do not exist.  Errors as for the
 * decode; PKV_ERR_UNSUPPORTED for PKV_F32.
 */
size_t pkv_paged_attention_prefill_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                                  int32_t num_heads, int32_t num_kv_heads,
                                                  int32_t head_size, int32_t max_context_len,
                                                  int32_t partition_size);
int pkv_paged_attention_prefill(void* out, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                float scale, int32_t num_seqs, int32_t num_tokens,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                int32_t block_size, int32_t max_num_blocks_per_seq,
                                int32_t max_context_len, int32_t dtype, int32_t partition_size,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same multi-query attention over an 8-bit (FP8 E4M3) KV cache, in the layouts and with
 * the per-cache scales of pkv_paged_attention_decode_fp8 (key = code x k_scale, value =
 * code x v_scale; k_scale, v_scale host floats, finite and > 0).  query and out stay PKV_F16
 * or PKV_BF16 (`dtype`); the chunk's keys and values must already be in the cache
 * (pkv_reshape_and_cache_fp8).  Everything else -- rows, partitioning, workspace
 * (pkv_paged_attention_prefill_workspace_size), errors -- as for pkv_paged_attention_prefill.
 */
int pkv_paged_attention_prefill_fp8(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* query_start_loc,
                                    float scale, float k_scale, float v_scale, int32_t num_seqs,
                                    int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t block_size,
                                    int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                    int32_t dtype, int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * The same multi-query attention over an 8-bit integer KV cache (codes and scales of
 * pkv_paged_attention_decode_int8; the chunk written by pkv_reshape_and_cache_int8).
 * Everything else as for pkv_paged_attention_prefill_fp8.
 */
int pkv_paged_attention_prefill_int8(void* out, const void* query, const void* key_cache,
                                     const void* value_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* query_start_loc,
                                     float scale, float k_scale, float v_scale, int32_t num_seqs,
                                     int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_size, int32_t block_size,
                                     int32_t max_num_blocks_per_seq, int32_t max_context_len,
                                     int32_t dtype, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Measurement aid (not part of the attention path): read `bytes` of device memory at `src`
 * with the non-temporal 16-byte loads the decode kernels use for the KV cache, as fast as the
 * memory system allows, to measure the achievable HBM read ceiling on the running GPU.
 * `sink` is a device word the kernel may write (practically never).  src and bytes must be
 * multiples of 16.  Asynchronous on `stream`; errors as elsewhere.
 */
int pkv_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/*
 * Scatter new tokens' keys and values into their cache slots (the KV-cache
 * write of the cybasar.com nano-vLLM article, section 5.2.3, in the block
 * layout above):
 *   blk = slot_mapping[i] / block_size, off = slot_mapping[i] % block_size
 *   key_cache[blk][h][d / x][off][d % x] = key[i][h][d]
 *   value_cache[blk][h][d][off]          = value[i][h][d]
 * A negative slot means "skip this token" (the article's -1 sentinel).  Slots
 * >= num_blocks * block_size are also skipped (never written).
 *   key, value   device, token i's row starts at element i * key_stride
 *                (value_stride); inside a row heads are contiguous, then dims
 *                (the article's stride asserts: stride(-1) == 1,
 *                stride(1) == head_size)
 *   slot_mapping device int64 [num_tokens]
 * Bit-exact copy; no arithmetic on the values.  Distinct tokens must name
 * distinct slots (otherwise which one lands is unspecified).
 */
int pkv_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_size, int32_t block_size, int64_t num_blocks,
                          int64_t key_stride, int64_t value_stride, int32_t dtype, void* stream);

/*
 * pkv_reshape_and_cache into an 8-bit cache (layouts of
 * pkv_paged_attention_decode_fp8): each element x of key / value (PKV_F16 or
 * PKV_BF16, `dtype`) is stored as the E4M3 code of clamp(x / scale, -448,
 * 448), the division rounded to float32 and the conversion to the nearest
 * code, ties to even; a NaN input gives a NaN code.  Slots, strides, skipping
 * and errors as for pkv_reshape_and_cache; head_size a multiple of 16;
 * key_cache 16-byte aligned.
 */
int pkv_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                              void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                              int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                              int32_t dtype, float k_scale, float v_scale, void* stream);

/*
 * pkv_reshape_and_cache into an 8-bit integer cache (codes of
 * pkv_paged_attention_decode_int8): each element x is stored as the integer
 * nearest to x / scale (the division rounded to float32; ties to even),
 * clamped to [-127, 127]; a NaN input gives code 0.  Everything else as for
 * pkv_reshape_and_cache_fp8.
 */
int pkv_reshape_and_cache_int8(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                               int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                               int32_t dtype, float k_scale, float v_scale, void* stream);

/*
 * Copy whole blocks inside the device cache, for every layer (CacheEngine
 * "copy", the "Vllm" page, section "CacheEngine"; the pairs come from the
 * block manager's copy-on-write, the AIGC interview book section 23,
 * append_slots).
 *   key_cache_ptrs, value_cache_ptrs  device uint64 [num_layers]: the base
 *                address of each layer's key / value cache
 *   block_mapping device int64 [num_pairs, 2] = (src, dst)
 *   block_bytes   bytes of one block of one cache (a multiple of 16); the
 *                 same for keys and values
 *   num_blocks    blocks per layer cache; pairs with an id outside
 *                 [0, num_blocks) are skipped
 * dst ids must be distinct and no dst may also be a src in the same call
 * (a copy-on-write destination is always a fresh block); otherwise the
 * result is unspecified.  Bit-exact.
 */
int pkv_copy_blocks(const uint64_t* key_cache_ptrs, const uint64_t* value_cache_ptrs,
                    int32_t num_layers, const int64_t* block_mapping, int32_t num_pairs,
                    int64_t block_bytes, int64_t num_blocks, void* stream);

/*
 * Move blocks between the device cache and a page-locked host cache
 * (CacheEngine swap_in = host -> device, swap_out = device -> host; the
 * host cache is pinned memory, the "Vllm" page, "CacheEngine").  Called once
 * for keys and once for values.
 *   dst, src       base addresses; for PKV_SWAP_IN src is pinned host memory
 *                  and dst device memory, for PKV_SWAP_OUT the reverse
 *   block_mapping  HOST int64 [num_pairs, 2] = (src block, dst block), read
 *                  before the call returns
 *   src_num_blocks, dst_num_blocks  pool sizes, for range checks
 * When the device addresses the pinned memory at the host pointer itself
 * (mapped host memory; both bases 8-byte aligned, block_bytes a multiple
 * of 8), one kernel launch moves up to 112 blocks, the pair list passed in
 * its arguments; otherwise runs of consecutive ids become one asynchronous
 * copy each.  Returns PKV_ERR_NOT_PINNED if the host side is not page-locked
 * host memory and PKV_ERR_INVALID_ARG for an id out of range.  The host
 * buffer must stay alive and untouched until the stream has passed the
 * call's work.
 */
int pkv_swap_blocks(void* dst, const void* src, const int64_t* block_mapping, int32_t num_pairs,
                    int64_t block_bytes, int64_t src_num_blocks, int64_t dst_num_blocks,
                    int32_t direction, void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
