/*
 * pkv block manager -- host-side bookkeeping of the paged KV cache: which
 * physical blocks each sequence owns, with reference counts, copy-on-write,
 * fork and swap planning.  It decides; the cache operations of pkv.h move the
 * data (pkv_reshape_and_cache for the new token's slot, pkv_copy_blocks for
 * the copy-on-write pairs, pkv_swap_blocks for the swap pairs).  Host memory
 * only; nothing here touches the GPU.
 *
 * Model (the BlockSpaceManager of the AIGC interview book, section 23, and the
 * "Vllm" page, "Scheduler & BlockSpaceManager"; copy-on-write as in the
 * mlqm.cn explainer's "PagedAttention" worked example):
 *  - two pools of physical blocks, GPU ids [0, num_gpu_blocks) and CPU ids
 *    [0, num_cpu_blocks), each block with a reference count; a pool hands out
 *    its lowest free id first;
 *  - each sequence (an int64 id chosen by the caller) has a length in tokens
 *    and a block table: logical block j -> physical block, all on one device;
 *    token t lives in table[t / block_size] at offset t % block_size;
 *  - allocate: a new sequence of n tokens takes ceil(n / block_size) fresh
 *    GPU blocks (reference count 1);
 *  - fork: a child sequence shares every block of its parent (each block's
 *    count + 1), as beam search or parallel sampling do;
 *  - append: the sequence grows by one token; if that token needs a new
 *    logical block, a fresh block is appended; otherwise, if the last block
 *    is shared (count > 1), it is copied first (copy-on-write): a fresh block
 *    replaces it in this sequence's table, the old block's count drops by 1,
 *    and the pair (old, new) must be copied before the token is written;
 *  - free: every block of the sequence loses one reference; blocks that reach
 *    0 return to their pool;
 *  - swap out / in: all blocks of a set of sequences move to the other pool;
 *    a block shared by several of them moves once and keeps its count.
 *
 * Calls return PKV_OK (0) or a negative PKV_ERR_* code of pkv.h; on error
 * nothing changed.  pkv_last_error() gives the message.  A manager is not
 * thread-safe: one caller at a time.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

enum pkv_alloc_status { PKV_ALLOC_OK = 0, PKV_ALLOC_LATER = 1, PKV_ALLOC_NEVER = 2 };
enum pkv_device { PKV_DEVICE_GPU = 0, PKV_DEVICE_CPU = 1 };

/* New manager; watermark is the fraction of GPU blocks kept free when new
 * sequences are admitted (pkv_bm_can_allocate).  NULL on invalid arguments. */
pkv_block_manager* pkv_bm_create(int32_t block_size, int32_t num_gpu_blocks,
                                 int32_t num_cpu_blocks, float watermark);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Admission of a new sequence of num_tokens: PKV_ALLOC_NEVER if even an empty
 * pool could not hold it above the watermark, PKV_ALLOC_OK if the free GPU
 * blocks minus its blocks stay at or above the watermark, else PKV_ALLOC_LATER. */
int pkv_bm_can_allocate(const pkv_block_manager* bm, int32_t num_tokens);
/* Give sequence seq_id (new) num_tokens tokens in fresh GPU blocks. */
int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq_id, int32_t num_tokens);
/* child (new) shares all of parent's blocks and has its length. */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);
/* 1 if num_seqs sequences can each append a token now (one free GPU block each
 * in the worst case), else 0. */
int pkv_bm_can_append(const pkv_block_manager* bm, int32_t num_seqs);
/* One new token for a GPU-resident sequence.  *slot receives its slot
 * (block * block_size + offset); *cow_src / *cow_dst the copy-on-write pair,
 * or -1 / -1 when no copy is needed.  PKV_ERR_WORKSPACE if no GPU block is free. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int64_t* slot, int64_t* cow_src,
                  int64_t* cow_dst);
/* Drop the sequence and its references. */
int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id);
/* Move the blocks of seq_ids[0..n) (all on the GPU) to the CPU pool, or back.
 * pairs receives (from, to) block ids, at most cap pairs; *num_pairs their
 * count.  PKV_ERR_WORKSPACE if the target pool or `pairs` is too small. */
int pkv_bm_swap_out(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n, int64_t* pairs,
                    int32_t cap, int32_t* num_pairs);
int pkv_bm_swap_in(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n, int64_t* pairs,
                   int32_t cap, int32_t* num_pairs);

/* Queries.  pkv_bm_block_table copies up to cap ids into table (int32, the
 * block_tables row format of pkv_paged_attention_decode) and the count into *n. */
int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table, int32_t cap,
                       int32_t* n);
/* length in tokens (>= 0), or a negative PKV_ERR_* code */
int64_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id);
/* PKV_DEVICE_GPU / PKV_DEVICE_CPU, or a negative PKV_ERR_* code */
int pkv_bm_seq_device(const pkv_block_manager* bm, int64_t seq_id);
/* free blocks of a pool, or a negative PKV_ERR_* code */
int32_t pkv_bm_num_free(const pkv_block_manager* bm, int32_t device);
/* reference count of a block (0 = free), or a negative PKV_ERR_* code */
int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t device, int32_t block);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
