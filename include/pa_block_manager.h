/*
 * pa_block_manager.h — host-side KV block manager of libpa (C ABI).
 *
 * The block manager hands out the fixed-size blocks of one KV pool to
 * sequences, frees them when a request ends and hands them out again
 * ("Nano-vLLM：轻量高效的大模型推理框架…", 三.1 推理引擎架构, 块管理器). With prefix
 * caching on, every full block carries a hash chained over the token ids of all
 * blocks before it; a new sequence whose leading full blocks hash (and compare)
 * equal to cached ones reuses them instead of recomputing their KV (same page,
 * 三.2 (1) 前缀缓存). Blocks can be shared within and across requests through
 * the block tables ("DeepSeek复刻vLLM反超原版：AI推理新标杆", section vLLM：大模型
 * 推理的加速引擎与挑战); a forked sequence shares all blocks and gets a private copy
 * of a shared last block before writing into it (copy-on-write).
 *
 * Its output is what the kernels in pa.h consume: a block-table row per
 * sequence and the slot of every token (slot = block * block_size + offset).
 *
 * Conventions: host memory only; all pointers are read or written during the
 * call. A manager is not thread-safe (one caller at a time). Sequences are
 * named by int64 ids the manager returns. Status codes are pa.h's, plus
 * PA_ERR_NO_BLOCKS (the pool cannot hold the request; nothing was changed) and
 * PA_ERR_NOT_FOUND (unknown sequence id).
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager for a pool of num_blocks blocks of block_size tokens.
 * enable_prefix_caching: 0 or 1. *out receives the handle. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_caching,
                       pa_block_manager** out);

/* Releases the manager (NULL is ignored). */
void pa_bm_destroy(pa_block_manager* bm);

/* Blocks with no owner (including freed blocks still kept for prefix reuse). */
int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/* Adds a sequence holding num_tokens prompt tokens (token ids, used for prefix
 * hashing) and gives it ceil(num_tokens / block_size) blocks. Leading full
 * blocks whose hash chain and token ids match cached blocks are reused;
 * *num_cached_tokens receives how many leading tokens already have their KV in
 * the pool (a multiple of block_size), so only the rest needs computing and
 * storing. Fails with PA_ERR_NO_BLOCKS, changing nothing, if the pool is short. */
pa_status pa_bm_add_sequence(pa_block_manager* bm, const int32_t* tokens, int32_t num_tokens,
                             int64_t* seq_id, int32_t* num_cached_tokens);

/* Appends one token to a sequence and returns its slot. A new block is taken
 * when the last one is full. If the last block is shared (after pa_bm_fork) it
 * is first replaced by a private copy: *cow_src / *cow_dst receive the block to
 * copy from / to (both -1 when no copy is needed); the caller must copy it on
 * the GPU (pa_copy_blocks) before writing the token's KV. */
pa_status pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int32_t token, int32_t* slot,
                             int32_t* cow_src, int32_t* cow_dst);

/* A new sequence sharing every block (and token) of seq_id. */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t seq_id, int64_t* new_seq_id);

/* Ends a sequence: its blocks lose one owner each; blocks left without owner
 * become free, and cached ones stay reusable until they are handed out again
 * (least recently freed first). */
pa_status pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);

/* Token count and block count of a sequence. */
pa_status pa_bm_sequence_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                              int32_t* num_blocks);

/* Writes the sequence's block-table row: its blocks, then pad_block up to
 * max_blocks entries. PA_ERR_SHAPE if the sequence has more than max_blocks. */
pa_status pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* row,
                            int32_t max_blocks, int32_t pad_block);

/* Writes the slots of positions first_pos .. first_pos+count-1 of the sequence. */
pa_status pa_bm_slots(const pa_block_manager* bm, int64_t seq_id, int32_t first_pos, int32_t count,
                      int32_t* slots);

/* Owner count of a block (0 for a free block); -1 for an id outside the pool. */
int32_t pa_bm_block_refcount(const pa_block_manager* bm, int32_t block);

/* GPU: copies whole blocks (every KV head, K and V) inside one pool.
 *   pairs      device int32 [num_pairs][2] = {source block, destination block}
 * Destinations must be distinct and differ from every source; the pool layout
 * and dtype come from `cache`. Enqueued on `stream`. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                         const pa_cache_desc* cache, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
