/*
 * pkv_block_manager.h -- C ABI of the host-side block manager in
 * libpagedkv.so: the allocator that produces the block_table and
 * slot_mapping arrays the attention calls of include/pagedkv.h consume.
 *
 * The pool of num_blocks blocks of block_size tokens is allocated once (the
 * "Paged KV infra" page, section 2.3: a pre-allocated page pool with a free
 * list; the vLLM-on-CANN page's PagedKVCache: free_blocks, allocate_slots).
 * A sequence of n tokens holds ceil(n / block_size) blocks (vLLM-on-CANN
 * page) and token pos lives at slot table[pos / bs] * bs + pos % bs (skill
 * page, section 3.1).
 *
 *  - Allocation takes the lowest-numbered free block (the ATB PagedAttention
 *    page's allocator scans for the first free page).
 *  - Blocks are reference counted (ATB page, "page reference counting"): a
 *    new block has count 1, pkv_bm_fork() shares every block of a sequence
 *    with a new one (+1 each), freeing a sequence releases its blocks (-1)
 *    and a block returns to the free list at 0.
 *  - Copy-on-write (ATB page, ExtendKVPage): appending to a sequence whose
 *    last block is partly filled and shared first moves the sequence to a
 *    fresh block and records the pair (old, new). The pool lives on the
 *    device, so the caller takes the pairs (pkv_bm_take_copies) and applies
 *    them with paged_kv_copy_blocks() before writing the tokens whose slots
 *    were returned since the previous take. Until taken, the blocks of a
 *    pending pair are not handed out again, and an append that would copy
 *    from a pending destination returns PKV_ERR_PENDING_COPY.
 *  - An append that needs more blocks than can be handed out changes nothing
 *    and returns PKV_ERR_NO_BLOCKS.
 *
 * All pointers here are HOST pointers. A manager is not thread-safe: one
 * thread (the scheduler) owns it. Statuses are those of include/pagedkv.h.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* A manager for blocks 0 .. num_blocks-1 of block_size tokens; NULL if
 * num_blocks <= 0, block_size not in {16, 32, 64, 128}, num_blocks *
 * block_size > INT32_MAX, or memory is short. Destroy with pkv_bm_destroy. */
pkv_block_manager* pkv_bm_create(int64_t num_blocks, int32_t block_size);
void pkv_bm_destroy(pkv_block_manager* bm);

/* A new empty sequence; PKV_ERR_SHAPE if seq_id exists. */
int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id);

/* child_id becomes a sequence sharing all of parent_id's blocks and its
 * length; PKV_ERR_SHAPE if the parent is unknown or the child exists. */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Extend seq_id by num_tokens (>= 0) tokens and write their slots to
 * slots_out[0 .. num_tokens-1] (may be NULL when num_tokens is 0).
 * PKV_ERR_SHAPE: unknown sequence or num_tokens < 0; PKV_ERR_NO_BLOCKS and
 * PKV_ERR_PENDING_COPY as above; on any error nothing changes. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens, int32_t* slots_out);

/* One scheduler step: pkv_bm_append(seq_ids[i], tokens_each, slots_out +
 * i * tokens_each) for i = 0, 1, ... in order, stopping at the first call
 * that fails. Returns the number of sequences extended (num_seqs on
 * success); the failing sequence's status is what pkv_bm_append would return
 * for it now. A negative return is a status for invalid arguments. */
int64_t pkv_bm_append_each(pkv_block_manager* bm, const int64_t* seq_ids, int64_t num_seqs,
                           int64_t tokens_each, int32_t* slots_out);

/* Release every block of seq_id and forget it; PKV_ERR_SHAPE if unknown. */
int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/* Blocks whose reference count is 0 (including any held back by pending
 * copies); the number a leak check watches (the "Paged KV infra" page,
 * section 5.5, monitors the free-page count). */
int64_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);

/* Length of seq_id in tokens, or -1 if unknown. */
int64_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq_id);

/* Reference count of a block, or -1 outside the pool. */
int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block);

/* Fill table_out [num_seqs, max_blocks_per_seq] (row-major int32, -1 past a
 * sequence's blocks) and lens_out [num_seqs] for the given sequences: the
 * block_table / context_lens arguments of the attention calls. PKV_ERR_SHAPE
 * if a sequence is unknown or holds more than max_blocks_per_seq blocks
 * (nothing is written then). */
int pkv_bm_block_table(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t* table_out, int32_t* lens_out);

/* Number of (source, destination) block copies recorded and not yet taken. */
int64_t pkv_bm_num_pending_copies(const pkv_block_manager* bm);

/* Move every pending copy, in the order recorded, to pairs_out [n, 2] and
 * return n (>= 0); PKV_ERR_SHAPE if more than max_pairs are pending (nothing
 * is taken then). */
int64_t pkv_bm_take_copies(pkv_block_manager* bm, int32_t* pairs_out, int64_t max_pairs);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
