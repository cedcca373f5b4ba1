/*
 * pagedkv.h -- C ABI of libpagedkv.so: attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The KV cache is a pool of fixed-size physical blocks shared by every
 * sequence. A sequence reaches its tokens through a row of `block_table`
 * (logical block -> physical block id) and a length. Token `pos` of
 * sequence `b` lives at
 *     slot = block_table[b, pos / block_size] * block_size + pos % block_size
 * ("model-infer-kvcache" skill page, section 3.1, physical layout and
 * logical mapping). New tokens are written by slot (`slot_mapping`, same
 * page, section 3.3); attention reads them back through `block_table`.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensor arguments are DEVICE pointers owned by the caller. The library
 *    never frees, retains or allocates memory.
 *  - All tensors are dense, row-major (C order), with no padding. Tensor
 *    data pointers (queries, outputs, keys / values, the pool) are 16-byte
 *    aligned, as device allocations are: the kernels move 16-byte pieces.
 *    A call given one that is not returns PKV_ERR_UNSUPPORTED.
 *  - Pool layout (k_cache and v_cache alike): [num_blocks, block_size,
 *    num_kv_heads, head_dim]. Slot s is row s of the pool viewed as
 *    [num_blocks * block_size, num_kv_heads * head_dim].
 *  - Integer metadata (block_table, context_lens, seq_lens, slot_mapping,
 *    cu_seqlens_q) is int32. The skill page's notes require an int32
 *    block_table.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it and returns; it never synchronises the device.
 *    Ordering between calls (write before read) is the stream's order.
 *  - Return value: PKV_OK (0) on success, or a negative pkv_status. A
 *    negative status means nothing was launched, except PKV_ERR_HIP, which
 *    reports a failed launch. pkv_status_string() describes a status.
 *  - Supported: head_dim in {64, 128}; block_size in {16, 32, 64, 128};
 *    num_q_heads a positive multiple of num_kv_heads; num_blocks *
 *    block_size <= INT32_MAX.
 *  - Device-side contents are the caller's contract: block ids in
 *    [0, num_blocks) for every block a sequence uses, context lengths
 *    <= max_blocks_per_seq * block_size, cu_seqlens_q non-decreasing from 0
 *    to total_q, slots unique. The kernels clamp what they read to the pool
 *    and the table so that a violation never makes them access memory
 *    outside the buffers, but the numerical result of such a call is
 *    unspecified.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, out, key, value and the pool. */
typedef enum {
  PKV_F32 = 0,  /* IEEE binary32 */
  PKV_F16 = 1,  /* IEEE binary16 */
  PKV_BF16 = 2, /* bfloat16 (upper half of a binary32) */
  PKV_I8 = 3    /* int8 codes (accepted where a call says so) */
} pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  PKV_ERR_DTYPE = -3,       /* dtype code unknown or not accepted by this call */
  PKV_ERR_UNSUPPORTED = -4, /* head_dim / block_size / GQA group outside the supported
                               set, or a tensor pointer not 16-byte aligned */
  PKV_ERR_WORKSPACE = -5,   /* decode workspace missing or too small */
  PKV_ERR_HIP = -6,         /* the HIP runtime rejected a launch */
  PKV_ERR_NO_BLOCKS = -7,   /* block manager: not enough free blocks */
  PKV_ERR_PENDING_COPY = -8, /* block manager: take and apply pending block copies first */
  PKV_ERR_SCRATCH = -9       /* paged_kv_write_decode_noalloc: partials exceed its scratch */
} pkv_status;

/*
 * paged_kv_write -- scatter new K/V tokens into the pool by slot.
 *
 * For every t < num_tokens with s = slot_mapping[t] >= 0, copies key[t]
 * into k_cache row s and value[t] into v_cache row s (all kv heads, all
 * dims). A bit copy: no rounding, NaN payloads preserved. Tokens with a
 * negative slot are skipped (a -1 entry marks "no slot"; the "Paged KV infra"
 * page initialises unused table entries to -1). Slots >= num_blocks *
 * block_size are skipped too. Duplicate slots race; which token lands is
 * unspecified. Defined by the skill page, section 3.3 (slot_mapping drives
 * the cache write) and section 3.1 (slot -> block, offset).
 *
 *   k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim], dtype
 *   key, value       : [num_tokens, num_kv_heads, head_dim], dtype
 *   slot_mapping     : [num_tokens] int32
 *   num_tokens       : >= 0 (0 is a no-op that returns PKV_OK)
 */
int paged_kv_write(void* k_cache, void* v_cache, const void* key, const void* value,
                   const int32_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                   void* stream);

/*
 * paged_attention_decode_workspace_size -- bytes of device workspace that
 * paged_attention_decode needs for these sizes: the split-KV partial results,
 * one (max, sum, unnormalised output) triple per sequence, query head and
 * context partition, fp32. Partitions are counted at 512 tokens, or at 128
 * tokens for small problems (num_seqs x num_q_heads x ceil(max_blocks_per_seq
 * x block_size / 512) < 4096), where the call may split contexts finer to
 * give every compute unit work; then one 8-byte exchange word per sequence
 * and query head (the hand-over of paired rows, below). Returns 0 when no
 * workspace is needed (contexts of at most one partition) and for invalid
 * sizes.
 */
size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_blocks_per_seq,
                                             int32_t block_size);

/*
 * paged_attention_decode -- one query token per sequence attends over its
 * paged context.
 *
 * For sequence b and query head h (kv head h / (num_q_heads / num_kv_heads)):
 *   out[b, h] = sum_j softmax_j(scale * <q[b, h], K_j>) * V_j
 * over the context_lens[b] tokens j read through block_table[b]. A context
 * length of 0 gives an all-zero output row. This is the decode setting of the
 * skill page (Appendix C, sparse_mode 0: no mask, the KV length alone bounds
 * the keys; section 3.6: the KV length includes the token just written), and
 * the per-page attention of the "ATB PagedAttention" page. Long contexts are
 * split into partitions whose partial softmax results are merged exactly
 * (the vLLM-on-CANN page: scattered blocks are merged block by block with an
 * online softmax). When every context fits one workgroup and the batch has
 * 2 to 64 sequences, rows of unequal length are paired (longest with
 * shortest) and the longer row's tail is attended by the shorter row's
 * workgroup; the two partial results are merged the same way, in the call.
 *
 *   out              : [num_seqs, num_q_heads, head_dim], dtype (written)
 *   q                : [num_seqs, num_q_heads, head_dim], dtype
 *   k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim], dtype
 *   block_table      : [num_seqs, max_blocks_per_seq] int32
 *   context_lens     : [num_seqs] int32, each in [0, max_blocks_per_seq*block_size]
 *   scale            : softmax scale (1/sqrt(head_dim) in the pages' usage)
 *   workspace        : device scratch of workspace_bytes bytes, where
 *                      workspace_bytes >= paged_attention_decode_workspace_size(...)
 *                      (may be NULL when that size is 0). Its contents on
 *                      entry do not matter; it is clobbered, except that
 *                      every call leaves the exchange words zero. (Each call
 *                      tags the words with a number unique to the call, so
 *                      stale contents are told apart; a replayed graph
 *                      reuses its number and relies on the words being
 *                      zero.) Calls that share a workspace must be ordered
 *                      on one stream.
 * Accepts dtype PKV_F32, PKV_F16, PKV_BF16. Accumulation is fp32.
 */
int paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* context_lens,
                           int32_t block_size, float scale, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_write_decode -- one decode step: the new token of every sequence
 * is written into the pool (paged_kv_write) and then attended over
 * (paged_attention_decode), in a single launch.
 *
 * Equivalent to paged_kv_write(k_cache, v_cache, key, value, slot_mapping,
 * num_seqs, ...) followed by paged_attention_decode(...) on the same
 * arguments, the sequence of the skill page's section 3.6 (the KV length
 * includes the token just written). Token b of key/value is sequence b's
 * new token and normally sits at its last position, context_lens[b] - 1:
 * when slot_mapping[b] is the table's slot of that position, the attention
 * takes the token's K/V from key/value directly (the values the write stores
 * there), so no part of the call waits for the store. Precondition for the
 * equivalence: no sequence of the call reads a slot written by the call
 * other than at that position (a sequence's last block is its own).
 * Rounding may differ from the two separate calls in the last bits.
 *
 *   out, q, block_table, context_lens, scale, workspace : as paged_attention_decode
 *   k_cache, v_cache : the pool (written: the new rows)
 *   key, value       : [num_seqs, num_kv_heads, head_dim], dtype
 *   slot_mapping     : [num_seqs] int32; negative or >= num_blocks*block_size
 *                      entries are skipped, as in paged_kv_write
 *   workspace_bytes  : >= paged_attention_decode_workspace_size(...)
 * Accepts dtype PKV_F32, PKV_F16, PKV_BF16 (for PKV_F32 the library runs the
 * write and the decode as two launches).
 */
int paged_kv_write_decode(void* out, const void* q, void* k_cache, void* v_cache,
                          const void* key, const void* value, const int32_t* slot_mapping,
                          const int32_t* block_table, const int32_t* context_lens,
                          int32_t block_size, float scale, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_write_decode_noalloc -- paged_kv_write_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, semantics and results as paged_kv_write_decode (the same
 * kernels), without the workspace pair: the split-KV partials go to a
 * device array that the library holds, PKV_NOALLOC_SCRATCH_BYTES (64 MiB)
 * on each GPU it runs on, from the first call on that GPU until the process
 * ends. That first call looks the array's address up (hipGetSymbolAddress,
 * for the device of `stream`); no call allocates or frees device or host
 * memory. Calls whose partials need more than the array,
 * paged_attention_decode_workspace_size(...) > PKV_NOALLOC_SCRATCH_BYTES,
 * return PKV_ERR_SCRATCH and launch nothing.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's partials (each call writes every partial it reads, so nothing
 * needs clearing) and its exchange words, zero at load and left zero by
 * every call. Calls that may overlap on one GPU -- on different
 * streams, or from different host threads without ordering -- race on it
 * and must be serialised by the caller.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int paged_kv_write_decode_noalloc(void* out, const void* q, void* k_cache, void* v_cache,
                                  const void* key, const void* value,
                                  const int32_t* slot_mapping, const int32_t* block_table,
                                  const int32_t* context_lens, int32_t block_size, float scale,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t dtype, void* stream);

/*
 * paged_attention_varlen -- packed variable-length (prefill) attention over
 * the paged cache.
 *
 * Sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q and
 * out, and keys/values 0 .. seq_lens[b]-1 read through block_table[b]
 * (the packed layout of the "Paged KV infra" page, section 3.1: cu_seqlens
 * has num_seqs+1 entries starting at 0, and each sequence gets its own
 * causal mask over its own length, without padding). With causal != 0,
 * local query i of a sequence with Lq queries and Lk keys sees keys
 * j <= i + Lk - Lq (aligned to the last key, so that Lq == Lk is the usual
 * lower-triangular mask and Lq == 1 is decode). A query row with no visible
 * key outputs zeros. The softmax scale is 1/sqrt(head_dim) (the skill
 * page's FA settings).
 *
 *   out              : [total_q, num_q_heads, head_dim], dtype (written)
 *   q                : [total_q, num_q_heads, head_dim], dtype
 *   cu_seqlens_q     : [num_seqs + 1] int32
 *   k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim], dtype
 *   block_table      : [num_seqs, max_blocks_per_seq] int32
 *   seq_lens         : [num_seqs] int32 (KV length per sequence)
 * Accepts dtype PKV_F16 and PKV_BF16 (matrix-core path); fp32 accumulation.
 */
int paged_attention_varlen(void* out, const void* q, const int32_t* cu_seqlens_q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens, int causal,
                           int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                           void* stream);

/*
 * Attention variants: sliding window and ALiBi
 * --------------------------------------------
 * The skill page's FA mask modes include "Band" (a sliding window, used for
 * prefill and decode of sliding-window models, given a count of preceding
 * tokens), and the FA call on the cann-recipes-infer page takes alibi_slopes
 * for ALiBi positional encoding. Readings: positions are aligned to the last
 * key as for the causal mask (local query i of a sequence with Lq queries and
 * Lk keys sits at p = i + Lk - Lq; a decode query at p = Lk - 1);
 *   window_left >= 0 : the query sees keys j >= p - window_left (itself and
 *                      window_left keys before it); negative: no window;
 *   alibi_slopes     : NULL, or [num_q_heads] float32 (device); query head h
 *                      adds alibi_slopes[h] * (j - p) to the scaled score.
 * A query with no visible key outputs zeros.
 */

/* paged_attention_decode with the variants above; q/out fp16 or bf16. Other
 * arguments and the workspace rule are those of paged_attention_decode. */
int paged_attention_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens,
                              int32_t block_size, float scale, const float* alibi_slopes,
                              int32_t window_left, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/* paged_attention_varlen with the variants above (window and ALiBi; the
 * window bounds keys below the query, and with causal == 0 keys after it
 * stay visible). Other arguments as paged_attention_varlen. */
int paged_attention_varlen_ex(void* out, const void* q, const int32_t* cu_seqlens_q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, int causal,
                              const float* alibi_slopes, int32_t window_left, int32_t num_seqs,
                              int64_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t dtype, void* stream);

/*
 * Split varlen: long key ranges over several workgroups
 * -----------------------------------------------------
 * paged_attention_varlen_split computes exactly what paged_attention_varlen
 * computes (same arguments and reading), for batches where a few query rows
 * sit over long contexts -- the decode rows of a mixed decode + prefill
 * batch, or the last few queries of a prefill over a long context. The last
 * query tile of a sequence, when its (query, head) rows fit one wave (at
 * most 32: e.g. up to 8 queries with 4 query heads per kv head) and its keys
 * run past one chunk, is cut into chunks attended by separate workgroups,
 * and their partial softmax results are merged exactly with the log-sum-exp
 * rule of the split decode (the vLLM-on-CANN page: scattered blocks merged
 * block by block with an online softmax). Chunks hold at least 512 keys; a
 * tile is cut into at most 16 of them. Full tiles are not cut (they already
 * spread over many workgroups).
 *
 * paged_attention_varlen_workspace_size -- bytes of device workspace the
 * split call needs for these sizes: per chunk, fp32 (max, sum) and the
 * unnormalised output of the (up to 32) rows of each sequence's last tile
 * per kv head. 0 when no tile can be cut (contexts of at most 512 keys: the
 * split call then is the plain one) and for invalid sizes.
 *
 *   workspace : device scratch of workspace_bytes bytes, workspace_bytes >=
 *               paged_attention_varlen_workspace_size(...) (may be NULL when
 *               that is 0). Its contents on entry do not matter; it is
 *               clobbered. Calls that share a workspace must be ordered on
 *               one stream.
 * Returns PKV_ERR_WORKSPACE when it is missing or too small; other statuses
 * as paged_attention_varlen.
 */
size_t paged_attention_varlen_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t max_blocks_per_seq,
                                             int32_t block_size);
int paged_attention_varlen_split(void* out, const void* q, const int32_t* cu_seqlens_q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, int causal,
                                 int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Int8 KV cache
 * -------------
 * The skill page lists int8 KV-cache quantisation among the ways to shrink
 * the cache (its further-techniques list: "INT8 / W8A8C8"; its FA parameter
 * table: antiquant_scale, dequant_scale_key / dequant_scale_value). The pages
 * fix neither the granularity nor the rounding; these calls take the plainest
 * reading: symmetric codes, one float32 scale per kv head for K and another
 * for V, value = code * scale.
 *
 *   k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim] int8
 *   k_scale, v_scale : [num_kv_heads] float32 (device), positive
 */

/*
 * paged_kv_write_int8 -- quantise new K/V rows and scatter them by slot.
 *
 * For every t < num_tokens with s = slot_mapping[t] in [0, num_blocks *
 * block_size), element x of kv head h of key[t] becomes
 *     code = clamp(rne(x / k_scale[h]), -127, 127)
 * in k_cache row s (rne: round half to even; the quotient is an IEEE
 * binary32 division of x widened to binary32); value[t] likewise with
 * v_scale. Slot rules as paged_kv_write (skill page, sections 3.1 and 3.3).
 * A NaN input gives an unspecified code.
 *
 *   key, value : [num_tokens, num_kv_heads, head_dim], dtype (F32, F16, BF16)
 *   slot_mapping : [num_tokens] int32
 */
int paged_kv_write_int8(void* k_cache, void* v_cache, const void* key, const void* value,
                        const float* k_scale, const float* v_scale, const int32_t* slot_mapping,
                        int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream);

/*
 * paged_attention_decode_int8 -- paged_attention_decode over an int8 cache:
 * key j of kv head h is k_scale[h] * k_cache code, value j likewise with
 * v_scale; the attention itself is the one paged_attention_decode defines
 * (skill page Appendix C, sparse_mode 0; split-KV partitions merged exactly).
 * q and out are fp16 or bf16 (dtype); the workspace rule is
 * paged_attention_decode_workspace_size(), as for paged_attention_decode.
 * Accumulation is fp32; codes enter the matrix cores exactly, the scales are
 * applied to the scores and to the output in fp32.
 */
int paged_attention_decode_int8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* block_table, const int32_t* context_lens,
                                int32_t block_size, float scale, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_write_decode_int8 -- one decode step over an int8 cache in a
 * single launch: paged_kv_write_int8(k_cache, v_cache, key, value, k_scale,
 * v_scale, slot_mapping, num_seqs tokens) followed by
 * paged_attention_decode_int8(...) on the same arguments, as
 * paged_kv_write_decode composes the 16-bit calls. key/value [num_seqs, num_kv_heads,
 * head_dim] are of dtype (fp16 or bf16, the q dtype); the codes stored and
 * attended are those paged_kv_write_int8 computes. Same precondition and
 * workspace rule as paged_kv_write_decode.
 */
int paged_kv_write_decode_int8(void* out, const void* q, void* k_cache, void* v_cache,
                               const void* key, const void* value, const float* k_scale,
                               const float* v_scale, const int32_t* slot_mapping,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t block_size, float scale, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_copy_blocks -- copy whole cache blocks: for every pair i,
 * block pairs[2i+1] of k_cache and of v_cache becomes a copy of block
 * pairs[2i] (all block_size rows, all kv heads, all dims; bit copy). This is
 * the device half of copy-on-write (the ATB PagedAttention page: a sequence
 * that extends a shared page first copies it to a fresh page); the pairs come
 * from pkv_bm_take_copies() (include/pkv_block_manager.h). The pairs of one
 * call are copied concurrently: no block may be both a source and a
 * destination, and no destination may repeat (the block manager guarantees
 * both). Pairs naming a block outside [0, num_blocks) are skipped.
 *
 *   k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim]
 *   pairs            : [num_pairs, 2] int32 (device): (source, destination)
 *   dtype            : element type of the pool (PKV_F32, PKV_F16, PKV_BF16, PKV_I8)
 */
int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int64_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, int32_t dtype, void* stream);

/* Static, human-readable text for a pkv_status value. Never NULL. */
const char* pkv_status_string(int status);

/*
 * Device-side contract reports (the debug build, libpagedkv_debug.so)
 * -------------------------------------------------------------------
 * Block ids, lengths, cu_seqlens_q and slots are read on the device, so the
 * host cannot validate them; the cann-recipes-infer page's fault table
 * (§5.1) traces crashes to a block_table or cu_seqlens of the wrong dtype or
 * shape. The kernels keep such values inside the buffers (see the contract
 * at the top) and say nothing. A build compiled with PKV_DEBUG_CHECKS=1 also
 * records, as bits of a per-device word, which kinds of violation its
 * kernels met; the default build compiles the reports out:
 */
#define PKV_DBG_BLOCK_ID 1u   /* a used block's id outside [0, num_blocks); a block is used
                                 when it holds keys below the length and, under a window,
                                 not only keys before the window */
#define PKV_DBG_LENGTH 2u     /* a context / KV length < 0 or > max_blocks_per_seq * block_size */
#define PKV_DBG_CU_SEQLENS 4u /* cu_seqlens_q not non-decreasing from 0 to total_q */
#define PKV_DBG_SLOT 8u       /* a slot >= num_blocks * block_size (negative slots are skips) */
#define PKV_DBG_COPY_PAIR 16u /* a paged_kv_copy_blocks pair naming a block outside the pool */

/* 1 when this library was built with PKV_DEBUG_CHECKS=1, else 0. */
int pkv_debug_checks(void);

/*
 * pkv_debug_take_errors -- waits for the current device (hipDeviceSynchronize),
 * stores in *bits the OR of the PKV_DBG_* bits that this library's kernels
 * reported on that device since the last take, and clears them. Returns
 * PKV_OK; PKV_ERR_NULL for a NULL bits; PKV_ERR_UNSUPPORTED (and *bits = 0)
 * in a build without the checks, which touches no device; PKV_ERR_HIP when
 * the runtime fails.
 */
int pkv_debug_take_errors(uint32_t* bits);

/*
 * Tokens per context partition that paged_attention_decode uses for these
 * sizes (informative; 0 for invalid sizes). Contexts longer than one
 * partition are split, and the partial softmax results of the pieces are
 * merged by an exact log-sum-exp reduce.
 */
int32_t pkv_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t dtype);

/*
 * pkv_time_next_kernel -- measurement hook. The next kernel that the calling
 * thread launches through this library (the first kernel of its next call:
 * the attention kernel itself for a decode call whose contexts are split, not
 * the reduce) records start_event when its dispatch begins and stop_event
 * when it ends, on the stream it is launched on (hipExtLaunchKernel events),
 * so that hipEventElapsedTime(start, stop) is that kernel's execution time
 * without the gaps around it. The events are hipEvent_t handles created by
 * the caller with timing enabled; either may be NULL. The setting is
 * per-thread and is consumed by one launch; NULL, NULL cancels it. A call
 * that fails validation launches nothing and leaves it pending. Returns
 * PKV_OK.
 */
int pkv_time_next_kernel(void* start_event, void* stop_event);

/*
 * pkv_decode_partition_override -- measurement and tuning hook. The calling
 * thread's fp16 / bf16 decode calls (paged_attention_decode, _ex, _int8,
 * paged_kv_write_decode and its int8 and no-allocation forms) cut every
 * context into partitions of partition_tokens tokens (512, 1024, 2048 or
 * 4096: 4-wave workgroups at 512, 8-wave ones above) instead of the launch
 * plan's choice, until the thread calls it with 0. The split-KV workspace
 * that paged_attention_decode_workspace_size reports covers every such
 * value. The results are the same up to summation order. Returns PKV_OK,
 * or PKV_ERR_SHAPE (and changes nothing) for any other value.
 */
int pkv_decode_partition_override(int32_t partition_tokens);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
